// The low-bit linear layer that consumes the packed weights: decode-shaped
// Y = Xs W'^T with W' dequantised on the fly from the integer codes.
//
// AWQ reading notes ("AWQ: Activation-Aware Weight Quantization For On-Device
// LLM Compression AND Acceleration"), section "Tiny Chat": the inference
// kernel dequantises inside the computation and never writes the dequantised
// weights back to DRAM, and the low-bit weights are reordered offline so the
// kernel can unpack them cheaply.  Section "Measures": with the scales folded,
// the layer computes (W diag(s)) (diag(s)^-1 x), so the packed codes quantise
// W diag(s) and the activations arrive already divided by s.
//
// Repacked layout (built once per layer by awq_lowbit_repack):
//   codes_t uint32 [K/32][N][bits]: the `bits` words holding the 32 codes of
//     chunk j (columns 32j .. 32j+31) of row n sit at ((j N) + n) bits, so the
//     64 lanes of a wave, one output row each, read consecutive words;
//   meta_t  float2 [K/group][N]: (delta, z) of group g of row n.
// Dequantisation: W'[n, k] = fp32((c - z) * delta), the same single rounding
// as the quantiser's own dequantisation, so W' is exact; products and sums
// are fp32 (fused multiply-add), partial sums of the k-splits are added in a
// fixed order.
#include "common.h"

namespace awq {
namespace {

constexpr int kRows = 256;        // output rows per workgroup, one per lane
constexpr int kMB = 8;            // activation rows per pass
constexpr int kMaxChunks = 32;    // chunks of 32 columns per k-split
constexpr int kTargetGroups = 1024;

struct Split {
  int s, cps;                     // number of k-splits, chunks per split
};

Split choose_split(int64_t N, int64_t K) {
  const int64_t chunks = K / 32;
  const int64_t row_blocks = (N + kRows - 1) / kRows;
  int64_t s = (kTargetGroups + row_blocks - 1) / row_blocks;
  const int64_t s_max = chunks / 4 > 0 ? chunks / 4 : 1;   // at least 4 chunks per split
  if (s > s_max) s = s_max;
  const int64_t s_min = (chunks + kMaxChunks - 1) / kMaxChunks;
  if (s < s_min) s = s_min;
  if (s < 1) s = 1;
  int64_t cps = (chunks + s - 1) / s;
  s = (chunks + cps - 1) / cps;
  return Split{(int)s, (int)cps};
}

// ---- repack --------------------------------------------------------------
__global__ __launch_bounds__(256) void repack_codes_kernel(const uint32_t* __restrict__ codes,
                                                           int64_t N, int64_t chunks, int bits,
                                                           uint32_t* __restrict__ codes_t) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // j * N + n
  if (t >= chunks * N) return;
  const int64_t j = t / N, n = t % N;
  const uint32_t* src = codes + (n * chunks + j) * bits;
  uint32_t* dst = codes_t + t * bits;
  for (int w = 0; w < bits; ++w) dst[w] = src[w];
}

__global__ __launch_bounds__(256) void repack_meta_kernel(const float* __restrict__ scales,
                                                          const uint8_t* __restrict__ zeros,
                                                          int64_t N, int64_t groups,
                                                          float2* __restrict__ meta_t) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // g * N + n
  if (t >= groups * N) return;
  const int64_t g = t / N, n = t % N;
  meta_t[t] = make_float2(scales[n * groups + g], (float)zeros[n * groups + g]);
}

// ---- GEMV -----------------------------------------------------------------
template <typename S>
__device__ __forceinline__ float ld_x(const S* p) { return to_f32(*p); }

// Grid: (row blocks, k-splits, activation-row blocks).  Lane = output row.
template <typename S, int BITS>
__global__ __launch_bounds__(kRows) void lowbit_gemv_kernel(
    const S* __restrict__ X, int64_t M, int64_t K, const uint32_t* __restrict__ codes_t,
    const float2* __restrict__ meta_t, int64_t N, int group, int cps,
    float* __restrict__ partials /* [splits][M][N] */) {
  __shared__ __attribute__((aligned(16))) float xs[kMB][kMaxChunks * 32];
  const int tid = threadIdx.x;
  const int64_t n = (int64_t)blockIdx.x * kRows + tid;
  const int split = blockIdx.y;
  const int64_t m0 = (int64_t)blockIdx.z * kMB;
  const int mb = (int)((M - m0) < kMB ? (M - m0) : kMB);
  const int64_t chunks = K / 32;
  const int64_t j0 = (int64_t)split * cps;
  const int nc = (int)((chunks - j0) < cps ? (chunks - j0) : cps);
  const int64_t k0 = j0 * 32;

  // stage this split's activations (fp32) in LDS; rows past M read as zero
  for (int i = tid; i < kMB * nc * 32; i += kRows) {
    const int m = i / (nc * 32), k = i % (nc * 32);
    xs[m][k] = m < mb ? ld_x(X + (m0 + m) * K + k0 + k) : 0.0f;
  }
  __syncthreads();

  float acc[kMB];
#pragma unroll
  for (int m = 0; m < kMB; ++m) acc[m] = 0.0f;
  const bool row_ok = n < N;
  const int chunks_per_group = group / 32;
  float2 gm = make_float2(0.0f, 0.0f);
  for (int c = 0; c < nc; ++c) {
    const int64_t j = j0 + c;
    if (c == 0 || j % chunks_per_group == 0)
      gm = row_ok ? meta_t[(j / chunks_per_group) * N + n] : make_float2(0.0f, 0.0f);
    uint32_t w[BITS];
    const uint32_t* src = codes_t + (j * N + (row_ok ? n : 0)) * BITS;
#pragma unroll
    for (int i = 0; i < BITS; ++i) w[i] = row_ok ? src[i] : 0u;
#pragma unroll
    for (int q = 0; q < 8; ++q) {             // 4 codes per step: one 16-byte LDS read per m
      float wq[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = q * 4 + e;              // code index inside the chunk
        const int p = BITS * i;
        const int wi = p >> 5, sh = p & 31;
        uint32_t code = w[wi] >> sh;
        if (sh + BITS > 32) code |= w[wi + 1] << (32 - sh);
        code &= (1u << BITS) - 1u;
        wq[e] = ((float)code - gm.y) * gm.x;
      }
#pragma unroll
      for (int m = 0; m < kMB; ++m) {
        const float4 xv = *reinterpret_cast<const float4*>(&xs[m][c * 32 + q * 4]);
        acc[m] = fmaf(wq[0], xv.x, acc[m]);
        acc[m] = fmaf(wq[1], xv.y, acc[m]);
        acc[m] = fmaf(wq[2], xv.z, acc[m]);
        acc[m] = fmaf(wq[3], xv.w, acc[m]);
      }
    }
  }
  if (!row_ok) return;
#pragma unroll
  for (int m = 0; m < kMB; ++m)
    if (m < mb) partials[((int64_t)split * M + m0 + m) * N + n] = acc[m];
}

// Y[m, n] = sum over splits in index order.
__global__ __launch_bounds__(256) void lowbit_reduce_kernel(const float* __restrict__ partials,
                                                            int splits, int64_t MN,
                                                            float* __restrict__ Y) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= MN) return;
  float v = 0.0f;
  for (int s = 0; s < splits; ++s) v += partials[s * MN + t];
  Y[t] = v;
}

template <typename S, int BITS>
hipError_t gemv_launch(const void* X, int64_t M, int64_t K, const uint32_t* codes_t,
                       const float2* meta_t, int64_t N, int group, float* Y, float* partials,
                       hipStream_t st) {
  const Split sp = choose_split(N, K);
  dim3 grid((unsigned)((N + kRows - 1) / kRows), (unsigned)sp.s, (unsigned)((M + kMB - 1) / kMB));
  {
    ProfScope p("awq_lowbit_gemv", st);
    lowbit_gemv_kernel<S, BITS><<<grid, kRows, 0, st>>>(static_cast<const S*>(X), M, K, codes_t,
                                                        meta_t, N, group, sp.cps, partials);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t MN = M * N;
  {
    ProfScope p("awq_lowbit_reduce", st);
    lowbit_reduce_kernel<<<(unsigned)((MN + 255) / 256), 256, 0, st>>>(partials, sp.s, MN, Y);
  }
  return hipGetLastError();
}

template <typename S>
hipError_t gemv_bits(int bits, const void* X, int64_t M, int64_t K, const uint32_t* codes_t,
                     const float2* meta_t, int64_t N, int group, float* Y, float* partials,
                     hipStream_t st) {
  switch (bits) {
    case 2: return gemv_launch<S, 2>(X, M, K, codes_t, meta_t, N, group, Y, partials, st);
    case 3: return gemv_launch<S, 3>(X, M, K, codes_t, meta_t, N, group, Y, partials, st);
    case 4: return gemv_launch<S, 4>(X, M, K, codes_t, meta_t, N, group, Y, partials, st);
    case 5: return gemv_launch<S, 5>(X, M, K, codes_t, meta_t, N, group, Y, partials, st);
    case 6: return gemv_launch<S, 6>(X, M, K, codes_t, meta_t, N, group, Y, partials, st);
    case 7: return gemv_launch<S, 7>(X, M, K, codes_t, meta_t, N, group, Y, partials, st);
    default: return gemv_launch<S, 8>(X, M, K, codes_t, meta_t, N, group, Y, partials, st);
  }
}

}  // namespace

size_t lowbit_gemv_ws_bytes(int64_t M, int64_t N, int64_t K) {
  const Split sp = choose_split(N, K);
  return (size_t)sp.s * (size_t)M * (size_t)N * sizeof(float);
}

hipError_t launch_lowbit_repack(const uint32_t* codes, const float* scales, const uint8_t* zeros,
                                int64_t N, int64_t K, int bits, int group, uint32_t* codes_t,
                                void* meta_t, hipStream_t st) {
  const int64_t chunks = K / 32, groups = K / group;
  {
    ProfScope p("awq_lowbit_repack", st);
    repack_codes_kernel<<<(unsigned)((chunks * N + 255) / 256), 256, 0, st>>>(codes, N, chunks,
                                                                               bits, codes_t);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope p("awq_lowbit_repack", st);
    repack_meta_kernel<<<(unsigned)((groups * N + 255) / 256), 256, 0, st>>>(
        scales, zeros, N, groups, static_cast<float2*>(meta_t));
  }
  return hipGetLastError();
}

hipError_t launch_lowbit_gemv(const void* X, awq_dtype_t dt, int64_t M, int64_t K,
                              const uint32_t* codes_t, const void* meta_t, int64_t N, int bits,
                              int group, float* Y, void* ws, hipStream_t st) {
  const float2* meta = static_cast<const float2*>(meta_t);
  float* partials = static_cast<float*>(ws);
  switch (dt) {
    case AWQ_F32: return gemv_bits<float>(bits, X, M, K, codes_t, meta, N, group, Y, partials, st);
    case AWQ_F16: return gemv_bits<_Float16>(bits, X, M, K, codes_t, meta, N, group, Y, partials, st);
    default: return gemv_bits<__bf16>(bits, X, M, K, codes_t, meta, N, group, Y, partials, st);
  }
}

}  // namespace awq
