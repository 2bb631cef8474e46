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
// Arithmetic: y[n] = sum_g delta_g * (sum_{k in g} x_k * (c_k - z_g)); the
// integers c - z and their products with x are exact, the sums are fp32.
//
// A workgroup owns 256 output rows (lane = row) and one run of up to 32
// chunks of 32 columns (a k-split), with the codes of the next 2 chunks in
// flight while 2 are summed.  The split's activations are staged in LDS and
// read as broadcasts (every lane needs the same ones).  With several splits
// the partial sums go to the workspace and a second kernel adds them in
// split order, so the result does not depend on scheduling.  (Letting the
// last workgroup of a row block add them instead needs a device-scope fence
// per workgroup to make the partials visible across XCDs, which measured
// slower than the second launch.)
#include <type_traits>

#include "common.h"

namespace awq {
namespace {

constexpr int kRows = 256;        // output rows per workgroup, one per lane
constexpr int kMB = 8;            // activation rows per pass
constexpr int kMaxChunks = 32;    // chunks of 32 columns per k-split
constexpr int kUnroll = 2;        // chunks whose codes are loaded together
constexpr int kTargetGroups = 2048;

struct Split {
  int s, cps;                     // number of k-splits, chunks per split
};

// Enough workgroups to keep every CU streaming, at least 4 chunks per split
// and at most kMaxChunks (the LDS staging of the activations).
Split choose_split(int64_t N, int64_t K) {
  const int64_t chunks = K / 32;
  const int64_t row_blocks = (N + kRows - 1) / kRows;
  int64_t s = (kTargetGroups + row_blocks - 1) / row_blocks;
  const int64_t s_max = chunks / 4 > 0 ? chunks / 4 : 1;
  if (s > s_max) s = s_max;
  const int64_t s_min = (chunks + kMaxChunks - 1) / kMaxChunks;
  if (s < s_min) s = s_min;
  if (s < 1) s = 1;
  const int64_t cps = (chunks + s - 1) / s;
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
// 16-bit activations (fp16 / bf16): the 32 codes of a chunk become 16 pairs
// (c - z) of the activation format -- exact, |c - z| <= 255 -- and each pair
// meets the matching pair of activations in one v_dot2 (two exact products,
// fp32 accumulation).  The group sum is scaled by delta once per group:
//   y = sum_g delta_g * sum_{k in g} x_k (c_k - z_g).
// Code pairs are (c_2t, c_2t+1), matching the activation pair in dword t.
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf162v __attribute__((ext_vector_type(2)));

template <int BITS>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&w)[BITS], int i) {
  const int p = BITS * i;                    // compile-time after unrolling
  const int wi = p >> 5, sh = p & 31;
  uint32_t c = w[wi] >> sh;
  if (sh + BITS > 32) c |= w[wi + 1] << (32 - sh);
  return c & ((1u << BITS) - 1u);
}

// Pair t of (c - z) as two fp16: 1024 + c is exact in fp16 for c < 1024, so
// OR-ing c into the mantissa of 1024 and adding -(1024 + z) is exact.
template <int BITS>
__device__ __forceinline__ uint32_t pair_f16(const uint32_t (&w)[BITS], int t, half2v negz) {
  const uint32_t v = (code_at<BITS>(w, 2 * t) | (code_at<BITS>(w, 2 * t + 1) << 16)) | 0x64006400u;
  const half2v h = __builtin_bit_cast(half2v, v) + negz;
  return __builtin_bit_cast(uint32_t, h);
}

// Pair t of (c - z) as two bf16: the integers are converted through fp32,
// where they are exact, and their upper halves (exact bf16) are packed.
template <int BITS>
__device__ __forceinline__ uint32_t pair_bf16(const uint32_t (&w)[BITS], int t, int z) {
  const float lo = (float)((int)code_at<BITS>(w, 2 * t) - z);
  const float hi = (float)((int)code_at<BITS>(w, 2 * t + 1) - z);
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

template <typename S>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c);
template <>
__device__ __forceinline__ float dot2<_Float16>(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, a), __builtin_bit_cast(half2v, b), c,
                                false);
}
template <>
__device__ __forceinline__ float dot2<__bf16>(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162v, a),
                                         __builtin_bit_cast(bf162v, b), c, false);
}

// Grid: (row blocks of 256, k-splits, activation-row blocks of MB).  Lane =
// output row; the workgroup sums chunks [split * cps, (split + 1) * cps).
template <typename S, int BITS, int MB>
__global__ __launch_bounds__(kRows) void lowbit_gemv_kernel(
    const S* __restrict__ X, int64_t M, int64_t K, const uint32_t* __restrict__ codes_t,
    const float2* __restrict__ meta_t, int64_t N, int group, int cps,
    float* __restrict__ partials /* [splits][M][N] */, float* __restrict__ Y) {
  constexpr bool kF32 = sizeof(S) == 4;
  constexpr bool kHalf = std::is_same<S, _Float16>::value;
  __shared__ __attribute__((aligned(16))) S xs[MB][kMaxChunks * 32];
  const int tid = threadIdx.x;
  const int64_t n = (int64_t)blockIdx.x * kRows + tid;
  const int split = blockIdx.y;
  const int64_t m0 = (int64_t)blockIdx.z * MB;
  const int mb = (int)((M - m0) < MB ? (M - m0) : MB);
  const bool row_ok = n < N;
  const int64_t nn = row_ok ? n : 0;        // rows past N load row 0 and store nothing
  const int cpg = group / 32;                // chunks per group
  const int chunks = (int)(K / 32);
  const int c_begin = split * cps;
  const int c_end = c_begin + cps < chunks ? c_begin + cps : chunks;
  const int nc = c_end - c_begin;

  // codes of kUnroll chunks in flight while the previous kUnroll are summed
  uint32_t wa[kUnroll][BITS], wb[kUnroll][BITS];
  float2 ga[kUnroll], gb[kUnroll];
  auto fetch = [&](int c0, uint32_t (&w)[kUnroll][BITS], float2 (&g)[kUnroll]) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (c0 + u < c_end) {
        const int64_t j = c0 + u;
        const uint32_t* src = codes_t + (j * N + nn) * BITS;
#pragma unroll
        for (int i = 0; i < BITS; ++i) w[u][i] = src[i];
        g[u] = meta_t[(j / cpg) * N + nn];
      }
    }
  };
  fetch(c_begin, wa, ga);

  // stage this split's activations in LDS (16-byte pieces; rows past M are zero)
  {
    constexpr int E = 16 / (int)sizeof(S);
    const int pieces = MB * nc * 32 / E;
    for (int i = tid; i < pieces; i += kRows) {
      const int m = i * E / (nc * 32), k = i * E % (nc * 32);
      i32x4 v = i32x4{0, 0, 0, 0};
      if (m < mb) v = *reinterpret_cast<const i32x4*>(X + (m0 + m) * K + (int64_t)c_begin * 32 + k);
      *reinterpret_cast<i32x4*>(&xs[m][k]) = v;
    }
  }
  __syncthreads();

  float acc[MB], accg[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) acc[m] = accg[m] = 0.0f;
  auto sum_chunks = [&](int c0, const uint32_t (&w)[kUnroll][BITS], const float2 (&g)[kUnroll]) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = c0 + u;
      if (j >= c_end) break;
      const int kl = (j - c_begin) * 32;      // column of the chunk inside the staged block
      if (kF32) {
        // fp32 activations: plain fp32 products of x and the exact (c - z)
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const float cz = (float)code_at<BITS>(w[u], i) - g[u].y;
#pragma unroll
          for (int m = 0; m < MB; ++m) accg[m] = fmaf(cz, (float)xs[m][kl + i], accg[m]);
        }
      } else {
        uint32_t pr[16];
        if (kHalf) {
          const _Float16 nz = (_Float16)(-(1024.0f + g[u].y));
          const half2v negz = {nz, nz};
#pragma unroll
          for (int t = 0; t < 16; ++t) pr[t] = pair_f16<BITS>(w[u], t, negz);
        } else {
          const int z = (int)g[u].y;
#pragma unroll
          for (int t = 0; t < 16; ++t) pr[t] = pair_bf16<BITS>(w[u], t, z);
        }
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          // the same 64 bytes for every lane: LDS broadcast reads
          const i32x4* x4 = reinterpret_cast<const i32x4*>(&xs[m][kl]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const i32x4 xv = x4[q];
            accg[m] = dot2<S>(pr[4 * q + 0], (uint32_t)xv.x, accg[m]);
            accg[m] = dot2<S>(pr[4 * q + 1], (uint32_t)xv.y, accg[m]);
            accg[m] = dot2<S>(pr[4 * q + 2], (uint32_t)xv.z, accg[m]);
            accg[m] = dot2<S>(pr[4 * q + 3], (uint32_t)xv.w, accg[m]);
          }
        }
      }
      if ((j + 1) % cpg == 0 || j + 1 == c_end) {   // group (or this split) ends
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          acc[m] = fmaf(accg[m], g[u].x, acc[m]);
          accg[m] = 0.0f;
        }
      }
    }
  };
  for (int c0 = c_begin; c0 < c_end; c0 += 2 * kUnroll) {
    if (c0 + kUnroll < c_end) fetch(c0 + kUnroll, wb, gb);
    sum_chunks(c0, wa, ga);
    if (c0 + kUnroll >= c_end) break;
    if (c0 + 2 * kUnroll < c_end) fetch(c0 + 2 * kUnroll, wa, ga);
    sum_chunks(c0 + kUnroll, wb, gb);
  }
  if (!row_ok) return;
  // one split: the sums are final
  float* dst = gridDim.y == 1 ? Y : partials + (int64_t)split * M * N;
#pragma unroll
  for (int m = 0; m < MB; ++m)
    if (m < mb) dst[(m0 + m) * N + n] = acc[m];
}

// Y[m, n] = sum over splits in index order.
__global__ __launch_bounds__(256) void lowbit_reduce_kernel(const float* __restrict__ partials,
                                                            int splits, int64_t MN,
                                                            float* __restrict__ Y) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= MN) return;
  float v = 0.0f;
#pragma unroll 8
  for (int s = 0; s < splits; ++s) v += partials[s * MN + t];
  Y[t] = v;
}

// Activation rows per pass: as many as M needs, up to kMB.
int rows_per_pass(int64_t M) { return M == 1 ? 1 : M == 2 ? 2 : M <= 4 ? 4 : kMB; }

template <typename S, int BITS, int MB>
void gemv_grid(const void* X, int64_t M, int64_t K, const uint32_t* codes_t, const float2* meta_t,
               int64_t N, int group, const Split& sp, float* partials, float* Y, hipStream_t st) {
  dim3 grid((unsigned)((N + kRows - 1) / kRows), (unsigned)sp.s, (unsigned)((M + MB - 1) / MB));
  lowbit_gemv_kernel<S, BITS, MB><<<grid, kRows, 0, st>>>(static_cast<const S*>(X), M, K, codes_t,
                                                          meta_t, N, group, sp.cps, partials, Y);
}

template <typename S, int BITS>
hipError_t gemv_launch(const void* X, int64_t M, int64_t K, const uint32_t* codes_t,
                       const float2* meta_t, int64_t N, int group, float* Y, float* partials,
                       hipStream_t st) {
  const Split sp = choose_split(N, K);
  {
    ProfScope p("awq_lowbit_gemv", st);
    switch (rows_per_pass(M)) {
      case 1: gemv_grid<S, BITS, 1>(X, M, K, codes_t, meta_t, N, group, sp, partials, Y, st); break;
      case 2: gemv_grid<S, BITS, 2>(X, M, K, codes_t, meta_t, N, group, sp, partials, Y, st); break;
      case 4: gemv_grid<S, BITS, 4>(X, M, K, codes_t, meta_t, N, group, sp, partials, Y, st); break;
      default: gemv_grid<S, BITS, kMB>(X, M, K, codes_t, meta_t, N, group, sp, partials, Y, st); break;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sp.s == 1) return e;
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
  return sp.s == 1 ? 0 : (size_t)sp.s * (size_t)M * (size_t)N * sizeof(float);
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
