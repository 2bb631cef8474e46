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
#include <algorithm>
#include <mutex>
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
// OR-ing c into the mantissa of 1024 and adding -(1024 + z) is exact (packed
// fp16 arithmetic: two codes per instruction).
template <int BITS>
__device__ __forceinline__ uint32_t pair_f16(const uint32_t (&w)[BITS], int t, half2v negz) {
  const uint32_t v = (code_at<BITS>(w, 2 * t) | (code_at<BITS>(w, 2 * t + 1) << 16)) | 0x64006400u;
  const half2v h = __builtin_bit_cast(half2v, v) + negz;
  return __builtin_bit_cast(uint32_t, h);
}

// (c - z) as fp32 without integer conversions.  A code c at bit sh of a dword,
// with sh + BITS <= 23, is AND-ed out in place and OR-ed under the exponent of
// 2^(23 - sh), whose mantissa step is 2^-sh: the float reads 2^(23 - sh) + c
// exactly, and subtracting 2^(23 - sh) + z (an integer below 2^24) leaves
// c - z exactly.  One AND-OR (and_or below) and one fp32 subtraction per
// code, no bit-field extracts or integer conversions.  The chunk's bitstream
// is read through windows: dwords starting at a code boundary b that hold the
// codes whose bits lie in [b, b + 23), chosen greedily from bit 0.
template <int BITS>
struct MagicWindows {
  static constexpr int kSpan = 23;                          // mantissa bits of fp32
  static constexpr int kPerWin = (kSpan - BITS) / BITS + 1;  // codes per window
  static constexpr int start(int i) { return (i / kPerWin) * kPerWin * BITS; }
  static constexpr int shift(int i) { return BITS * i - start(i); }
  static constexpr int last_bit(int i) {                    // last bit of i's window
    const int w_end = (i / kPerWin + 1) * kPerWin;          // first code of the next window
    return (w_end < 32 ? w_end : 32) * BITS - 1;
  }
};

// The AND-OR of the unpacking as one v_and_or_b32, mask in an SGPR and
// exponent in a VGPR.  Written out because the compiler splits (w & mask) |
// expo into a v_and_b32 and a v_or_b32 with literal operands, which measured
// slower (the 70B decode call took 36.5 us that way, 30.3 us with the single
// instruction).
// The constants come from magic_ops(), built once per kernel.
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t smask, uint32_t vexpo) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(smask), "v"(vexpo));
  return r;
}

// Masks (SGPRs) and exponents (VGPRs) of the window offsets sh = BITS t.
template <int BITS, int N>
struct MagicOps {
  uint32_t mask[N];
  uint32_t expo[N];
};
template <int BITS, int N>
__device__ __forceinline__ MagicOps<BITS, N> magic_ops() {
  MagicOps<BITS, N> o;
#pragma unroll
  for (int t = 0; t < N; ++t) {
    asm("s_mov_b32 %0, %1" : "=s"(o.mask[t]) : "i"(((1u << BITS) - 1u) << (BITS * t)));
    asm("v_mov_b32 %0, %1" : "=v"(o.expo[t]) : "i"((uint32_t)(150 - BITS * t) << 23));
  }
  return o;
}

template <int BITS>
__device__ __forceinline__ uint32_t magic_window(const uint32_t (&w)[BITS], int i) {
  using MW = MagicWindows<BITS>;
  const int b = MW::start(i);                    // compile-time after unrolling
  const int wi = b >> 5, sh = b & 31;
  if (sh == 0) return w[wi];
  if ((MW::last_bit(i) >> 5) == wi) return w[wi] >> sh;
  return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh);
}

// Subtrahends 2^(23 - sh) + z for the window offsets sh = 0, BITS, 2 BITS, ...
template <int BITS>
struct MagicNeg {
  float v[MagicWindows<BITS>::kPerWin];
};

template <int BITS>
__device__ __forceinline__ MagicNeg<BITS> magic_neg(float z) {
  MagicNeg<BITS> n;
#pragma unroll
  for (int t = 0; t < MagicWindows<BITS>::kPerWin; ++t)
    n.v[t] = (float)(1 << (23 - BITS * t)) + z;
  return n;
}

template <int BITS>
using GemvOps = MagicOps<BITS, MagicWindows<BITS>::kPerWin>;

template <int BITS>
__device__ __forceinline__ float magic_cz(const uint32_t (&w)[BITS], int i,
                                          const MagicNeg<BITS>& neg, const GemvOps<BITS>& ops) {
  using MW = MagicWindows<BITS>;
  const int sh = MW::shift(i);
  // the float reads 2^(23 - sh) + c
  const float m = __uint_as_float(and_or(magic_window<BITS>(w, i), ops.mask[sh / BITS], ops.expo[sh / BITS]));
  return m - neg.v[sh / BITS];
}

// Pair t of (c - z) as two bf16 (exact: |c - z| <= 255 has 8 significant bits).
template <int BITS>
__device__ __forceinline__ uint32_t pair_bf16(const uint32_t (&w)[BITS], int t,
                                              const MagicNeg<BITS>& neg, const GemvOps<BITS>& ops) {
  const bf162v p = {(__bf16)magic_cz<BITS>(w, 2 * t, neg, ops),
                    (__bf16)magic_cz<BITS>(w, 2 * t + 1, neg, ops)};
  return __builtin_bit_cast(uint32_t, p);
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
  __shared__ __attribute__((aligned(16))) S xs[MB][kMaxChunks * 32];
  const int tid = threadIdx.x;
  const int64_t n = (int64_t)blockIdx.x * kRows + tid;
  const int split = blockIdx.y;
  const int64_t m0 = (int64_t)blockIdx.z * MB;
  const int mb = (int)((M - m0) < MB ? (M - m0) : MB);
  const bool row_ok = n < N;
  const int64_t nn = row_ok ? n : 0;        // rows past N load row 0 and store nothing
  // chunks per group: a power of two (the group size is one), so the group of
  // chunk j and its last chunk come from a shift and a mask
  const int lg_cpg = __builtin_ctz((unsigned)group >> 5), cmask = (1 << lg_cpg) - 1;
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
        // (delta, z) once per group: at its first chunk, or the split's
        if ((j & cmask) == 0 || j == c_begin) g[u] = meta_t[(j >> lg_cpg) * N + nn];
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
  float2 gc = {0.0f, 0.0f};                  // the current group's (delta, z)
  MagicNeg<BITS> neg;                         // and its subtrahends
  const GemvOps<BITS> ops = magic_ops<BITS, MagicWindows<BITS>::kPerWin>();
  auto sum_chunks = [&](int c0, const uint32_t (&w)[kUnroll][BITS], const float2 (&g)[kUnroll]) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = c0 + u;
      if (j >= c_end) break;
      if ((j & cmask) == 0 || j == c_begin) {
        gc = g[u];
        neg = magic_neg<BITS>(gc.y);
      }
      const int kl = (j - c_begin) * 32;      // column of the chunk inside the staged block
      if constexpr (kF32) {
        // fp32 activations: plain fp32 products of x and the exact (c - z)
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const float cz = magic_cz<BITS>(w[u], i, neg, ops);
#pragma unroll
          for (int m = 0; m < MB; ++m) accg[m] = fmaf(cz, (float)xs[m][kl + i], accg[m]);
        }
      } else {
        uint32_t pr[16];
        if constexpr (std::is_same<S, _Float16>::value) {
          const _Float16 nz = (_Float16)(-(1024.0f + gc.y));
          const half2v negz = {nz, nz};
#pragma unroll
          for (int t = 0; t < 16; ++t) pr[t] = pair_f16<BITS>(w[u], t, negz);
        } else {
#pragma unroll
          for (int t = 0; t < 16; ++t) pr[t] = pair_bf16<BITS>(w[u], t, neg, ops);
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
      if (((j + 1) & cmask) == 0 || j + 1 == c_end) {   // group (or this split) ends
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          acc[m] = fmaf(accg[m], gc.x, acc[m]);
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

// Y[m, n] = sum over splits in index order.  kBatch splits' loads are issued
// before any is added: all of them (32) when the grid is smaller than the chip
// and each thread's round trips are the cost, 8 when many threads share the
// memory system.
template <int kBatch>
__global__ __launch_bounds__(256) void lowbit_reduce_kernel(const float* __restrict__ partials,
                                                            int splits, int64_t MN,
                                                            float* __restrict__ Y) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= MN) return;
  float v = 0.0f;
  for (int s0 = 0; s0 < splits; s0 += kBatch) {
    float p[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) p[i] = s0 + i < splits ? partials[(s0 + i) * MN + t] : 0.0f;
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (s0 + i < splits) v += p[i];
  }
  Y[t] = v;
}

hipError_t launch_reduce(const float* partials, int splits, int64_t MN, float* Y, hipStream_t st) {
  const unsigned blocks = (unsigned)((MN + 255) / 256);
  if (MN <= 256 * 256)
    lowbit_reduce_kernel<32><<<blocks, 256, 0, st>>>(partials, splits, MN, Y);
  else
    lowbit_reduce_kernel<8><<<blocks, 256, 0, st>>>(partials, splits, MN, Y);
  return hipGetLastError();
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
  ProfScope p("awq_lowbit_reduce", st);
  return launch_reduce(partials, sp.s, MN, Y, st);
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

// ---- prefill-sized GEMM on the matrix cores ------------------------------------
// Y [M, N] = Xs W'^T for many activation rows: a 256 x 128 output tile per
// workgroup of 8 waves, one workgroup per CU.  Each wave owns a 64 x 64 block
// (2 x 2 v_mfma_f32_32x32x16 on fp16 / bf16).  K advances 32 per stage.  The
// weights are not dequantised to W' but to the exact integers c - z (the
// GEMV's pairs), so the MFMA sums exact products x (c - z) in fp32; at the end
// of each group the group's sums are scaled by its delta (one product per
// group and output) and added to the running totals, as in the GEMV, and the
// next group's first MFMAs start from zero.  The dequantised weights never
// leave LDS, and each 128-row weight tile serves 256 activation rows.
//
// The waves run ping-pong: group 0 (waves 0-3, tile rows 0-127) and group 1
// (waves 4-7, rows 128-255) hold one wave on each SIMD.  Each stage has two
// halves separated by a barrier: in one, group 0 issues its MFMAs, with its
// share of the unpacking two stages ahead between them, while group 1 reads
// its fragments, issues its transfers and applies the group-end scaling of its
// previous stage; in the other the roles swap.  Each SIMD's matrix pipe is
// thus fed by its two waves in turn, and one wave's memory work runs while the
// other's MFMAs execute.
//
// Everything a stage needs arrives by wave-wide global -> LDS transfers
// (buffer_load_dwordx4 ... lds, 1 KB each), issued in the wave's working
// half: two per wave of the activation tile (16 KB, each lane fetching the
// chunk that the swizzle puts at its LDS position) four stages ahead into a
// ring of five slots, and, six stages ahead into rings of eight, one more per
// wave from as many waves as needed: the stage's packed codes (128 rows x bits
// words, contiguous in the repacked layout) and the (delta, z) pairs of the
// stage's group.  Before every barrier each wave lets only its last two stages
// of transfers stay in flight.  The unpacked B tiles live in a ring of three.
// Rows of 64 bytes; 16-byte chunk c of row r sits at c ^ ((r >> 1) & 3) (no
// bank conflicts for the fragment reads).  The LDS traffic of a stage (about
// 100 KB: fragment reads, transfers, unpacking) is what bounds this kernel.
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kGM = 256;                         // activation rows per tile
constexpr int kGN = 128;                         // output rows per tile
constexpr int kGWaves = 8;
constexpr int kGThreads = 64 * kGWaves;
constexpr int kXRing = 5, kXAhead = 4;           // activation slots, stages ahead
constexpr int kCRing = 8, kCAhead = 6;           // code and (delta, z) slots, stages ahead
constexpr int kBRing = 3;                        // unpacked weight slots (two stages ahead)
constexpr int kXSlot = kGM * 64;                 // 16 KB
constexpr int kBSlot = kGN * 64;                 // 8 KB
constexpr int kPerStage = 3;                     // transfers per stage of a wave with a third one

__device__ __forceinline__ int g_off(int r, int c) { return r * 64 + 16 * (c ^ ((r >> 1) & 3)); }

// Buffer resource of a raw byte range: loads at offsets >= num_bytes return 0.
__device__ __forceinline__ i32x4 byte_range(const void* base, uint32_t num_bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)b, (int)(uint32_t)(b >> 32), (int)num_bytes, 0x00020000};
}

// 16 bytes per lane from rsrc + voff into LDS at lds_addr + 16 * lane.  Inline
// asm, so that the compiler does not wait for every transfer before each LDS
// read; the kernel waits with explicit counts.  m0 is declared clobbered (the
// compiler keeps nothing of its own in it across the transfer and pads its own
// next use), and the SALU write of m0 gets the one wait state an LDS-DMA load
// needs before it reads m0.  clang warns about any reserved register in a
// clobber list; the clobber is honoured all the same.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void to_lds16(i32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most n transfers of this lane are outstanding.
template <int n>
__device__ __forceinline__ void vm_wait() {
  static_assert(n >= 0 && n < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most the transfers of the last n stages this wave issued are
// in flight (three per stage for a wave with a third transfer, else two).
template <int n>
__device__ __forceinline__ void stage_wait(bool third) {
  if (third) vm_wait<n * kPerStage>();
  else vm_wait<n * (kPerStage - 1)>();
}

// Barrier that the instruction scheduler may not move anything across; before
// it, only the wave's last two stages of transfers stay in flight.
__device__ __forceinline__ void half_barrier(bool third) {
  stage_wait<2>(third);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}

template <int BITS>
struct GemmLds {
  static constexpr int kCodeOps = (BITS + 1) / 2;          // 1 KB transfers of a stage's codes
  static_assert(kCodeOps + 1 <= kGWaves, "one code or pairs transfer per wave");
  static constexpr int kCodeSlot = kCodeOps * 1024;
  static constexpr int kX = 0;
  static constexpr int kB = kX + kXRing * kXSlot;
  static constexpr int kC = kB + kBRing * kBSlot;
  static constexpr int kMeta = kC + kCRing * kCodeSlot;     // (delta, z) slots of 1 KB, by stage
  static constexpr int kBytes = kMeta + kCRing * 1024;
  static_assert(kBytes <= 160 * 1024, "LDS of one CU");
};

template <typename S>
__device__ __forceinline__ f32x16 mfma32(i32x4 a, i32x4 b, f32x16 c);
template <>
__device__ __forceinline__ f32x16 mfma32<_Float16>(i32x4 a, i32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8, a),
                                                __builtin_bit_cast(half8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32<__bf16>(i32x4 a, i32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Code T of 8 consecutive ones (bits [T BITS, T BITS + BITS) of hi:lo) as
// the fp32 value c - z without integer conversions: the code is masked in
// place inside a window dword that starts at a code boundary and holds it
// below bit 23 - BITS, OR-ed under the exponent of 2^(23 - sh), so the float
// reads 2^(23 - sh) + c exactly; sub[sh / BITS] = 2^(23 - sh) + z.
template <int BITS>
struct QuarterWindows {
  static constexpr int kPer = (23 - BITS) / BITS + 1;   // codes per window
};
template <int BITS>
using QuarterOps = MagicOps<BITS, QuarterWindows<BITS>::kPer>;

template <int BITS, int T>
__device__ __forceinline__ float quarter_cz(uint32_t lo, uint32_t hi, const float* sub,
                                            const QuarterOps<BITS>& ops) {
  constexpr int kPer = QuarterWindows<BITS>::kPer;
  constexpr int w0 = (T / kPer) * kPer * BITS;          // first bit of T's window
  constexpr int sh = T * BITS - w0;
  uint32_t win;
  if constexpr (w0 == 0) win = lo;
  else if constexpr (w0 >= 32) win = hi >> (w0 - 32);
  else win = __builtin_amdgcn_alignbit(hi, lo, w0);
  return __uint_as_float(and_or(win, ops.mask[sh / BITS], ops.expo[sh / BITS])) - sub[sh / BITS];
}

// Pair P of a quarter as two bf16 (c - z), exact: the upper halves of the
// exact fp32 values.
template <int BITS, int P>
__device__ __forceinline__ uint32_t quarter_pair_bf16(uint32_t lo, uint32_t hi, const float* sub,
                                                      const QuarterOps<BITS>& ops) {
  const float f0 = quarter_cz<BITS, 2 * P>(lo, hi, sub, ops);
  const float f1 = quarter_cz<BITS, 2 * P + 1>(lo, hi, sub, ops);
  return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
}

// Code t of 8 consecutive ones held in bits [t BITS, t BITS + BITS) of hi:lo.
template <int BITS, int T>
__device__ __forceinline__ uint32_t code_of(uint32_t lo, uint32_t hi) {
  constexpr int b = T * BITS;
  constexpr uint32_t mask = (1u << BITS) - 1u;
  if constexpr (b + BITS <= 32) return (lo >> b) & mask;
  else if constexpr (b >= 32) return (hi >> (b - 32)) & mask;
  else return __builtin_amdgcn_alignbit(hi, lo, b) & mask;
}

// Pair P (codes 2P, 2P + 1) of 8 codes as two S values (c - z), exact.
template <typename S, int BITS, int P>
__device__ __forceinline__ uint32_t pair_of(uint32_t lo, uint32_t hi, half2v negz, int z) {
  const uint32_t c0 = code_of<BITS, 2 * P>(lo, hi), c1 = code_of<BITS, 2 * P + 1>(lo, hi);
  if constexpr (std::is_same<S, _Float16>::value) {
    // 1024 + c is exact in fp16; adding -(1024 + z) is exact
    const uint32_t v = c0 | (c1 << 16) | 0x64006400u;
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, v) + negz);
  } else {
    // small integers are exact in fp32 and their upper halves are exact bf16
    const float f0 = (float)((int)c0 - z), f1 = (float)((int)c1 - z);
    return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  }
}

template <typename S, int BITS>
__global__ __launch_bounds__(kGThreads, 1) void lowbit_gemm_kernel(
    const S* __restrict__ X, int64_t M, int64_t K, const uint32_t* __restrict__ codes_t,
    const float2* __restrict__ meta_t, int64_t N, int lg_cpg, float* __restrict__ Y) {
  using L = GemmLds<BITS>;
  __shared__ __attribute__((aligned(1024))) char lds[L::kBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, w4 = wave & 3;
  const int wm = grp * 128 + (w4 >> 1) * 64, wn = (w4 & 1) * 64;
  const int64_t m0 = (int64_t)blockIdx.y * kGM, n0 = (int64_t)blockIdx.x * kGN;
  const int chunks = (int)(K / 32), cmask = (1 << lg_cpg) - 1;
  const int64_t rows = M - m0 < kGM ? M - m0 : kGM;
  const i32x4 rx = byte_range(X + m0 * K, (uint32_t)(rows * K * (int64_t)sizeof(S)));
  const uint32_t base = (uint32_t)(uintptr_t)lds;
  const uint32_t lane16 = (uint32_t)lane * 16;
  // Activation transfers: this lane's row and chunk in each of the wave's two
  // 16-row slabs, as running offsets of the next stage to be issued.
  uint32_t xoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 16 * (2 * wave + i) + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 1) & 3);
    xoff[i] = (uint32_t)(((int64_t)row * K + 8 * c) * (int64_t)sizeof(S));
  }
  // The wave's third transfer of stage s, fixed for the kernel: waves
  // 0 .. kCodeOps - 1 fetch a kilobyte of the stage's codes, the next wave the
  // (delta, z) pairs of the stage's group, the others have none.  For unit
  // u = s >> a_shift: source a_src + u a_step.  32-bit wrap-around of a source
  // offset can only touch stages past the end, which are never used.
  const bool third = wave <= L::kCodeOps;
  i32x4 a_rsrc;
  uint32_t a_dst, a_dstride, a_src, a_step;
  int a_shift;
  if (wave < L::kCodeOps) {
    a_rsrc = byte_range(codes_t, (uint32_t)((uint64_t)chunks * N * BITS * 4));
    a_dst = base + L::kC + wave * 1024;
    a_dstride = L::kCodeSlot;
    a_src = (uint32_t)((uint64_t)n0 * BITS * 4) + wave * 1024;
    a_step = (uint32_t)((uint64_t)N * BITS * 4);
    a_shift = 0;
  } else {
    a_rsrc = byte_range(meta_t, (uint32_t)((uint64_t)(K >> (lg_cpg + 5)) * N * 8));
    a_dst = base + L::kMeta;
    a_dstride = 1024;
    a_src = (uint32_t)((uint64_t)n0 * 8);
    a_step = (uint32_t)((uint64_t)N * 8);
    a_shift = lg_cpg;
  }
  int aux_s = 0, x_slot = 0;
  auto issue_aux = [&]() {
    if (third) {
      const uint32_t u = (uint32_t)(aux_s >> a_shift);
      to_lds16(a_rsrc, a_dst + (uint32_t)(aux_s & (kCRing - 1)) * a_dstride, a_src + u * a_step + lane16);
    }
    ++aux_s;
  };
  auto issue_x = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      to_lds16(rx, base + L::kX + x_slot * kXSlot + (2 * wave + i) * 1024, xoff[i]);
      xoff[i] += 32 * (uint32_t)sizeof(S);
    }
    x_slot = x_slot == kXRing - 1 ? 0 : x_slot + 1;
  };
  // Unpacking, split between the two groups: thread -> B row lr, codes
  // [8 lq, 8 lq + 8) of the chunk for each of its group's two quarters, which
  // sit in bits [8 lq BITS, 8 lq BITS + 8 BITS) of the row's words.
  const int lr = tid & (kGN - 1);
  const int lq = __builtin_amdgcn_readfirstlane((tid >> 7) & 1) + 2 * grp;
  const int qbit = 8 * lq * BITS, qw = qbit >> 5, qoff = qbit & 31;
  const int qw1 = qw + 1 < BITS ? qw + 1 : BITS - 1, qw2 = qw + 2 < BITS ? qw + 2 : BITS - 1;
  struct Codes {
    uint32_t w0, w1, w2;
    int z;
  };
  auto dq_load = [&](int s) {
    const uint32_t* cw =
        reinterpret_cast<const uint32_t*>(lds + L::kC + (s & (kCRing - 1)) * L::kCodeSlot) + lr * BITS;
    Codes c;
    c.w0 = cw[qw];
    c.w1 = cw[qw1];
    c.w2 = BITS == 7 ? cw[qw2] : 0u;
    c.z = (int)reinterpret_cast<const float2*>(lds + L::kMeta + (s & (kCRing - 1)) * 1024)[lr].y;
    return c;
  };
  auto dq_store = [&](int s, const Codes& c) {
    uint32_t lo, hi;
    if constexpr (BITS == 2 || BITS == 4) {
      lo = c.w0 >> qoff;
      hi = 0u;
    } else if constexpr (BITS == 7) {
      lo = __builtin_amdgcn_alignbit(c.w1, c.w0, qoff);
      hi = __builtin_amdgcn_alignbit(c.w2, c.w1, qoff);
    } else {
      lo = __builtin_amdgcn_alignbit(c.w1, c.w0, qoff);
      hi = c.w1 >> qoff;
    }
    const int z = c.z;
    const _Float16 nzh = (_Float16)(-(1024 + z));
    const half2v negz = {nzh, nzh};
    const i32x4 v = {(int)pair_of<S, BITS, 0>(lo, hi, negz, z), (int)pair_of<S, BITS, 1>(lo, hi, negz, z),
                     (int)pair_of<S, BITS, 2>(lo, hi, negz, z), (int)pair_of<S, BITS, 3>(lo, hi, negz, z)};
    *reinterpret_cast<i32x4*>(lds + L::kB + (s % kBRing) * kBSlot + g_off(lr, lq)) = v;
  };
  auto dequant = [&](int s) { dq_store(s, dq_load(s)); };
  f32x16 acc[2][2], tot[2][2];
  const f32x16 zero16 = {};
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = zero16;
      tot[i][j] = zero16;
    }
  // fragment rows and 16-byte chunk of this lane: row l % 32, chunk 2 ks + l / 32
  const int fr = lane & 31, fh = lane >> 5;
  int a_frag[2], b_frag[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    a_frag[ks] = g_off(wm + fr, 2 * ks + fh);      // + 2048 for the second 32-row block
    b_frag[ks] = g_off(wn + fr, 2 * ks + fh);
  }
  i32x4 fa[2][2], fb[2][2];
  auto read_frags = [&](int s, int xslot) {
    const char* A = lds + L::kX + xslot * kXSlot;
    const char* B = lds + L::kB + (s % kBRing) * kBSlot;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        fa[i][ks] = *reinterpret_cast<const i32x4*>(A + a_frag[ks] + 2048 * i);
        fb[i][ks] = *reinterpret_cast<const i32x4*>(B + b_frag[ks] + 2048 * i);
      }
  };
  auto mfmas = [&](int s) {
    if ((s & cmask) == 0) {
      // a group's first stage: its sums start from zero
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) acc[i][jj] = mfma32<S>(fa[i][0], fb[jj][0], zero16);
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) acc[i][jj] = mfma32<S>(fa[i][0], fb[jj][0], acc[i][jj]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) acc[i][jj] = mfma32<S>(fa[i][1], fb[jj][1], acc[i][jj]);
  };
  // The group's sums of stage s times its delta, per output column, when s
  // ends a group.
  auto scale = [&](int s) {
    if (((s + 1) & cmask) != 0) return;
    const float2* meta = reinterpret_cast<const float2*>(lds + L::kMeta + (s & (kCRing - 1)) * 1024);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const float d = meta[wn + 32 * jj + fr].x;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) tot[i][jj][e] = fmaf(d, acc[i][jj][e], tot[i][jj][e]);
    }
  };
  // A wave's multiplying half of stage s: its MFMAs, with its share of the
  // unpacking of stage s + 2 between them (the codes read first, the
  // conversion after the first MFMAs, the store last).  Its working half: the
  // fragment reads of stage f and the next stage's transfers first, then the
  // group-end scaling of stage sc (if any) while those are in flight.  Work on
  // stages past the end reads and writes only ring slots that are never used
  // again.
  auto multiply = [&](int s) {
    const Codes c = dq_load(s + 2);
    mfmas(s);
    dq_store(s + 2, c);
  };
  auto work = [&](int f, int fslot, int sc, bool do_scale) {
    read_frags(f, fslot);
    issue_aux();
    issue_x();
    __builtin_amdgcn_sched_barrier(0);
    if (do_scale) scale(sc);
  };
  // Prologue: codes and pairs of stages 0 .. 5 and activations of stages
  // 0 .. 3, in the order the loop continues (stage t + 2's third transfer
  // before stage t's activations).
  issue_aux();
  issue_aux();
#pragma unroll
  for (int t = 0; t < kXAhead; ++t) {
    issue_aux();
    issue_x();
  }
  stage_wait<kXAhead>(third);                // codes and pairs of stages 0 and 1
  __syncthreads();
  dequant(0);
  dequant(1);
  stage_wait<kXAhead - 1>(third);            // activations of stage 0
  __syncthreads();
  // Each group runs its own copy of the loop (same barriers in the same
  // order), so that its registers are allocated for its own schedule.
  auto run = [&](auto group) {
    constexpr int G = decltype(group)::value;
    int xr = 0;                              // activation slot of stage k + 1 (group 0) / k (group 1)
    if constexpr (G == 0) {
      read_frags(0, 0);
      xr = 1;
      for (int k = 0; k < chunks; ++k) {
        multiply(k);                         // first half: multiply
        half_barrier(third);
        work(k + 1, xr, k, true);            // second half: work
        xr = xr == kXRing - 1 ? 0 : xr + 1;
        half_barrier(third);
      }
    } else {
      for (int k = 0; k < chunks; ++k) {
        work(k, xr, k - 1, k > 0);           // first half: work
        xr = xr == kXRing - 1 ? 0 : xr + 1;
        half_barrier(third);
        multiply(k);                         // second half: multiply
        half_barrier(third);
      }
      scale(chunks - 1);
    }
  };
  if (grp == 0) run(std::integral_constant<int, 0>());
  else run(std::integral_constant<int, 1>());
  vm_wait<0>();                              // no transfer may outlive the workgroup
  // lane l holds column l % 32 and rows 8 (e / 4) + 4 (l / 32) + e % 4 of a block
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int64_t n = n0 + wn + 32 * jj + fr;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + wm + 32 * i + 8 * (e >> 2) + 4 * fh + (e & 3);
        if (m < M && n < N) Y[m * N + n] = tot[i][jj][e];
      }
    }
}


// ---- prefill-sized GEMM, 256 x 256 tiles with running sums in step units ----------
// The same Y [M, N] = Xs W'^T, now with one accumulator set per wave, which
// lets each wave own 128 x 64 outputs (8 x 4 v_mfma_f32_16x16x32 blocks) and a
// workgroup of 8 waves a 256 x 256 tile: half the operand traffic through LDS
// per multiply-add of the 256 x 128 kernel above, whose two sets (the group's
// sums and the totals) limit a wave to 64 x 64.
//
// Arithmetic.  The MFMA still sums exact products x (c - z) in fp32; the
// running sum of an output row n is kept in units of U, the step of the
// current group (or, while a group's step is zero, of the last non-zero step
// before it; 1 before any).  When group g begins, the sum is multiplied by
// U_{g-1} / U_g (correctly rounded quotient); a group whose step is zero is
// unpacked as zeros and leaves U as it is; at the end y = sum * U.  Each
// product x (c - z) thus reaches y through at most K fp32 additions, two
// roundings per later group start and the final product:
// |y - y_exact| <= (K + 2 K / G + 2) 2^-24 sum |x w'| (first order).  Steps
// must be finite; where the steps of one row differ by more than a factor of
// 2^100 the scaled sums may leave the fp32 range.
//
// Schedule (ping-pong as in the search GEMM): group 0 (waves 0-3, tile rows
// 0-127) and group 1 (rows 128-255) hold one wave on each SIMD.  Each stage of
// 32 k has two halves separated by a barrier.  In its multiplying half a group
// issues its 32 MFMAs of stage k with the unpacking of stage k + 2 between
// them; in its working half it reads the fragments of the stage it multiplies
// next and that stage's codes (stage + 2), and rescales its sums if that stage
// starts a group.  Transfers (buffer_load_dwordx4 ... lds, 1 KB each) go in
// issue units, one per wave and stage: two of the activation tile (16 KB a
// stage, each lane fetching the chunk that the swizzle puts at its LDS
// position) four stages ahead into a ring of four, and the stage's packed
// codes (256 rows x bits words, contiguous in the repacked layout) and
// (delta, z) pairs of its group (2 KB) five stages ahead into rings of four:
// item i of those bits + 2 kilobytes goes to waves i and i - 8.  A unit's
// activations overwrite the slot of the stage group 1 has just read, so group
// 0 issues in its working half and group 1 at the start of its multiplying
// half, both after the barrier that ends group 1's reads.  Before the barrier
// that precedes a working half each wave lets only its last issue unit stay
// in flight, before the other barrier its last two.  Thread t unpacks codes
// [16 (t / 256), +16) of weight row t % 256 into a ring of three B tiles;
// group 0's threads also write the row's unit and, at a group start, the
// factor U_{g-1} / U_g next to the tile.  Rows of 64 bytes; 16-byte chunk c
// of row r at c ^ ((r >> 1) & 3).
constexpr int kTM = 256, kTN = 256;             // activation rows, output rows per tile
constexpr int kTWaves = 8;
constexpr int kTThreads = 64 * kTWaves;
constexpr int kTXRing = 4, kTXAhead = 4;        // activation slots, stages ahead
constexpr int kTCRing = 4, kTCAhead = 5;        // code and (delta, z) slots, stages ahead
constexpr int kTBRing = 3;                      // unpacked weight and unit slots
constexpr int kTMI = 8, kTNI = 4;               // 16 x 16 blocks of a wave: 128 x 64

template <int BITS>
struct TileLds {
  static constexpr int kCodeSlot = BITS * 1024;            // 256 rows x BITS words
  static constexpr int kAux = BITS + 2;                    // kilobytes of codes and pairs a stage
  static constexpr int kX = 0;
  static constexpr int kB = kX + kTXRing * kTM * 64;
  static constexpr int kC = kB + kTBRing * kTN * 64;
  static constexpr int kMeta = kC + kTCRing * kCodeSlot;   // 256 (delta, z) pairs per slot
  static constexpr int kUnit = kMeta + kTCRing * 2048;     // per slot: factor [256], unit [256]
  static constexpr int kBytes = kUnit + kTBRing * 2048;
  static_assert(kBytes <= 160 * 1024, "LDS of one CU");
  static_assert(kAux <= 2 * kTWaves, "at most two aux transfers per wave");
};

template <typename S>
__device__ __forceinline__ f32x4 mfma16x32(i32x4 a, i32x4 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma16x32<_Float16>(i32x4 a, i32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                __builtin_bit_cast(half8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma16x32<__bf16>(i32x4 a, i32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Wait until at most the last U issue units of this wave (2 + n_aux
// transfers each) are in flight.
template <int U>
__device__ __forceinline__ void unit_wait(int n_aux) {
  if (n_aux == 0) vm_wait<2 * U>();
  else if (n_aux == 1) vm_wait<3 * U>();
  else vm_wait<4 * U>();
}

template <int U = 2>
__device__ __forceinline__ void tile_barrier(int n_aux) {
  unit_wait<U>(n_aux);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}

template <typename S, int BITS>
__global__ __launch_bounds__(kTThreads, 1) void lowbit_tile_kernel(
    const S* __restrict__ X, int64_t M, int64_t K, const uint32_t* __restrict__ codes_t,
    const float2* __restrict__ meta_t, int64_t N, int lg_cpg, float* __restrict__ Y) {
  using L = TileLds<BITS>;
  __shared__ __attribute__((aligned(1024))) char lds[L::kBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, w4 = wave & 3;
  const int64_t m0 = (int64_t)blockIdx.y * kTM, n0 = (int64_t)blockIdx.x * kTN;
  const int chunks = (int)(K / 32), cmask = (1 << lg_cpg) - 1;
  const int64_t rows = M - m0 < kTM ? M - m0 : kTM;
  const i32x4 rx = byte_range(X + m0 * K, (uint32_t)(rows * K * (int64_t)sizeof(S)));
  const uint32_t base = (uint32_t)(uintptr_t)lds;
  const uint32_t lane16 = (uint32_t)lane * 16;

  // activation transfers: this lane's row and chunk in the wave's two 16-row
  // slabs, as running offsets of the next stage to be issued
  uint32_t xoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 16 * (2 * wave + i) + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 1) & 3);
    xoff[i] = (uint32_t)(((int64_t)row * K + 8 * c) * (int64_t)sizeof(S));
  }
  // aux transfers: item wave and item wave + 8 of the stage's BITS code
  // kilobytes and two pair kilobytes.  Item i < BITS: source codes of chunk j
  // at (j N + n0) BITS words + i KB; else pairs of group j >> lg_cpg at
  // (g N + n0) pairs + (i - BITS) KB.  32-bit wrap-around of a source offset
  // can only touch stages past the end, which are never used.
  const int n_aux = __builtin_amdgcn_readfirstlane((wave < L::kAux) + (wave + 8 < L::kAux));
  const i32x4 rc = byte_range(codes_t, (uint32_t)((uint64_t)chunks * N * BITS * 4));
  const i32x4 rm = byte_range(meta_t, (uint32_t)((uint64_t)(K >> (lg_cpg + 5)) * N * 8));
  int aux_s = 0, x_s = 0;
  auto issue_item = [&](int item, int s) __attribute__((always_inline)) {
    const int slot = s & (kTCRing - 1);
    if (item < BITS) {
      const uint32_t src = (uint32_t)(((uint64_t)s * N + n0) * BITS * 4) + item * 1024 + lane16;
      to_lds16(rc, base + L::kC + slot * L::kCodeSlot + item * 1024, src);
    } else {
      const uint32_t g = (uint32_t)(s >> lg_cpg);
      const uint32_t src = (uint32_t)(((uint64_t)g * N + n0) * 8) + (item - BITS) * 1024 + lane16;
      to_lds16(rm, base + L::kMeta + slot * 2048 + (item - BITS) * 1024, src);
    }
  };
  auto issue_aux = [&]() __attribute__((always_inline)) {
    if (n_aux > 0) issue_item(wave, aux_s);
    if (n_aux > 1) issue_item(wave + 8, aux_s);
    ++aux_s;
  };
  auto issue_x = [&]() __attribute__((always_inline)) {
    const int slot = x_s & (kTXRing - 1);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      to_lds16(rx, base + L::kX + slot * (kTM * 64) + (2 * wave + i) * 1024, xoff[i]);
      xoff[i] += 32 * (uint32_t)sizeof(S);
    }
    ++x_s;
  };

  // Unpacking: thread -> weight row lr, quarters 2 grp and 2 grp + 1 (codes
  // [8 q, 8 q + 8) of the chunk, bits [8 q BITS, 8 q BITS + 8 BITS) of the
  // row's words).
  const int lr = tid & (kTN - 1);
  float unit = 1.0f;                           // group 0's threads: the row's unit
  struct Quarter {
    uint32_t w0, w1, w2;
  };
  struct Codes {
    Quarter q[2];
    float2 dz;
  };
  auto dq_load = [&](int s) __attribute__((always_inline)) {
    const int slot = s & (kTCRing - 1);
    const uint32_t* cw =
        reinterpret_cast<const uint32_t*>(lds + L::kC + slot * L::kCodeSlot) + lr * BITS;
    Codes c;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int qbit = 8 * (2 * grp + h) * BITS, qw = qbit >> 5;
      const int qw1 = qw + 1 < BITS ? qw + 1 : BITS - 1, qw2 = qw + 2 < BITS ? qw + 2 : BITS - 1;
      c.q[h].w0 = cw[qw];
      c.q[h].w1 = cw[qw1];
      c.q[h].w2 = BITS == 7 ? cw[qw2] : 0u;
    }
    c.dz = reinterpret_cast<const float2*>(lds + L::kMeta + slot * 2048)[lr];
    return c;
  };
  const QuarterOps<BITS> qops = magic_ops<BITS, QuarterWindows<BITS>::kPer>();
  auto dq_store = [&](int s, const Codes& c) __attribute__((always_inline)) {
    // a zero step unpacks as zeros: codes and zero-point read as 0, so every
    // c - z is 0
    const bool live = c.dz.x != 0.0f;
    const int z = live ? (int)c.dz.y : 0;
    char* brow = lds + L::kB + (s % kTBRing) * (kTN * 64);
    float sub[QuarterWindows<BITS>::kPer];
#pragma unroll
    for (int t = 0; t < QuarterWindows<BITS>::kPer; ++t) sub[t] = (float)(1 << (23 - BITS * t)) + (float)z;
    const _Float16 nzh = (_Float16)(-(1024 + z));
    const half2v negz = {nzh, nzh};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int qbit = 8 * (2 * grp + h) * BITS, qoff = qbit & 31;
      uint32_t lo, hi;
      if constexpr (BITS == 2 || BITS == 4) {
        lo = c.q[h].w0 >> qoff;
        hi = 0u;
      } else if constexpr (BITS == 7) {
        lo = __builtin_amdgcn_alignbit(c.q[h].w1, c.q[h].w0, qoff);
        hi = __builtin_amdgcn_alignbit(c.q[h].w2, c.q[h].w1, qoff);
      } else {
        lo = __builtin_amdgcn_alignbit(c.q[h].w1, c.q[h].w0, qoff);
        hi = c.q[h].w1 >> qoff;
      }
      lo = live ? lo : 0u;
      hi = live ? hi : 0u;
      i32x4 v;
      if constexpr (std::is_same<S, _Float16>::value) {
        v = i32x4{(int)pair_of<S, BITS, 0>(lo, hi, negz, z), (int)pair_of<S, BITS, 1>(lo, hi, negz, z),
                  (int)pair_of<S, BITS, 2>(lo, hi, negz, z), (int)pair_of<S, BITS, 3>(lo, hi, negz, z)};
      } else {
        v = i32x4{(int)quarter_pair_bf16<BITS, 0>(lo, hi, sub, qops),
                  (int)quarter_pair_bf16<BITS, 1>(lo, hi, sub, qops),
                  (int)quarter_pair_bf16<BITS, 2>(lo, hi, sub, qops),
                  (int)quarter_pair_bf16<BITS, 3>(lo, hi, sub, qops)};
      }
      *reinterpret_cast<i32x4*>(brow + g_off(lr, 2 * grp + h)) = v;
    }
    if (grp == 0) {
      // the row's unit after stage s, and at a group start the factor that
      // takes the running sums from the previous unit to this one
      float* u = reinterpret_cast<float*>(lds + L::kUnit + (s % kTBRing) * 2048);
      if ((s & cmask) == 0) {
        const float nu = live ? c.dz.x : unit;
        u[lr] = unit / nu;
        unit = nu;
      }
      u[256 + lr] = unit;
    }
  };

  f32x4 acc[kTMI][kTNI];
#pragma unroll
  for (int i = 0; i < kTMI; ++i)
#pragma unroll
    for (int j = 0; j < kTNI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // fragments: A rows 128 grp + 16 i + l % 16, B rows 64 w4 + 16 j + l % 16,
  // chunk l / 16 of the stage (8 consecutive k)
  const int frow = lane & 15, fch = lane >> 4;
  const uint32_t a_frag = (uint32_t)g_off(grp * 128 + frow, fch);
  const uint32_t b_frag = (uint32_t)g_off(w4 * 64 + frow, fch);
  i32x4 fa[kTMI], fb[kTNI];
  auto read_frags = [&](int s) __attribute__((always_inline)) {
    const char* A = lds + L::kX + (s & (kTXRing - 1)) * (kTM * 64);
    const char* B = lds + L::kB + (s % kTBRing) * (kTN * 64);
#pragma unroll
    for (int i = 0; i < kTMI; ++i) fa[i] = *reinterpret_cast<const i32x4*>(A + a_frag + i * 1024);
#pragma unroll
    for (int j = 0; j < kTNI; ++j) fb[j] = *reinterpret_cast<const i32x4*>(B + b_frag + j * 1024);
  };
  auto mfmas = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kTMI; ++i)
#pragma unroll
      for (int j = 0; j < kTNI; ++j) acc[i][j] = mfma16x32<S>(fa[i], fb[j], acc[i][j]);
  };
  // at the start of group g > 0: the running sums of output column n times
  // U_{g-1} / U_g (lane l holds column l % 16 of each 16-wide block)
  const int ecol = lane & 15;
  auto rescale = [&](int s) __attribute__((always_inline)) {
    if (s == 0 || s >= chunks || (s & cmask) != 0) return;
    const float* u = reinterpret_cast<const float*>(lds + L::kUnit + (s % kTBRing) * 2048);
#pragma unroll
    for (int j = 0; j < kTNI; ++j) {
      const float r = u[w4 * 64 + 16 * j + ecol];
#pragma unroll
      for (int i = 0; i < kTMI; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][e] *= r;
    }
  };
  // A wave's working half for stage f: fragment reads of f and its codes of
  // stage f + 2, then (group 0) one issue unit, then the rescale before f's
  // MFMAs.  Its multiplying half of stage s: (group 1) one issue unit, then
  // its MFMAs, with the unpacking of the codes it read (stage s + 2) between
  // them.  An issue unit's activations go to the slot of the stage that group
  // 1 reads in its working half of the same iteration; group 1 issues after
  // the barrier that ends it, group 0 issues in the half after it.  Work on
  // stages past the end reads and writes only ring slots that are never used
  // again.
  Codes held;
  auto issue = [&]() __attribute__((always_inline)) {
    issue_aux();
    issue_x();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto multiply = [&](int s) __attribute__((always_inline)) {
    if (grp == 1) issue();
    mfmas();
    dq_store(s + 2, held);
  };
  auto work = [&](int f) __attribute__((always_inline)) {
    read_frags(f);
    held = dq_load(f + 2);
    if (grp == 0) issue();
    rescale(f);
  };
  // Prologue: issue units {aux 0}, then {aux t + 1, activations t} for
  // t = 0 .. 2, in the loop's order; unpack stages 0 and 1 once units -1 and 0
  // have landed; then unit 3, whose codes go to stage 0's slot.
  issue_aux();
#pragma unroll
  for (int t = 0; t < kTXAhead - 1; ++t) {
    issue_aux();
    issue_x();
  }
  tile_barrier(n_aux);                       // units 1 and 2 may be in flight
  dq_store(0, dq_load(0));
  dq_store(1, dq_load(1));
  __syncthreads();                           // every thread is done with slots 0 and 1
  issue_aux();
  issue_x();
  tile_barrier(n_aux);                       // unit 1 (stage 2's codes) has landed
  // Each group runs its own copy of the loop (same barriers in the same
  // order), so that its registers are allocated for its own schedule.
  auto run = [&](auto group) __attribute__((always_inline)) {
    constexpr int G = decltype(group)::value;
    // Before the barrier that precedes a working half (stage f: activations
    // of issue unit f, codes of unit f + 1) at most one issue unit per wave
    // may be in flight, before the other barrier two.
    if constexpr (G == 0) {
      read_frags(0);
      held = dq_load(2);
      for (int k = 0; k < chunks; ++k) {
        multiply(k);                         // first half: multiply
        tile_barrier<1>(n_aux);
        work(k + 1);                         // second half: work
        tile_barrier<2>(n_aux);
      }
    } else {
      for (int k = 0; k < chunks; ++k) {
        work(k);                             // first half: work
        tile_barrier<1>(n_aux);
        multiply(k);                         // second half: multiply
        tile_barrier<2>(n_aux);
      }
    }
  };
  if (grp == 0) run(std::integral_constant<int, 0>());
  else run(std::integral_constant<int, 1>());
  vm_wait<0>();                              // no transfer may outlive the workgroup
  // y = sum * U of the last stage; lane l holds column l % 16 and rows
  // 4 (l / 16) .. + 3 of each block
  const float* ul = reinterpret_cast<const float*>(lds + L::kUnit + ((chunks - 1) % kTBRing) * 2048) + 256;
  const int erow = (lane >> 4) * 4;
#pragma unroll
  for (int j = 0; j < kTNI; ++j) {
    const int nl = w4 * 64 + 16 * j + ecol;
    const int64_t n = n0 + nl;
    const float u = ul[nl];
#pragma unroll
    for (int i = 0; i < kTMI; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t m = m0 + grp * 128 + 16 * i + erow + e;
        if (m < M && n < N) Y[m * N + n] = acc[i][j][e] * u;
      }
  }
}

// ---- small-M layer on the matrix cores --------------------------------------------
// Up to 64 activation rows.  The GEMV's cost is vector work that grows with
// the rows (one v_dot2 per pair of codes per row); here every code is unpacked
// once, in registers, by the lane whose MFMA fragment holds it, and the matrix
// cores do the multiply-adds for all rows.  Workgroup: 4 waves, each owning 32
// output rows (the weight side of v_mfma_f32_32x32x16), MB blocks of 32
// activation rows (rows past M are zero).  The k order inside a 16-deep MFMA
// step is free as long as both operands agree: lane half h takes codes
// [16 h, 16 h + 16) of each 32-column chunk (k step t takes 8 of them), so its
// codes are one run of 16 fields: ceil(bits / 2) words of the repacked layout
// and one funnel shift.  The activations go through LDS 256 columns at a time
// (double-buffered, staged through registers a fill ahead; 16-byte chunk c of
// row m at c ^ (m % 32)).  The codes and (delta, z) pairs of stage s + 2 are
// loaded while stage s is multiplied.  Same arithmetic as the GEMV: exact
// products x (c - z) summed in fp32 per group, one product by delta per group
// and output (or per split end), k-splits summed in order by a second kernel.
constexpr int kSmRows = 128;                 // output rows per workgroup
constexpr int kSmTarget = 1024;              // workgroups aimed at
constexpr int kSmMinM = 5;                   // below this the vector kernel is faster
constexpr int64_t kGemmMaxK = 1ll << 22;     // the large-tile kernel's limits (32-bit tile offsets,
constexpr int64_t kGemmMaxM = 65535ll * 128; // activation-row tiles on grid y)
constexpr int kSmMaxM = 1024;

// Code T of 16 consecutive ones held in bits [T BITS, T BITS + BITS) of sw.
template <int BITS, int NW, int T>
__device__ __forceinline__ uint32_t code_in(const uint32_t (&sw)[NW]) {
  constexpr int b = T * BITS, w = b >> 5, o = b & 31;
  constexpr uint32_t mask = (1u << BITS) - 1u;
  if constexpr (o + BITS <= 32) return (sw[w] >> o) & mask;
  else return __builtin_amdgcn_alignbit(sw[w + 1], sw[w], o) & mask;
}

// Code T of the run as fp32 (c - z) in the magic-exponent form of the
// quarter unpacking: windows of QuarterWindows<BITS>::kPer codes start at code
// boundaries, sub[sh / BITS] = 2^(23 - sh) + z.
template <int BITS, int NW, int T>
__device__ __forceinline__ float small_cz(const uint32_t (&sw)[NW], const float* sub,
                                          const QuarterOps<BITS>& ops) {
  constexpr int kPer = QuarterWindows<BITS>::kPer;
  constexpr int w0 = (T / kPer) * kPer * BITS, wi = w0 >> 5, o = w0 & 31;
  constexpr int sh = T * BITS - w0;
  uint32_t win;
  if constexpr (o == 0) win = sw[wi];
  else if constexpr (wi + 1 >= NW || o + sh + BITS <= 32) win = sw[wi] >> o;
  else win = __builtin_amdgcn_alignbit(sw[wi + 1], sw[wi], o);
  return __uint_as_float(and_or(win, ops.mask[sh / BITS], ops.expo[sh / BITS])) - sub[sh / BITS];
}

// Codes 2P and 2P + 1 of the run as two S values (c - z), exact.
template <typename S, int BITS, int NW, int P>
__device__ __forceinline__ int small_pair(const uint32_t (&sw)[NW], half2v negz, const float* sub,
                                          const QuarterOps<BITS>& ops) {
  if constexpr (std::is_same<S, _Float16>::value) {
    const uint32_t c0 = code_in<BITS, NW, 2 * P>(sw), c1 = code_in<BITS, NW, 2 * P + 1>(sw);
    const uint32_t v = c0 | (c1 << 16) | 0x64006400u;
    return (int)__builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, v) + negz);
  } else {
    // small integers are exact in fp32 and their upper halves are exact bf16
    const float f0 = small_cz<BITS, NW, 2 * P>(sw, sub, ops);
    const float f1 = small_cz<BITS, NW, 2 * P + 1>(sw, sub, ops);
    return (int)__builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  }
}

// MB blocks of 32 activation rows per workgroup (grid z walks the row tiles),
// FS 32-column stages per activation fill.
template <typename S, int BITS, int MB, int FS>
__global__ __launch_bounds__(256, 2) void lowbit_small_kernel(
    const S* __restrict__ X, int64_t M, int64_t K, const uint32_t* __restrict__ codes_t,
    const float2* __restrict__ meta_t, int64_t N, int lg_cpg, int cps,
    float* __restrict__ partials, float* __restrict__ Y) {
  constexpr int NW = (BITS + 1) / 2;          // words holding a lane's 16 codes
  constexpr int kXRows = 32 * MB;
  constexpr int kCPR = 4 * FS;                // 16-byte chunks per activation row and fill
  constexpr int kRowB = 16 * kCPR;
  constexpr int kPer = kXRows * kCPR / 256;   // chunks per thread and fill
  __shared__ __attribute__((aligned(16))) char xs[2][kXRows * kRowB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int fr = lane & 31, h = lane >> 5;
  const int64_t n = (int64_t)blockIdx.x * kSmRows + wave * 32 + fr;
  const int64_t nc = n < N ? n : N - 1;       // rows past N load row N - 1 (never stored)
  const int chunks = (int)(K / 32), cmask = (1 << lg_cpg) - 1;
  const int split = blockIdx.y;
  const int s0 = split * cps, s1 = min(chunks, s0 + cps);
  const int nfill = (s1 - s0 + FS - 1) / FS;
  const int64_t m_base = (int64_t)blockIdx.z * kXRows;
  const int qbit = 16 * h * BITS, qw = qbit >> 5, qoff = qbit & 31;

  i32x4 xr[kPer];
  auto load_x = [&](int f) {
    const int64_t col0 = (int64_t)(s0 + FS * f) * 32;
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int idx = tid + 256 * p, row = idx / kCPR, c = idx % kCPR;
      const int64_t col = col0 + 8 * c, m = m_base + row;
      xr[p] = (m < M && col < K) ? *reinterpret_cast<const i32x4*>(X + m * K + col)
                                 : i32x4{0, 0, 0, 0};
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int idx = tid + 256 * p, row = idx / kCPR, c = idx % kCPR;
      *reinterpret_cast<i32x4*>(xs[buf] + row * kRowB + 16 * (c ^ (row & (kCPR - 1)))) = xr[p];
    }
  };
  uint32_t cw[4][NW];
  float2 mt[4];
  auto load_codes = [&](int s, int set) {
    const int sc = s < s1 ? s : s1 - 1;
    const uint32_t* cp = codes_t + ((int64_t)sc * N + nc) * BITS + qw;
#pragma unroll
    for (int i = 0; i < NW; ++i) cw[set][i] = cp[i];
    mt[set] = meta_t[(int64_t)(sc >> lg_cpg) * N + nc];
  };
  f32x16 acc[MB], tot[MB];
  const f32x16 zero16 = {};
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    acc[i] = zero16;
    tot[i] = zero16;
  }
  const QuarterOps<BITS> qops = magic_ops<BITS, QuarterWindows<BITS>::kPer>();
  // one stage: unpack this lane's 16 codes, read the activation fragments,
  // multiply; scale the group's sums at a group or split end
  auto stage = [&](int s, int set, const char* xb, int u) {
    uint32_t sw[NW];
    if constexpr (BITS % 2 == 1) {
#pragma unroll
      for (int i = 0; i + 1 < NW; ++i) sw[i] = __builtin_amdgcn_alignbit(cw[set][i + 1], cw[set][i], qoff);
      sw[NW - 1] = cw[set][NW - 1] >> qoff;
    } else {
#pragma unroll
      for (int i = 0; i < NW; ++i) sw[i] = cw[set][i];
    }
    const int z = (int)mt[set].y;
    const _Float16 nzh = (_Float16)(-(1024 + z));
    const half2v negz = {nzh, nzh};
    float sub[QuarterWindows<BITS>::kPer];
#pragma unroll
    for (int t = 0; t < QuarterWindows<BITS>::kPer; ++t) sub[t] = (float)(1 << (23 - BITS * t)) + (float)z;
    const i32x4 fb0 = {small_pair<S, BITS, NW, 0>(sw, negz, sub, qops), small_pair<S, BITS, NW, 1>(sw, negz, sub, qops),
                       small_pair<S, BITS, NW, 2>(sw, negz, sub, qops), small_pair<S, BITS, NW, 3>(sw, negz, sub, qops)};
    const i32x4 fb1 = {small_pair<S, BITS, NW, 4>(sw, negz, sub, qops), small_pair<S, BITS, NW, 5>(sw, negz, sub, qops),
                       small_pair<S, BITS, NW, 6>(sw, negz, sub, qops), small_pair<S, BITS, NW, 7>(sw, negz, sub, qops)};
    i32x4 fa[MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int row = 32 * mb + fr, c = 4 * u + 2 * h + t;
        fa[mb][t] = *reinterpret_cast<const i32x4*>(xb + row * kRowB + 16 * (c ^ (fr & (kCPR - 1))));
      }
    if (s == s0 || (s & cmask) == 0) {
      // a group's (or the split's) first stage: its sums start from zero
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma32<S>(fa[mb][0], fb0, zero16);
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma32<S>(fa[mb][0], fb0, acc[mb]);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma32<S>(fa[mb][1], fb1, acc[mb]);
    if (s == s1 - 1 || ((s + 1) & cmask) == 0) {
      const float d = mt[set].x;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) tot[mb][e] = fmaf(d, acc[mb][e], tot[mb][e]);
    }
  };
  load_x(0);
  load_codes(s0, 0);
  load_codes(s0 + 1, 1);
  store_x(0);
  __syncthreads();
  for (int f = 0; f < nfill; ++f) {
    const int buf = f & 1;
    if (f + 1 < nfill) load_x(f + 1);
#pragma unroll
    for (int u = 0; u < FS; ++u) {
      const int s = s0 + FS * f + u;
      load_codes(s + 2, (u + 2) & 3);
      if (s < s1) stage(s, u & 3, xs[buf], u);
    }
    if (f + 1 < nfill) store_x(buf ^ 1);
    __syncthreads();
  }
  if (n >= N) return;
  float* dst = gridDim.y == 1 ? Y : partials + (int64_t)split * M * N;
  // lane l holds column l % 32 and rows 8 (e / 4) + 4 (l / 32) + e % 4 of a block
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int64_t m = m_base + 32 * mb + 8 * (e >> 2) + 4 * h + (e & 3);
      if (m < M) dst[m * N + n] = tot[mb][e];
    }
}

// Activation-row blocks per workgroup and stages per fill, by M: one or two
// 32-row blocks with 256-column fills up to 64 rows; beyond, three blocks (a
// 96-row tile per workgroup, grid z over the tiles: four would not fit two
// waves per SIMD without spilling) with 128-column fills.
struct SmallShape {
  int mb, fs;
};
SmallShape small_shape(int64_t M) { return M <= 32 ? SmallShape{1, 8} : M <= 64 ? SmallShape{2, 8} : SmallShape{3, 4}; }

// k-splits of the small-M kernel: the largest power of two that keeps about
// kSmTarget workgroups, at least one activation fill per split, and the
// partial sums (S M N fp32, written and read back) under 64 MiB.  A power of
// two keeps the splits whole numbers of fills where K allows; a sweep of S on
// the layer shapes puts this within about 10% of the best split everywhere.
Split small_split(int64_t M, int64_t N, int64_t K) {
  const int64_t chunks = K / 32;
  const SmallShape sh = small_shape(M);
  const int64_t tiles = (N + kSmRows - 1) / kSmRows * ((M + 32 * sh.mb - 1) / (32 * sh.mb));
  int64_t lim = (kSmTarget + tiles - 1) / tiles;
  lim = std::min(lim, chunks / sh.fs);
  lim = std::min(lim, (int64_t)(64ll << 20) / (M * N * 8));
  int64_t s = 1;
  while (2 * s <= lim) s *= 2;
  const int64_t cps = (chunks + s - 1) / s;
  s = (chunks + cps - 1) / cps;
  return Split{(int)s, (int)cps};
}

// fp16 / bf16 activations from 5 rows: the unpacking is paid once per code and
// row tile here, once per code and row block of 8 in the vector kernel, which
// is the faster one for 1 to 4 rows (less work per code, no MFMA padding).
// Beyond 64 rows the large-tile kernel (unpacking amortised over 256 rows)
// wins once it has enough tiles to fill the chip (measured on the layer
// shapes: the 70B MLP layer at 256 rows, 224 tiles: 180 us there, 263 us here;
// the 4096-row layers at 256 rows, 32 tiles: 34 us here, 82 us there).
constexpr int64_t kGemmFullTiles = 200;
bool use_small(awq_dtype_t dt, int64_t M, int64_t N) {
  if (dt == AWQ_F32 || M < kSmMinM || M > kSmMaxM) return false;
  return M <= 64 || (N + 127) / 128 * ((M + 255) / 256) < kGemmFullTiles;
}

template <typename S, int BITS>
hipError_t small_launch(const void* X, int64_t M, int64_t K, const uint32_t* codes_t,
                        const float2* meta_t, int64_t N, int group, float* Y, float* partials,
                        hipStream_t st) {
  const Split sp = small_split(M, N, K);
  const SmallShape sh = small_shape(M);
  const int lg_cpg = __builtin_ctz((unsigned)(group / 32));
  const dim3 grid((unsigned)((N + kSmRows - 1) / kSmRows), (unsigned)sp.s,
                  (unsigned)((M + 32 * sh.mb - 1) / (32 * sh.mb)));
  const S* x = static_cast<const S*>(X);
  {
    ProfScope p("awq_lowbit_gemv", st);
    if (sh.mb == 1)
      lowbit_small_kernel<S, BITS, 1, 8><<<grid, 256, 0, st>>>(x, M, K, codes_t, meta_t, N, lg_cpg,
                                                                sp.cps, partials, Y);
    else if (sh.mb == 2)
      lowbit_small_kernel<S, BITS, 2, 8><<<grid, 256, 0, st>>>(x, M, K, codes_t, meta_t, N, lg_cpg,
                                                                sp.cps, partials, Y);
    else
      lowbit_small_kernel<S, BITS, 3, 4><<<grid, 256, 0, st>>>(x, M, K, codes_t, meta_t, N, lg_cpg,
                                                                sp.cps, partials, Y);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sp.s == 1) return e;
  const int64_t MN = M * N;
  ProfScope p("awq_lowbit_reduce", st);
  return launch_reduce(partials, sp.s, MN, Y, st);
}

template <typename S>
hipError_t small_bits(int bits, const void* X, int64_t M, int64_t K, const uint32_t* codes_t,
                      const float2* meta_t, int64_t N, int group, float* Y, float* partials,
                      hipStream_t st) {
  switch (bits) {
    case 2: return small_launch<S, 2>(X, M, K, codes_t, meta_t, N, group, Y, partials, st);
    case 3: return small_launch<S, 3>(X, M, K, codes_t, meta_t, N, group, Y, partials, st);
    case 4: return small_launch<S, 4>(X, M, K, codes_t, meta_t, N, group, Y, partials, st);
    case 5: return small_launch<S, 5>(X, M, K, codes_t, meta_t, N, group, Y, partials, st);
    case 6: return small_launch<S, 6>(X, M, K, codes_t, meta_t, N, group, Y, partials, st);
    case 7: return small_launch<S, 7>(X, M, K, codes_t, meta_t, N, group, Y, partials, st);
    default: return small_launch<S, 8>(X, M, K, codes_t, meta_t, N, group, Y, partials, st);
  }
}

// The large-tile kernels: 256 x 256 tiles (one accumulator set, rescaled at
// group starts) or 256 x 128 tiles (two sets).  One round of 256x256 tiles over
// the chip takes about 1.47 times as long as a round of 256x128 tiles (70B
// MLP layer, K = 8192: 253 against 172 us) for twice the outputs, so the wide
// tiles are used when they need fewer rounds by more than that factor: from a
// few hundred tiles on, not where a layer fills the chip only once either way.
bool use_wide_tiles(int64_t M, int64_t N) {
  const int64_t g = gemm_grid();
  const int64_t mt = (M + kTM - 1) / kTM;
  const int64_t r_wide = ((N + kTN - 1) / kTN * mt + g - 1) / g;
  const int64_t r_narrow = ((N + kGN - 1) / kGN * mt + g - 1) / g;
  return 100 * r_narrow > 147 * r_wide;
}

template <typename S, int BITS>
hipError_t gemm_launch(const void* X, int64_t M, int64_t K, const uint32_t* codes_t,
                       const float2* meta_t, int64_t N, int group, float* Y, hipStream_t st) {
  const int lg_cpg = __builtin_ctz((unsigned)(group / 32));   // group is a power of two >= 32
  if (use_wide_tiles(M, N)) {
    ProfScope p("awq_lowbit_gemm_wide", st);
    const dim3 grid((unsigned)((N + kTN - 1) / kTN), (unsigned)((M + kTM - 1) / kTM));
    lowbit_tile_kernel<S, BITS><<<grid, kTThreads, 0, st>>>(static_cast<const S*>(X), M, K,
                                                            codes_t, meta_t, N, lg_cpg, Y);
  } else {
    ProfScope p("awq_lowbit_gemm_narrow", st);
    const dim3 grid((unsigned)((N + kGN - 1) / kGN), (unsigned)((M + kGM - 1) / kGM));
    lowbit_gemm_kernel<S, BITS><<<grid, kGThreads, 0, st>>>(static_cast<const S*>(X), M, K,
                                                            codes_t, meta_t, N, lg_cpg, Y);
  }
  return hipGetLastError();
}

template <typename S>
hipError_t gemm_bits(int bits, const void* X, int64_t M, int64_t K, const uint32_t* codes_t,
                     const float2* meta_t, int64_t N, int group, float* Y, hipStream_t st) {
  switch (bits) {
    case 2: return gemm_launch<S, 2>(X, M, K, codes_t, meta_t, N, group, Y, st);
    case 3: return gemm_launch<S, 3>(X, M, K, codes_t, meta_t, N, group, Y, st);
    case 4: return gemm_launch<S, 4>(X, M, K, codes_t, meta_t, N, group, Y, st);
    case 5: return gemm_launch<S, 5>(X, M, K, codes_t, meta_t, N, group, Y, st);
    case 6: return gemm_launch<S, 6>(X, M, K, codes_t, meta_t, N, group, Y, st);
    case 7: return gemm_launch<S, 7>(X, M, K, codes_t, meta_t, N, group, Y, st);
    default: return gemm_launch<S, 8>(X, M, K, codes_t, meta_t, N, group, Y, st);
  }
}

}  // namespace

namespace {
// The kernel a call of these sizes runs; the workspace size and the launch
// both follow it.
enum class Route { kVector, kSmall, kTiles };
Route gemv_route(awq_dtype_t dt, int64_t M, int64_t N, int64_t K) {
  if (use_small(dt, M, N)) return Route::kSmall;
  if (dt != AWQ_F32 && M > 4 && K <= kGemmMaxK && M <= kGemmMaxM) return Route::kTiles;
  return Route::kVector;
}
}  // namespace

size_t lowbit_gemv_ws_bytes(awq_dtype_t dt, int64_t M, int64_t N, int64_t K) {
  Split sp{1, 0};
  switch (gemv_route(dt, M, N, K)) {
    case Route::kSmall: sp = small_split(M, N, K); break;
    case Route::kVector: sp = choose_split(N, K); break;
    case Route::kTiles: break;                      // no partial sums
  }
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
  const Route r = gemv_route(dt, M, N, K);
  if (r == Route::kSmall) {
    if (dt == AWQ_F16) return small_bits<_Float16>(bits, X, M, K, codes_t, meta, N, group, Y, partials, st);
    return small_bits<__bf16>(bits, X, M, K, codes_t, meta, N, group, Y, partials, st);
  }
  if (r == Route::kTiles) return launch_lowbit_gemm(X, dt, M, K, codes_t, meta_t, N, bits, group, Y, st);
  switch (dt) {
    case AWQ_F32: return gemv_bits<float>(bits, X, M, K, codes_t, meta, N, group, Y, partials, st);
    case AWQ_F16: return gemv_bits<_Float16>(bits, X, M, K, codes_t, meta, N, group, Y, partials, st);
    default: return gemv_bits<__bf16>(bits, X, M, K, codes_t, meta, N, group, Y, partials, st);
  }
}

// ---- allocation-free GEMV: the partial sums in a static array ----------------
// One array per GPU: the runtime places it when this code object is loaded on
// the device and it stays until the process ends.  In host code `scratch`
// names a host-side stand-in, not the device address, so every use goes
// through the address hipGetSymbolAddress returns, looked up once per device
// with that device current.
static __device__ __align__(256) unsigned char scratch[AWQ_LOWBIT_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t lowbit_static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_lowbit_gemm(const void* X, awq_dtype_t dt, int64_t M, int64_t K,
                              const uint32_t* codes_t, const void* meta_t, int64_t N, int bits,
                              int group, float* Y, hipStream_t st) {
  const float2* meta = static_cast<const float2*>(meta_t);
  if (dt == AWQ_F16) return gemm_bits<_Float16>(bits, X, M, K, codes_t, meta, N, group, Y, st);
  return gemm_bits<__bf16>(bits, X, M, K, codes_t, meta, N, group, Y, st);
}

}  // namespace awq
