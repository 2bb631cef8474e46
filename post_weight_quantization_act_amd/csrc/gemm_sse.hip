// Candidate-output GEMM with a fused squared-error epilogue, the reference
// output GEMM, and the loss reduction / argmin.
//
// AWQ Q&A page (aivaro.ru), section 6: each candidate is scored by the mean
// squared error between the outputs of the original layer and of the scaled,
// quantised one.  AWQ reading notes, section "Measures": the output
// perturbation of y = W x is (W_hat - W) x, and the exponent alpha with the
// smallest output error is kept.
//
// C[t, n] = sum_k X[t, k] * B[n, k]: X [T, K] and B [N, K] are both
// K-contiguous, which is the operand layout the MFMA wants (every lane feeds
// 8 consecutive k values of one row).  fp16/bf16 layers use
// v_mfma_f32_16x16x32_{f16,bf16} with fp32 accumulation; fp32 layers use a
// vector-ALU fp32 kernel.  The epilogue never writes C: it either stores the
// reference output once, or reduces sum((Y - C)^2) / sum(C^2) over the tile
// into one fp64 partial, so candidate outputs never reach HBM.
#include "common.h"

namespace awq {
namespace {

// ============================================================================
// MFMA path (fp16 / bf16)
// ============================================================================
constexpr int BM = 256;          // tokens per workgroup tile
constexpr int BN = 256;          // output channels per workgroup tile
constexpr int BK = 64;           // k per LDS stage (128 bytes per row)
constexpr int kThreads = 256;    // 4 waves, 2 x 2
constexpr int WTM = BM / 2;      // wave tile 128 x 128
constexpr int WTN = BN / 2;
constexpr int MI = WTM / 16;     // 16x16 MFMA blocks per wave along M
constexpr int NI = WTN / 16;
constexpr int kChunksPerRow = BK / 8;                       // 16-byte chunks per LDS row
constexpr int kLoadsPerThread = BM * kChunksPerRow / kThreads;  // per operand
constexpr int kGroupM = 8;       // row tiles per raster group

static_assert(BM == BN, "A and B tiles share the load mapping");

// 16-byte chunk c of LDS row r is stored at chunk c ^ (r & 7): the 16 lanes
// that read one fragment column hit 8 distinct chunks of 8 consecutive rows.
__device__ __forceinline__ int lds_chunk_offset(int row, int chunk) {
  return row * kChunksPerRow + (chunk ^ (row & 7));
}

template <typename S>
__device__ __forceinline__ f32x4 mfma16(i32x4 a, i32x4 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma16<_Float16>(i32x4 a, i32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                __builtin_bit_cast(half8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma16<__bf16>(i32x4 a, i32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Workgroup id -> (batch, tile_m, tile_n).  The dispatcher hands consecutive
// workgroup ids to the 8 XCDs in turn; the first remap makes the ids one XCD
// receives consecutive logical tiles (so they share operand blocks in that
// XCD's L2), the second orders tiles in groups of kGroupM row tiles.
struct TileId {
  int b, tm, tn;
};
__device__ __forceinline__ TileId map_tile(int g, int total, int tiles_m, int tiles_n) {
  const int per = total / 8, rem = total % 8;
  const int xcd = g % 8, idx = g / 8;
  const int L = (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  const int per_b = tiles_m * tiles_n;
  TileId t;
  t.b = L / per_b;
  const int r = L % per_b;
  const int span = kGroupM * tiles_n;
  const int grp = r / span;
  const int first_m = grp * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int in = r % span;
  t.tm = first_m + in % gm;
  t.tn = in / gm;
  return t;
}

template <typename S, Epi kEpi>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_mfma_kernel(const S* __restrict__ X, const S* __restrict__ B, int nb, int T, int N,
                      int K, float* __restrict__ Y, double* __restrict__ partials, int a0,
                      int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) i32x4 lds_a[2][BM * kChunksPerRow];
  __shared__ __attribute__((aligned(16))) i32x4 lds_b[2][BN * kChunksPerRow];
  __shared__ double red[kThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const TileId tile = map_tile(blockIdx.x, gridDim.x, tiles_m, tiles_n);
  const int m0 = tile.tm * BM;
  const int n0 = tile.tn * BN;

  // Buffer resources: out-of-range offsets read as zero, which pads the
  // ragged edges of T, N and K.
  const uint32_t a_bytes = (uint32_t)((uint64_t)T * K * sizeof(S));
  const uint32_t b_bytes = (uint32_t)((uint64_t)N * K * sizeof(S));
  const S* Bb = B + (int64_t)tile.b * N * K;
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)X, (short)0, (int)a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc((void*)Bb, (short)0, (int)b_bytes, 0x00020000);

  // Load mapping: chunk id = tid + kThreads*i -> (row = id / 8, chunk = id % 8).
  uint32_t a_off[kLoadsPerThread], b_off[kLoadsPerThread];
  int st_off[kLoadsPerThread];
#pragma unroll
  for (int i = 0; i < kLoadsPerThread; ++i) {
    const int id = tid + kThreads * i;
    const int r = id / kChunksPerRow, c = id % kChunksPerRow;
    st_off[i] = lds_chunk_offset(r, c);
    const int gr = m0 + r, gn = n0 + r;
    a_off[i] = gr < T ? (uint32_t)(((int64_t)gr * K + c * 8) * sizeof(S)) : a_bytes;
    b_off[i] = gn < N ? (uint32_t)(((int64_t)gn * K + c * 8) * sizeof(S)) : b_bytes;
  }
  const int my_chunk = tid % kChunksPerRow;

  i32x4 stage_a[kLoadsPerThread], stage_b[kLoadsPerThread];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
    const bool k_ok = k0 + my_chunk * 8 < K;
    const uint32_t kb = (uint32_t)(k0 * sizeof(S));
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
      const uint32_t oa = (k_ok && a_off[i] != a_bytes) ? a_off[i] + kb : a_bytes;
      const uint32_t ob = (k_ok && b_off[i] != b_bytes) ? b_off[i] + kb : b_bytes;
      stage_a[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, oa, 0, 0);
      stage_b[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, ob, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
      lds_a[buf][st_off[i]] = stage_a[i];
      lds_b[buf][st_off[i]] = stage_b[i];
    }
  };

  f32x4 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + BK - 1) / BK;
  const int frow = lane & 15;   // fragment row within a 16-row block
  const int fk = lane >> 4;     // which 8-wide k slice of the 32-wide step

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      i32x4 fa[MI], fb[NI];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        fa[i] = lds_a[cur][lds_chunk_offset(wm * WTM + i * 16 + frow, kk * 4 + fk)];
#pragma unroll
      for (int j = 0; j < NI; ++j)
        fb[j] = lds_b[cur][lds_chunk_offset(wn * WTN + j * 16 + frow, kk * 4 + fk)];
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = mfma16<S>(fa[i], fb[j], acc[i][j]);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue.  Lane l of a 16x16 block holds rows 4*(l/16) + r, column l%16.
  const int ecol = lane & 15;
  const int erow = (lane >> 4) * 4;
  if (kEpi == Epi::kStore) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int n = n0 + wn * WTN + j * 16 + ecol;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = m0 + wm * WTM + i * 16 + erow + r;
          if (t < T && n < N) Y[(int64_t)t * N + n] = acc[i][j][r];
        }
      }
    return;
  }
  double sse = 0.0;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int n = n0 + wn * WTN + j * 16 + ecol;
      float part = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = m0 + wm * WTM + i * 16 + erow + r;
        float e;
        if (kEpi == Epi::kSseRef) {
          e = (t < T && n < N) ? Y[(int64_t)t * N + n] - acc[i][j][r] : 0.0f;
        } else {
          e = acc[i][j][r];
        }
        part += e * e;
      }
      sse += (double)part;
    }
  // wave reduction in fp64, then the 4 waves in order
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sse += __shfl_xor(sse, off);
  if (lane == 0) red[wave] = sse;
  __syncthreads();
  if (tid == 0) {
    const double s = (red[0] + red[1]) + (red[2] + red[3]);
    partials[((int64_t)(a0 + tile.b) * tiles_m + tile.tm) * tiles_n + tile.tn] = s;
  }
}

// ============================================================================
// fp32 path (vector ALU): 64 x 64 tiles, 16-deep k stages, 4 x 4 outputs per
// lane.  Used for fp32 layers, which are small.
// ============================================================================
constexpr int FT = 64;
constexpr int FK = 16;

__global__ __launch_bounds__(256) void gemm_f32_kernel(Epi epi, const float* __restrict__ X,
                                                       const float* __restrict__ B, int T, int N,
                                                       int K, float* __restrict__ Y,
                                                       double* __restrict__ partials, int a0,
                                                       int tiles_m, int tiles_n) {
  __shared__ float xs[FK][FT + 4];
  __shared__ float bs[FK][FT + 4];
  __shared__ double red[4];
  const int per_b = tiles_m * tiles_n;
  const int b = blockIdx.x / per_b;
  const int r = blockIdx.x % per_b;
  const int tm = r / tiles_n, tn = r % tiles_n;
  const int m0 = tm * FT, n0 = tn * FT;
  const float* Bb = B + (int64_t)b * N * K;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += FK) {
    for (int e = threadIdx.x; e < FT * FK; e += 256) {
      const int rr = e / FK, kk = e % FK;
      const int t = m0 + rr, n = n0 + rr, k = k0 + kk;
      xs[kk][rr] = (t < T && k < K) ? X[(int64_t)t * K + k] : 0.0f;
      bs[kk][rr] = (n < N && k < K) ? Bb[(int64_t)n * K + k] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FK; ++kk) {
      float xv[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xv[i] = xs[kk][ty * 4 + i];
        bv[i] = bs[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xv[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  double sse = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (t >= T || n >= N) continue;
      if (epi == Epi::kStore) {
        Y[(int64_t)t * N + n] = acc[i][j];
      } else {
        const float e = (epi == Epi::kSseRef) ? Y[(int64_t)t * N + n] - acc[i][j] : acc[i][j];
        sse += (double)(e * e);
      }
    }
  if (epi == Epi::kStore) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sse += __shfl_xor(sse, off);
  if (lane == 0) red[wave] = sse;
  __syncthreads();
  if (threadIdx.x == 0)
    partials[((int64_t)(a0 + b) * tiles_m + tm) * tiles_n + tn] =
        (red[0] + red[1]) + (red[2] + red[3]);
}

// ============================================================================
// loss[k] = (sum of partials of alpha k, fixed order) / (T N); argmin (lowest
// index on a tie); s_best = s_table[argmin].  One workgroup.
// ============================================================================
__global__ __launch_bounds__(256) void loss_argmin_kernel(const double* __restrict__ partials,
                                                          int n_alpha, int64_t tiles,
                                                          double inv_count,
                                                          const float* __restrict__ s_table,
                                                          int64_t K, double* __restrict__ losses,
                                                          int32_t* __restrict__ best,
                                                          float* __restrict__ s_best) {
  __shared__ double red[256];
  __shared__ int best_sh;
  for (int k = 0; k < n_alpha; ++k) {
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < tiles; i += 256) s += partials[(int64_t)k * tiles + i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
      if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
      __syncthreads();
    }
    if (threadIdx.x == 0) losses[k] = red[0] * inv_count;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    int bi = 0;
    for (int k = 1; k < n_alpha; ++k)
      if (losses[k] < losses[bi]) bi = k;
    best_sh = bi;
    *best = bi;
  }
  __syncthreads();
  const float* src = s_table + (int64_t)best_sh * K;
  for (int64_t j = threadIdx.x; j < K; j += 256) s_best[j] = src[j];
}

template <typename S, Epi kEpi>
hipError_t launch_mfma(const void* X, const void* B, int nb, int64_t T, int64_t N, int64_t K,
                       float* Y, double* partials, int a0, hipStream_t st) {
  const int tiles_m = (int)((T + BM - 1) / BM);
  const int tiles_n = (int)((N + BN - 1) / BN);
  const int total = tiles_m * tiles_n * nb;
  gemm_mfma_kernel<S, kEpi><<<total, kThreads, 0, st>>>(
      static_cast<const S*>(X), static_cast<const S*>(B), nb, (int)T, (int)N, (int)K, Y, partials,
      a0, tiles_m, tiles_n);
  return hipGetLastError();
}

template <typename S>
hipError_t dispatch_epi(Epi epi, const void* X, const void* B, int nb, int64_t T, int64_t N,
                        int64_t K, float* Y, double* partials, int a0, hipStream_t st) {
  switch (epi) {
    case Epi::kStore: return launch_mfma<S, Epi::kStore>(X, B, nb, T, N, K, Y, partials, a0, st);
    case Epi::kSseRef: return launch_mfma<S, Epi::kSseRef>(X, B, nb, T, N, K, Y, partials, a0, st);
    default: return launch_mfma<S, Epi::kSseDelta>(X, B, nb, T, N, K, Y, partials, a0, st);
  }
}

}  // namespace

GemmTiles gemm_tiles(awq_dtype_t dt) {
  if (dt == AWQ_F32) return GemmTiles{FT, FT};
  return GemmTiles{BM, BN};
}

hipError_t launch_gemm(Epi epi, awq_dtype_t dt, const void* X, const void* B, int nb, int64_t T,
                       int64_t N, int64_t K, float* Y, double* partials, int a0, hipStream_t st) {
  ProfScope p(epi == Epi::kStore ? "awq_gemm_ref_output" : "awq_gemm_sse", st);
  if (dt == AWQ_F32) {
    const int tiles_m = (int)((T + FT - 1) / FT);
    const int tiles_n = (int)((N + FT - 1) / FT);
    gemm_f32_kernel<<<tiles_m * tiles_n * nb, 256, 0, st>>>(
        epi, static_cast<const float*>(X), static_cast<const float*>(B), (int)T, (int)N, (int)K, Y,
        partials, a0, tiles_m, tiles_n);
    return hipGetLastError();
  }
  if (dt == AWQ_F16) return dispatch_epi<_Float16>(epi, X, B, nb, T, N, K, Y, partials, a0, st);
  return dispatch_epi<__bf16>(epi, X, B, nb, T, N, K, Y, partials, a0, st);
}

hipError_t launch_loss_argmin(const double* partials, int n_alpha, int64_t tiles_per_alpha,
                              double inv_count, const float* s_table, int64_t K, double* losses,
                              int32_t* best, float* s_best, hipStream_t st) {
  ProfScope p("awq_loss_argmin", st);
  loss_argmin_kernel<<<1, 256, 0, st>>>(partials, n_alpha, tiles_per_alpha, inv_count, s_table, K,
                                        losses, best, s_best);
  return hipGetLastError();
}

}  // namespace awq
