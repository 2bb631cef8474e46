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
//
// Workgroup tile 256 x 256, 4 waves in a 2 x 2 arrangement, each wave owns a
// 128 x 128 block = 8 x 8 MFMA 16x16x32 accumulators (256 fp32 registers).
// K advances 32 per stage through a ring of 4 LDS stages (32 KB each: A and B
// tiles of 256 rows x 64 bytes).  Operand tiles go global -> LDS directly
// (buffer_load_dwordx4 ... lds), three stages ahead of the MFMAs, so the
// ~1000-cycle MFMA time of a stage hides three stages of load latency and no
// VGPRs are spent on staging.  One barrier per stage.
// ============================================================================
constexpr int BM = 256;          // tokens per workgroup tile
constexpr int BN = 256;          // output channels per workgroup tile
constexpr int BK = 32;           // k per LDS stage: 64 bytes per row
constexpr int kStages = 4;
constexpr int kThreads = 256;    // 4 waves, 2 x 2
constexpr int WTM = BM / 2;      // wave tile 128 x 128
constexpr int WTN = BN / 2;
constexpr int MI = WTM / 16;     // 16x16 MFMA blocks per wave along M
constexpr int NI = WTN / 16;
constexpr int kRowBytes = BK * 2;                       // 64
constexpr int kTileBytes = BM * kRowBytes;              // 16 KB per operand per stage
constexpr int kStageBytes = 2 * kTileBytes;             // A then B
constexpr int kSlabRows = 64 * 16 / kRowBytes;          // rows one wave-wide DMA fills: 16
constexpr int kDmaPerWave = BM / kSlabRows / 4;         // per operand per stage: 4
constexpr int kGroupM = 8;       // row tiles per raster group

static_assert(BM == BN, "A and B tiles share the load mapping");
static_assert(kRowBytes == 64, "swizzle below assumes 4 chunks of 16 bytes per row");

// 16-byte chunk c of LDS row r sits at chunk c ^ ((r >> 1) & 3): the 8 lanes
// of a ds_read_b128 phase (8 consecutive rows, one chunk) cover all 32 banks.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 3); }

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

// Buffer resource of a raw byte range: loads at offsets >= num_bytes return 0.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t num_bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)b, (int)(uint32_t)(b >> 32), (int)num_bytes, 0x00020000};
}

// 16 bytes per lane from rsrc + voff into LDS at m0 + 16 * lane.  Issued as
// inline asm so the compiler does not serialise the ring with a full
// vmcnt(0) before every LDS read; the kernel waits with explicit counts.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory");
}

// Wait until at most n DMA instructions of this lane are outstanding.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
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
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStageBytes];
  __shared__ double red[kThreads / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const TileId tile = map_tile(blockIdx.x, gridDim.x, tiles_m, tiles_n);
  const int m0 = tile.tm * BM;
  const int n0 = tile.tn * BN;

  const uint32_t a_bytes = (uint32_t)((uint64_t)T * K * sizeof(S));
  const uint32_t b_bytes = (uint32_t)((uint64_t)N * K * sizeof(S));
  const i32x4 ra = make_rsrc(X, a_bytes);
  const i32x4 rb = make_rsrc(B + (int64_t)tile.b * N * K, b_bytes);

  // DMA mapping: wave w, instruction i fills slab w*4 + i (16 rows); lane l
  // lands on row l/4, physical chunk l%4 and so fetches logical chunk
  // swz(row, l%4) of that row.  Rows past T or N read as zero.
  uint32_t a_off[kDmaPerWave], b_off[kDmaPerWave];
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int row = (wave * kDmaPerWave + i) * kSlabRows + (lane >> 2);
    const int c = swz(row, lane & 3);
    a_off[i] = (m0 + row < T) ? (uint32_t)(((int64_t)(m0 + row) * K + c * 8) * sizeof(S)) : a_bytes;
    b_off[i] = (n0 + row < N) ? (uint32_t)(((int64_t)(n0 + row) * K + c * 8) * sizeof(S)) : b_bytes;
  }
  const uint32_t smem_base = (uint32_t)(uintptr_t)smem;
  auto issue = [&](int kt) {
    const uint32_t st = smem_base + (uint32_t)((kt % kStages) * kStageBytes);
    const uint32_t kb = (uint32_t)(kt * BK * sizeof(S));
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
      const uint32_t slab = (uint32_t)((wave * kDmaPerWave + i) * 1024);
      dma16(ra, __builtin_amdgcn_readfirstlane(st + slab),
            a_off[i] == a_bytes ? a_bytes : a_off[i] + kb);
      dma16(rb, __builtin_amdgcn_readfirstlane(st + kTileBytes + slab),
            b_off[i] == b_bytes ? b_bytes : b_off[i] + kb);
    }
  };

  // Fragment reads: row = wave block + i*16 + lane%16, chunk lane/16; the
  // swizzle term depends on lane%16 only, so the in-block offset is per-lane.
  const int frow = lane & 15;
  const uint32_t frag_off = (uint32_t)(frow * kRowBytes + 16 * swz(frow, lane >> 4));
  const uint32_t a_frag = (uint32_t)(wm * WTM * kRowBytes) + frag_off;
  const uint32_t b_frag = (uint32_t)(kTileBytes + wn * WTN * kRowBytes) + frag_off;

  f32x4 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto read_frags = [&](int kt, i32x4 (&fa)[MI], i32x4 (&fb)[NI]) {
    const char* st = smem + (kt % kStages) * kStageBytes;
#pragma unroll
    for (int i = 0; i < MI; ++i)
      fa[i] = *reinterpret_cast<const i32x4*>(st + a_frag + i * 16 * kRowBytes);
#pragma unroll
    for (int j = 0; j < NI; ++j)
      fb[j] = *reinterpret_cast<const i32x4*>(st + b_frag + j * 16 * kRowBytes);
  };

  // Pipeline: stage s is DMA'd into buffer s % 4 four stages before its
  // MFMAs; its fragments are read into registers during the previous stage's
  // MFMAs.  At the top of iteration kt every wave has finished reading buffer
  // kt % 4 (it read stage kt's fragments in iteration kt - 1), so after the
  // barrier that buffer can take stage kt + 4.
  const int nk = K / BK;                      // K is a multiple of 32
#pragma unroll
  for (int s = 0; s < kStages; ++s)
    if (s < nk) issue(s);
  if (nk > 3) wait_vm<3 * 2 * kDmaPerWave>();
  else if (nk > 2) wait_vm<2 * 2 * kDmaPerWave>();
  else if (nk > 1) wait_vm<2 * kDmaPerWave>();
  else wait_vm<0>();
  __syncthreads();
  i32x4 fa[MI], fb[NI], ga[MI], gb[NI];
  read_frags(0, fa, fb);

  // One stage: wait for stage kt + 1, let the ring advance, read stage
  // kt + 1's fragments into (na, nb) while the MFMAs consume (ca, cb).
  auto step = [&](int kt, i32x4(&ca)[MI], i32x4(&cb)[NI], i32x4(&na)[MI], i32x4(&nb)[NI]) {
    // stage kt + 1 has landed once only stages kt + 2 and kt + 3 may pend
    if (kt + 3 < nk) wait_vm<2 * 2 * kDmaPerWave>();
    else if (kt + 2 < nk) wait_vm<2 * kDmaPerWave>();
    else wait_vm<0>();
    __syncthreads();
    if (kt + kStages < nk) issue(kt + kStages);
    if (kt + 1 < nk) read_frags(kt + 1, na, nb);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) acc[i][j] = mfma16<S>(ca[i], cb[j], acc[i][j]);
  };
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(kt, fa, fb, ga, gb);
    step(kt + 1, ga, gb, fa, fb);
  }
  if (kt < nk) step(kt, fa, fb, ga, gb);

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
  for (int i = 0; i < MI; ++i) {
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int n = n0 + wn * WTN + j * 16 + ecol;
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
