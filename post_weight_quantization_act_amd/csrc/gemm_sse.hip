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
#include <type_traits>

#include "common.h"

namespace awq {
namespace {

// ============================================================================
// MFMA path (fp16 / bf16)
//
// Workgroup tile 256 tokens x 256 output channels, 8 waves in a 2 x 4
// arrangement, each wave owning a 128 x 64 block = 8 x 4 MFMA 16x16x32
// accumulators (128 fp32 registers).  K advances 32 per stage through a ring of
// 4 LDS stages (32 KB each: the A and B tiles, 256 rows x 64 bytes).  Operands
// are read in the tiled layout (see common.h), so each stage of each operand is
// one contiguous 16 KB block: wave-wide global -> LDS transfers
// (buffer_load_dwordx4 ... lds) of 1 KB, i.e. whole 128-byte lines, issued
// four stages ahead of their MFMAs and copied verbatim, already swizzled for
// the fragment reads.
//
// The waves run ping-pong: group 0 (waves 0-3, tile rows 0-127) and group 1
// (waves 4-7, rows 128-255) hold one wave on each SIMD.  In the first half of
// stage k group 0 issues its 32 MFMAs while group 1 reads stage k's fragments
// and transfers the B tile of stage k + 3; in the second half group 1 issues
// its MFMAs while group 0 transfers the A tile of stage k + 4 and reads stage
// k + 1's fragments.  A barrier separates the halves, so each SIMD's matrix
// pipe is fed by the two waves in turn and the memory work of one hides behind
// the MFMAs of the other.
//
// The kernel is persistent: one workgroup per CU walks the tiles
// first, first + G, first + 2G, ... (G workgroups), and the ring runs on across
// tile boundaries, so the first stages of the next tile are in flight while the
// last stages and the epilogue of the current one execute.
//
// The reference-output GEMM reads the caller's row-major W as its B operand
// instead (B_TILED = false): each lane then fetches its swizzled chunk of a
// row directly, and rows past N read as zero.
// ============================================================================
constexpr int BM = kTileRows;    // tokens per workgroup tile
constexpr int BN = kTileRows;    // output channels per workgroup tile
constexpr int BK = kStageK;      // k per LDS stage: 64 bytes per row
constexpr int kStages = 4;
constexpr int kWaves = 8;
constexpr int kWavesN = 4;       // 2 x 4 waves
constexpr int kThreads = 64 * kWaves;
constexpr int WTM = BM / (kWaves / kWavesN);   // wave tile 128 x 64
constexpr int WTN = BN / kWavesN;
constexpr int MI = WTM / 16;     // 16x16 MFMA blocks per wave along M
constexpr int NI = WTN / 16;
constexpr int kRowBytes = BK * 2;                       // 64
constexpr int kTileBytes = BM * kRowBytes;              // 16 KB per operand per stage
constexpr int kStageBytes = 2 * kTileBytes;             // A then B
constexpr int kSlabRows = 64 * 16 / kRowBytes;          // rows one wave-wide transfer fills: 16
constexpr int kDmaPerWave = BM / kSlabRows / (kWaves / 2);   // per operand per stage per wave of its group: 4
constexpr int kGroupM = 8;       // row tiles per raster group

static_assert(BM == BN, "A and B tiles share the load mapping");
static_assert(kTileBytes == kBlockBytes, "an LDS stage tile is one block of the tiled layout");
static_assert(kRowBytes == 64, "swizzle assumes 4 chunks of 16 bytes per row");

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
// INT8 operands travel as pairs of bytes through the same tiles (a 16-byte
// fragment is 16 int8 along k, and v_mfma_i32_16x16x64_i8 takes lane group g's
// bytes as k = 16 g .. 16 g + 15, the byte positions of the 16-bit case); the
// int32 accumulators ride in the fp32 accumulator registers bit for bit.
template <>
__device__ __forceinline__ f32x4 mfma16<I8Pair>(i32x4 a, i32x4 b, f32x4 c) {
  return __builtin_bit_cast(
      f32x4, __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, __builtin_bit_cast(i32x4, c), 0, 0, 0));
}

// The epilogue's value of an accumulator: fp32 as is; an INT8 product
// rescaled to real units, fp32(fp32(fp32(acc) * rs[t]) * cs[n]).
template <typename S>
__device__ __forceinline__ float acc_value(float a, const float* rs, const float* cs, int t, int n) {
  if constexpr (std::is_same<S, I8Pair>::value) {
    const float v = (float)__builtin_bit_cast(int, a) * rs[t];
    return v * cs[n];
  } else {
    return a;
  }
}

// Buffer resource of a raw byte range: loads at offsets >= num_bytes return 0.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t num_bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)b, (int)(uint32_t)(b >> 32), (int)num_bytes, 0x00020000};
}

// 16 bytes per lane from rsrc + voff into LDS at m0 + 16 * lane.  Issued as
// inline asm so the compiler does not serialise the ring with a full
// vmcnt(0) before every LDS read; the kernel waits with explicit counts.
// m0 is declared clobbered, so the compiler neither keeps a value of its own
// in m0 across the transfer nor skips the wait state it owes before its own
// next use of m0; inside the block, an SALU write of m0 needs one wait state
// before an LDS-DMA load reads it, hence the s_nop.  clang warns that m0 is a
// reserved register whenever it appears in a clobber list; the clobber is
// honoured all the same (the hazard recognizer pads after the block).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most n transfers of this lane are outstanding.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Logical tile index -> (batch, tile_m, tile_n), in groups of kGroupM row tiles
// so that consecutive indices share X row tiles and candidate column tiles.
// Workgroup g runs on XCD g % 8 (the dispatcher deals workgroup ids to the 8
// XCDs in turn); the kernel gives the workgroups of one XCD consecutive
// logical indices in every round, so they share operand blocks in its L2.
struct TileId {
  int b, tm, tn;
};
__device__ __forceinline__ TileId raster(int L, int tiles_m, int tiles_n) {
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

// Workgroup barrier that the instruction scheduler may not move anything
// across (it would otherwise hoist register-only MFMAs over it and break the
// alternation of the two wave groups).
__device__ __forceinline__ void sync_sched() {
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}

template <typename S, Epi kEpi, bool B_TILED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_mfma_kernel(const S* __restrict__ Xt, const S* __restrict__ B, int nb, int T, int N,
                         int K, float* __restrict__ Y, double* __restrict__ partials, int a0,
                         int tiles_m, int tiles_n, const float* __restrict__ rs,
                         const float* __restrict__ cs, int tile0, int ntiles) {
  __shared__ __attribute__((aligned(1024))) char smem[kStages * kStageBytes];
  __shared__ double red[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);
  const uint32_t gw = (uint32_t)__builtin_amdgcn_readfirstlane(wave & 3);
  const int nk = K / BK;                        // K is a multiple of 32
  // The launch runs logical tiles [tile0, tile0 + ntiles) of the batch; this
  // workgroup takes tile0 + first + r * G for r < n_rounds.  G is a multiple
  // of 8; when nk < kStages the host launches one workgroup per tile, so the
  // look-ahead never has to reach past the next tile.
  const int G = gridDim.x;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8, per_xcd = G / 8;
  const int total = ntiles;
  const int first = xcd * per_xcd + slot;
  const int n_rounds = first < total ? (total - first + G - 1) / G : 0;
  if (n_rounds == 0) return;
  const int nq = n_rounds * nk;                 // stages over all tiles
  auto tile_of = [&](int r) {
    TileId t = raster(tile0 + r * G + first, tiles_m, tiles_n);
    t.b = __builtin_amdgcn_readfirstlane(t.b);
    t.tm = __builtin_amdgcn_readfirstlane(t.tm);
    t.tn = __builtin_amdgcn_readfirstlane(t.tn);
    return t;
  };
  const i32x4 ra = make_rsrc(Xt, (uint32_t)((uint64_t)tiles_m * nk * kBlockBytes));
  const uint32_t b_bytes_rm = (uint32_t)((uint64_t)N * K * sizeof(S));
  const uint32_t smem_base = (uint32_t)(uintptr_t)smem;
  // Operand addressing of one tile.  A candidate matrix gets its own buffer
  // resource: all candidates of a batch together can exceed a 32-bit range.
  struct Ops {
    uint32_t a_base, b_base;
    i32x4 rb;
    int n0;
  };
  auto ops_of = [&](TileId t) {
    Ops o;
    o.a_base = (uint32_t)(t.tm * nk) * kBlockBytes;
    o.n0 = t.tn * BN;
    if (B_TILED) {
      o.rb = make_rsrc(B + (int64_t)t.b * tiles_n * BN * K, (uint32_t)((uint64_t)tiles_n * nk * kBlockBytes));
      o.b_base = (uint32_t)(t.tn * nk) * kBlockBytes;
    } else {
      o.rb = make_rsrc(B, b_bytes_rm);
      o.b_base = 0;
    }
    return o;
  };
  auto issue_a = [&](const Ops& o, int kt, int buf) {
    const uint32_t st = smem_base + (uint32_t)(buf * kStageBytes);
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
      const uint32_t slab = (gw * kDmaPerWave + i) * 1024u;
      dma16(ra, st + slab, o.a_base + (uint32_t)kt * kBlockBytes + slab + lane * 16);
    }
  };
  auto issue_b = [&](const Ops& o, int kt, int buf) {
    const uint32_t st = smem_base + (uint32_t)(buf * kStageBytes) + kTileBytes;
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
      const uint32_t slab = (gw * kDmaPerWave + i) * 1024u;
      if (B_TILED) {
        dma16(o.rb, st + slab, o.b_base + (uint32_t)kt * kBlockBytes + slab + lane * 16);
      } else {
        const int row = ((int)gw * kDmaPerWave + i) * kSlabRows + (lane >> 2);
        const int c = swizzle_chunk(row, lane & 3);
        const uint32_t off = (o.n0 + row < N)
            ? (uint32_t)(((int64_t)(o.n0 + row) * K + kt * BK + c * 8) * sizeof(S)) : b_bytes_rm;
        dma16(o.rb, st + slab, off);
      }
    }
  };

  const int frow = lane & 15;
  const uint32_t frag_off = (uint32_t)(frow * kRowBytes + 16 * swizzle_chunk(frow, lane >> 4));
  const uint32_t a_frag = (uint32_t)(wm * WTM * kRowBytes) + frag_off;
  const uint32_t b_frag = (uint32_t)(kTileBytes + wn * WTN * kRowBytes) + frag_off;
  f32x4 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto read_frags = [&](int buf, i32x4 (&fa)[MI], i32x4 (&fb)[NI]) {
    const char* st = smem + buf * kStageBytes;
#pragma unroll
    for (int i = 0; i < MI; ++i) fa[i] = *reinterpret_cast<const i32x4*>(st + a_frag + i * 16 * kRowBytes);
#pragma unroll
    for (int j = 0; j < NI; ++j) fb[j] = *reinterpret_cast<const i32x4*>(st + b_frag + j * 16 * kRowBytes);
  };
  auto mma = [&](i32x4 (&fa)[MI], i32x4 (&fb)[NI]) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) acc[i][j] = mfma16<S>(fa[i], fb[j], acc[i][j]);
  };
  // Stage q' is transferred iff q' < nq, four (A) / three (B) stages ahead;
  // once stage q is consumed a group may leave its transfers of stages q + 2
  // and q + 3 pending.
  auto wait_next = [&](int q) {
    if (q + 3 < nq) wait_vm<2 * kDmaPerWave>();
    else if (q + 2 < nq) wait_vm<kDmaPerWave>();
    else wait_vm<0>();
  };
  TileId cur = tile_of(0);
  TileId nxt = n_rounds > 1 ? tile_of(1) : cur;
  Ops oc = ops_of(cur), on = ops_of(nxt);
  if (grp == 0) {
#pragma unroll
    for (int s = 0; s < kStages; ++s)
      if (s < nk) issue_a(oc, s, s);
    if (nk > 3) wait_vm<3 * kDmaPerWave>();
    else if (nk > 2) wait_vm<2 * kDmaPerWave>();
    else if (nk > 1) wait_vm<kDmaPerWave>();
    else wait_vm<0>();
  } else {
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
      if (s < nk) issue_b(oc, s, s);
    if (nk > 2) wait_vm<2 * kDmaPerWave>();
    else if (nk > 1) wait_vm<kDmaPerWave>();
    else wait_vm<0>();
  }
  __syncthreads();
  i32x4 fa[MI], fb[NI];
  const int ecol = lane & 15, erow = (lane >> 4) * 4;
  auto epilogue = [&]() {
    const int m0 = cur.tm * BM, n0 = cur.tn * BN;
    // this wave's float4 pieces of the tile in the fragment layout (kRefOut, kSseRef)
    const int64_t frag0 = (((int64_t)cur.tm * tiles_n + cur.tn) * kWaves + wave) * (MI * NI * 64) + lane;
    if (kEpi == Epi::kRefOut) {
      f32x4* const yfrag = reinterpret_cast<f32x4*>(Y) + frag0;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) yfrag[(i * NI + j) * 64] = acc[i][j];
    } else if (kEpi == Epi::kStore) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int n = n0 + wn * WTN + j * 16 + ecol;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int tt = m0 + wm * WTM + i * 16 + erow + rr;
            if (tt < T && n < N) Y[(int64_t)tt * N + n] = acc_value<S>(acc[i][j][rr], rs, cs, tt, n);
          }
        }
    } else {
      double sse = 0.0;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        float part = 0.0f;
        // one 16-byte piece of the reference per block: 1 KB a wave, contiguous
        f32x4 yr[NI];
        if (kEpi == Epi::kSseRef) {
          const f32x4* const yfrag = reinterpret_cast<const f32x4*>(Y) + frag0;
#pragma unroll
          for (int j = 0; j < NI; ++j) yr[j] = yfrag[(i * NI + j) * 64];
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int n = n0 + wn * WTN + j * 16 + ecol;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int tt = m0 + wm * WTM + i * 16 + erow + rr;
            float e;
            if (kEpi == Epi::kSseRef)
              e = (tt < T && n < N) ? yr[j][rr] - acc_value<S>(acc[i][j][rr], rs, cs, tt, n) : 0.0f;
            else e = acc[i][j][rr];
            part += e * e;
          }
        }
        sse += (double)part;
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) sse += __shfl_xor(sse, off);
      if (lane == 0) red[wave] = sse;
      __syncthreads();
      if (tid == 0) {
        double s2 = 0.0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s2 += red[w];
        partials[((int64_t)(a0 + cur.b) * tiles_m + cur.tm) * tiles_n + cur.tn] = s2;
      }
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  // Tile r + 1 becomes current; its stages are already in flight.
  auto advance = [&](int r) {
    cur = nxt;
    oc = on;
    if (r + 2 < n_rounds) {
      nxt = tile_of(r + 2);
      on = ops_of(nxt);
    }
  };
  // The two groups run separate loops (grp is wave-uniform) that meet at the
  // same sequence of barriers: two per stage and one per tile epilogue.
  if (grp == 0) {
    read_frags(0, fa, fb);
    for (int r = 0; r < n_rounds; ++r) {
      const bool more = r + 1 < n_rounds;
      for (int kt = 0; kt < nk; ++kt) {
        const int q = r * nk + kt;
        mma(fa, fb);
        wait_next(q);
        sync_sched();
        if (kt + 4 < nk) issue_a(oc, kt + 4, q & 3);
        else if (more) issue_a(on, kt + 4 - nk, q & 3);
        read_frags((q + 1) & 3, fa, fb);   // past the last stage: unused
        sync_sched();
      }
      epilogue();
      advance(r);
    }
  } else {
    for (int r = 0; r < n_rounds; ++r) {
      const bool more = r + 1 < n_rounds;
      for (int kt = 0; kt < nk; ++kt) {
        const int q = r * nk + kt;
        read_frags(q & 3, fa, fb);
        if (kt + 3 < nk) issue_b(oc, kt + 3, (q + 3) & 3);
        else if (more) issue_b(on, kt + 3 - nk, (q + 3) & 3);
        wait_next(q);
        sync_sched();
        mma(fa, fb);
        sync_sched();
      }
      epilogue();
      advance(r);
    }
  }
}

// Row-major [R, K] -> tiled layout, one lane per 16-byte chunk of the output
// (coalesced writes; each group of 4 lanes reads one row's 64-byte stage slice).
template <typename S>
__global__ __launch_bounds__(256) void tile_rows_kernel(const S* __restrict__ src, int64_t R,
                                                        int64_t K, int64_t chunks,
                                                        S* __restrict__ dst) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= chunks) return;
  const int64_t nk = K / BK;
  const int64_t block = q / (kBlockBytes / 16);
  const int within = (int)(q % (kBlockBytes / 16));
  const int r = within / 4, p = within % 4;
  const int64_t t = block / nk, s = block % nk;
  const int64_t row = t * BM + r;
  const int c = swizzle_chunk(r, p);   // the swizzle is an involution
  i32x4 v = i32x4{0, 0, 0, 0};
  if (row < R) v = *reinterpret_cast<const i32x4*>(src + row * K + s * BK + c * 8);
  reinterpret_cast<i32x4*>(dst)[q] = v;
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
      if (epi == Epi::kStore || epi == Epi::kRefOut) {   // row-major on this path
        Y[(int64_t)t * N + n] = acc[i][j];
      } else {
        const float e = (epi == Epi::kSseRef) ? Y[(int64_t)t * N + n] - acc[i][j] : acc[i][j];
        sse += (double)(e * e);
      }
    }
  if (epi == Epi::kStore || epi == Epi::kRefOut) return;
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
// loss[k] = (sum of partials of alpha k, fixed order) / (T N), one workgroup
// per alpha: lane t sums tiles t, t + 1024, ... in index order, then a fixed
// butterfly across each wave and a fixed sum over the 16 waves.  Then one
// workgroup takes the argmin (lowest index on a tie) and copies s_best =
// s_table[argmin].
// ============================================================================
constexpr int kLossThreads = 1024;

__global__ __launch_bounds__(kLossThreads) void loss_reduce_kernel(
    const double* __restrict__ partials, int64_t tiles, double inv_count,
    double* __restrict__ losses) {
  __shared__ double red[kLossThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const double* p = partials + (int64_t)blockIdx.x * tiles;
  double s0 = 0.0, s1 = 0.0;
  int64_t i = threadIdx.x;
  for (; i + kLossThreads < tiles; i += 2 * kLossThreads) {
    s0 += p[i];
    s1 += p[i + kLossThreads];
  }
  if (i < tiles) s0 += p[i];
  double s = s0 + s1;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) red[wave] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kLossThreads / 64; ++w) t += red[w];
    losses[blockIdx.x] = t * inv_count;
  }
}

__global__ __launch_bounds__(kLossThreads) void loss_argmin_kernel(
    const double* __restrict__ losses, int n_alpha, const float* __restrict__ s_table, int64_t K,
    int32_t* __restrict__ best, float* __restrict__ s_best) {
  __shared__ int best_sh;
  if (threadIdx.x == 0) {
    int bi = 0;
    for (int k = 1; k < n_alpha; ++k)
      if (losses[k] < losses[bi]) bi = k;
    best_sh = bi;
    *best = bi;
  }
  __syncthreads();
  const float* src = s_table + (int64_t)best_sh * K;
  for (int64_t j = threadIdx.x; j < K; j += kLossThreads) s_best[j] = src[j];
}

// Compute units of the current device rounded down to a multiple of 8 (cached
// per device).
int persistent_workgroups() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 8)
      cus = 8;
    cached[dev] = cus / 8 * 8;
  }
  return cached[dev];
}

// The launch runs logical tiles [tile0, tile0 + ntiles) of the batch's
// nb * tiles_m * tiles_n (ntiles < 0: all from tile0 on).
template <typename S, Epi kEpi, bool B_TILED>
hipError_t launch_mfma(const void* X, const void* B, int nb, int64_t T, int64_t N, int64_t K,
                       float* Y, double* partials, int a0, hipStream_t st,
                       const float* rs = nullptr, const float* cs = nullptr, int tile0 = 0,
                       int ntiles = -1) {
  const int tiles_m = (int)((T + BM - 1) / BM);
  const int tiles_n = (int)((N + BN - 1) / BN);
  const int all = tiles_m * tiles_n * nb;
  if (tile0 < 0 || tile0 > all) return hipErrorInvalidValue;
  const int total = ntiles < 0 ? all - tile0 : ntiles;
  if (total < 1 || total > all - tile0) return hipErrorInvalidValue;
  // One workgroup per CU (a multiple of 8, one share per XCD), or one per tile
  // when there are fewer tiles or the ring is deeper than a tile.
  const int64_t per_tile = (total + 7) / 8 * 8;
  int grid = (int)per_tile;
  if (K / BK >= kStages) {
    const int cus = persistent_workgroups();
    if (cus < grid) grid = cus;
  }
  gemm_mfma_kernel<S, kEpi, B_TILED><<<grid, kThreads, 0, st>>>(
      static_cast<const S*>(X), static_cast<const S*>(B), nb, (int)T, (int)N, (int)K, Y, partials,
      a0, tiles_m, tiles_n, rs, cs, tile0, total);
  return hipGetLastError();
}

template <typename S>
hipError_t dispatch_epi(Epi epi, const void* X, const void* B, bool b_tiled, int nb, int64_t T,
                        int64_t N, int64_t K, float* Y, double* partials, int a0, hipStream_t st,
                        int tile0, int ntiles) {
  if (!b_tiled) {   // the reference output, from the row-major weights
    if (epi != Epi::kRefOut) return hipErrorInvalidValue;
    return launch_mfma<S, Epi::kRefOut, false>(X, B, nb, T, N, K, Y, partials, a0, st);
  }
  switch (epi) {
    case Epi::kSseRef:
      return launch_mfma<S, Epi::kSseRef, true>(X, B, nb, T, N, K, Y, partials, a0, st, nullptr,
                                                nullptr, tile0, ntiles);
    case Epi::kSseDelta:
      return launch_mfma<S, Epi::kSseDelta, true>(X, B, nb, T, N, K, Y, partials, a0, st, nullptr,
                                                  nullptr, tile0, ntiles);
    default: return hipErrorInvalidValue;
  }
}

template <typename S>
hipError_t tile_rows(const void* src, int64_t R, int64_t K, void* dst, hipStream_t st) {
  const int64_t chunks = padded_rows(R) * K * (int64_t)sizeof(S) / 16;
  tile_rows_kernel<S><<<(unsigned)((chunks + 255) / 256), 256, 0, st>>>(
      static_cast<const S*>(src), R, K, chunks, static_cast<S*>(dst));
  return hipGetLastError();
}

}  // namespace

int gemm_grid() { return persistent_workgroups(); }

GemmTiles gemm_tiles(awq_dtype_t dt) {
  if (dt == AWQ_F32) return GemmTiles{FT, FT};
  return GemmTiles{BM, BN};
}

hipError_t launch_gemm(Epi epi, awq_dtype_t dt, const void* X, const void* B, bool b_tiled,
                       int nb, int64_t T, int64_t N, int64_t K, float* Y, double* partials,
                       int a0, hipStream_t st, int tile0, int ntiles) {
  if (epi == Epi::kStore) return hipErrorInvalidValue;   // the reference output is kRefOut
  ProfScope p(epi == Epi::kRefOut ? "awq_gemm_ref_output" : "awq_gemm_sse", st);
  if (dt == AWQ_F32) {
    if (tile0 != 0 || ntiles >= 0) return hipErrorInvalidValue;   // whole batch only
    const int tiles_m = (int)((T + FT - 1) / FT);
    const int tiles_n = (int)((N + FT - 1) / FT);
    gemm_f32_kernel<<<tiles_m * tiles_n * nb, 256, 0, st>>>(
        epi, static_cast<const float*>(X), static_cast<const float*>(B), (int)T, (int)N, (int)K, Y,
        partials, a0, tiles_m, tiles_n);
    return hipGetLastError();
  }
  if (dt == AWQ_F16)
    return dispatch_epi<_Float16>(epi, X, B, b_tiled, nb, T, N, K, Y, partials, a0, st, tile0,
                                  ntiles);
  return dispatch_epi<__bf16>(epi, X, B, b_tiled, nb, T, N, K, Y, partials, a0, st, tile0,
                              ntiles);
}

hipError_t launch_gemm_w8a8(Epi epi, const void* Xq, const void* Wq, int64_t T, int64_t N,
                            int64_t K, const float* sx, const float* sw, float* Y,
                            double* partials, hipStream_t st) {
  ProfScope p(epi == Epi::kStore ? "awq_gemm_w8a8_store" : "awq_gemm_w8a8_sse", st);
  const int64_t Kp = K / 2;   // byte pairs: the 2-byte elements of the tiled layout
  if (epi == Epi::kStore)
    return launch_mfma<I8Pair, Epi::kStore, true>(Xq, Wq, 1, T, N, Kp, Y, partials, 0, st, sx, sw);
  if (epi == Epi::kSseRef)
    return launch_mfma<I8Pair, Epi::kSseRef, true>(Xq, Wq, 1, T, N, Kp, Y, partials, 0, st, sx, sw);
  return hipErrorInvalidValue;
}

hipError_t launch_tile_rows(const void* src, int64_t R, int64_t K, void* dst, hipStream_t st) {
  ProfScope p("awq_tile_rows", st);
  return tile_rows<_Float16>(src, R, K, dst, st);   // 2-byte elements: dtype-agnostic copy
}

hipError_t launch_loss_argmin(const double* partials, int n_alpha, int64_t tiles_per_alpha,
                              double inv_count, const float* s_table, int64_t K, double* losses,
                              int32_t* best, float* s_best, hipStream_t st) {
  ProfScope p("awq_loss_argmin", st);
  loss_reduce_kernel<<<(unsigned)n_alpha, kLossThreads, 0, st>>>(partials, tiles_per_alpha,
                                                                 inv_count, losses);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  loss_argmin_kernel<<<1, kLossThreads, 0, st>>>(losses, n_alpha, s_table, K, best, s_best);
  return hipGetLastError();
}

}  // namespace awq
