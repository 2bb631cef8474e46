// GPTQ error feedback after the AWQ scaling (AWQ + GPTQ), all in fp64 except
// the quantiser itself.
//
// "52 · AWQ, GPTQ và SmoothQuant", section 4: the weights are rounded one
// column at a time and each column's rounding error is moved onto the columns
// not yet rounded, spread according to the second-order statistics of real
// inputs.  "GPTQ与AWQ" (study notes), GPTQ section: column-wise quantisation
// with Hessian-guided compensation of each column's error into the later
// columns, and a Cholesky factorisation done once up front instead of an
// inverse per column.  AWQ reading notes, section "Experiment": AWQ's scaling
// and GPTQ's compensation are complementary, so GPTQ runs on the scaled
// weights W diag(s) with the inputs they meet, X diag(s)^-1.
//
// With H = X'^T X' (X' = X diag(s)^-1), damped and with dead channels fixed,
// and U upper triangular with U^T U = H^-1, the column loop is
//   q_j = quant(w_j);  e = (w_j - q_j) / U[j, j];  w_k -= e U[j, k] (k > j)
// for every row independently.  U comes without forming H^-1:
//   reversed H (P H P, P the index reversal) = L L^T (Cholesky, lower L)
//   => H = R R^T with R = P L P upper  => U = R^-1 = P L^-1 P.
// So the path is: H of the reversed columns (one MFMA GEMM per token chunk),
// damping, a right-looking blocked Cholesky (64-wide panels), a bottom-up
// recursive inverse of L (every level two batched GEMMs), one in-place
// reversal that turns L^-1 into U, then the column loop in blocks of 64
// columns (one kernel, lane = weight row).  Errors are pushed on lazily, as
// GPTQ's batched updates do: each block's errors go at once to the rest of
// its 512-column super-block (a shallow GEMM), and every super-block's errors
// go to the columns beyond it in one deep GEMM.
//
// Every dense contraction runs on the fp64 MFMA (v_mfma_f64_16x16x4f64):
// a 64x64 or 128x128 tile per 256-thread workgroup, 2x2 waves, k staged
// through LDS 16 deep with the next stage prefetched into registers.
// Output lane layout of the MFMA (probed on gfx950): lane l, element i holds
// row (l / 16) + 4 i, column l % 16 of the 16x16 block; inputs: lane l gives
// A[l % 16][l / 16] and B[l / 16][l % 16].
#include <math.h>

#include <algorithm>

#include "common.h"

namespace awq {
namespace {

typedef double d4 __attribute__((ext_vector_type(4)));
typedef double d2 __attribute__((ext_vector_type(2)));

constexpr int kNb = 64;            // panel / block width of the factorisation
constexpr int kKS = 16;            // k depth of one LDS stage
constexpr int kPad = 16;           // LDS row padding (doubles): rows 128 B off the banks
constexpr int kThreads = 256;
constexpr float kDeltaMin = 1e-10f;
// Columns whose errors are pushed on lazily: inside a super-block of kSuper
// columns every 64-column block updates the rest of the super-block at once;
// the columns beyond it are updated once per super-block, by one deep GEMM.
// A multiple of every group size, so a group never straddles two.
constexpr int kSuper = 512;

// Tile jobs of the fp64 GEMM.  C(m, n) = alpha sum_k A(m, k) B(n, k) + beta C(m, n).
enum Map : int {
  kRect = 0,     // grid (n tiles, m tiles); rows < M and columns < Nn are stored
  kLower = 1,    // tiles (i, j), off <= j <= i < off + r, blockIdx.x enumerates them
  kInvT1 = 2,    // inverse level, first product (stored transposed)
  kInvT2 = 3,    // inverse level, second product
};

struct GArgs {
  const double* a;
  const double* b;
  double* c;
  int64_t lda, ldb, ldc;
  int64_t M, Nn;      // kRect bounds
  int depth;          // kRect / kLower k extent (multiple of kKS)
  int off, r;         // kLower
  int h, nblk;        // inverse level: half width in blocks, blocks in total
  double alpha, beta;
};

struct Job {
  const double* a0;   // A(m0, k0)
  const double* b0;   // B(n0, k0)
  double* c0;         // C(m0, n0)
  int nk;             // k extent
  int mlim, nlim;     // valid rows / columns of the tile
  bool valid;
};

// (i, j) with j <= i from a row-major enumeration of a lower triangle.
__device__ __forceinline__ void tri_index(int t, int& i, int& j) {
  int r = (int)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
  while (r * (r + 1) / 2 > t) --r;
  while ((r + 1) * (r + 2) / 2 <= t) ++r;
  i = r;
  j = t - r * (r + 1) / 2;
}

template <int TILE, bool A_KC, bool B_KC, int MAP>
__device__ __forceinline__ Job make_job(const GArgs& g) {
  Job jb;
  jb.valid = true;
  // element (m, k) of a k-contiguous operand sits at m * ld + k, of an
  // mn-contiguous one at k * ld + m
  auto at = [](const double* p, int64_t ld, bool kc, int64_t m, int64_t k) {
    return kc ? p + m * ld + k : p + k * ld + m;
  };
  if constexpr (MAP == kRect) {
    const int64_t m0 = (int64_t)blockIdx.y * TILE, n0 = (int64_t)blockIdx.x * TILE;
    jb.a0 = at(g.a, g.lda, A_KC, m0, 0);
    jb.b0 = at(g.b, g.ldb, B_KC, n0, 0);
    jb.c0 = g.c + m0 * g.ldc + n0;
    jb.nk = g.depth;
    jb.mlim = g.M - m0 < TILE ? (int)(g.M - m0) : TILE;
    jb.nlim = g.Nn - n0 < TILE ? (int)(g.Nn - n0) : TILE;
  } else if constexpr (MAP == kLower) {
    int ti, tj;
    tri_index((int)blockIdx.x, ti, tj);
    const int64_t m0 = (int64_t)(g.off + ti) * TILE, n0 = (int64_t)(g.off + tj) * TILE;
    jb.a0 = at(g.a, g.lda, A_KC, m0, 0);
    jb.b0 = at(g.b, g.ldb, B_KC, n0, 0);
    jb.c0 = g.c + m0 * g.ldc + n0;
    jb.nk = g.depth;
    jb.mlim = TILE;
    jb.nlim = TILE;
  } else {
    // Subproblem s covers blocks [start, end); its first half [start, split)
    // and second half [split, end) are already inverted.  Tile (mt, nt) is
    // block (split + mt, start + nt) of the off-diagonal part.
    const int s = blockIdx.z, mt = blockIdx.y, nt = blockIdx.x;
    const int start = s * 2 * g.h, split = start + g.h;
    const int end = min(start + 2 * g.h, g.nblk);
    jb.mlim = TILE;
    jb.nlim = TILE;
    if (split + mt >= end) {
      jb.valid = false;
      return jb;
    }
    const int64_t ld = g.lda;   // all operands live in the one factor matrix
    const int64_t row = (int64_t)(split + mt) * TILE, col = (int64_t)(start + nt) * TILE;
    if constexpr (MAP == kInvT1) {
      // T1 = L[row block, first half] Linv[first half, col block]; Linv is
      // lower so only k blocks >= start + nt contribute.  Stored transposed
      // in the (unused) upper triangle: T1(m, n) at (col + n, row + m).
      jb.a0 = g.a + row * ld + col;             // k-contiguous, k from block start + nt
      jb.b0 = g.a + col * ld + col;             // mn-contiguous: (n, k) at k * ld + n
      jb.c0 = g.c + col * ld + row;             // transposed store
      jb.nk = (split - start - nt) * TILE;
    } else {
      // T2 = -Linv[second half] T1: Linv lower, k blocks split .. split + mt.
      const int64_t sp = (int64_t)split * TILE;
      jb.a0 = g.a + row * ld + sp;              // k-contiguous
      jb.b0 = g.a + col * ld + sp;              // T1^T rows: (n, k) at n * ld + k
      jb.c0 = g.c + row * ld + col;
      jb.nk = (mt + 1) * TILE;
    }
  }
  return jb;
}

template <int TILE, bool A_KC, bool B_KC, int MAP, bool C_T>
__global__ __launch_bounds__(kThreads) void gemm64_kernel(GArgs g) {
  constexpr int WT = TILE / 2;          // wave tile
  constexpr int F = WT / 16;            // 16x16 blocks per wave side
  constexpr int LS = TILE + kPad;       // LDS row stride (doubles)
  constexpr int PER = TILE * kKS / kThreads;   // doubles per thread per operand stage
  __shared__ __attribute__((aligned(16))) double As[2][kKS][LS];
  __shared__ __attribute__((aligned(16))) double Bs[2][kKS][LS];

  const Job jb = make_job<TILE, A_KC, B_KC, MAP>(g);
  if (!jb.valid) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * WT, wn = (wave & 1) * WT;
  const int64_t lda = g.lda, ldb = g.ldb;

  // Global -> register staging of one k stage of an operand (rows < lim only).
  // k-contiguous: TILE rows x 16 k, (256 / TILE) threads per row.
  // mn-contiguous: 16 k rows x TILE, 16 threads per k row.
  auto load = [&](const double* base, int64_t ld, bool kc, int lim, int k0, d2* r) {
    if (kc) {
      constexpr int tpr = kThreads / TILE, kpt = kKS / tpr;
      const int m = tid / tpr, kq = (tid % tpr) * kpt;
      const double* p = base + (int64_t)m * ld + k0 + kq;
#pragma unroll
      for (int v = 0; v < PER / 2; ++v)
        r[v] = m < lim ? *(const d2*)(p + 2 * v) : d2{0.0, 0.0};
    } else {
      constexpr int mpt = TILE / 16;
      const int k = tid / 16, m = (tid % 16) * mpt;
      const double* p = base + (int64_t)(k0 + k) * ld + m;
#pragma unroll
      for (int v = 0; v < PER / 2; ++v)
        r[v] = m + 2 * v < lim ? *(const d2*)(p + 2 * v) : d2{0.0, 0.0};
    }
  };
  auto store = [&](double (*S)[LS], bool kc, const d2* r) {
    if (kc) {
      constexpr int tpr = kThreads / TILE, kpt = kKS / tpr;
      const int m = tid / tpr, kq = (tid % tpr) * kpt;
#pragma unroll
      for (int v = 0; v < PER / 2; ++v) {
        S[kq + 2 * v][m] = r[v].x;
        S[kq + 2 * v + 1][m] = r[v].y;
      }
    } else {
      constexpr int mpt = TILE / 16;
      const int k = tid / 16, m = (tid % 16) * mpt;
#pragma unroll
      for (int v = 0; v < PER / 2; ++v) *(d2*)&S[k][m + 2 * v] = r[v];
    }
  };

  d4 acc[F][F];
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int j = 0; j < F; ++j) acc[i][j] = d4{0.0, 0.0, 0.0, 0.0};

  d2 ra[PER / 2], rb[PER / 2];
  const int nst = jb.nk / kKS;
  if (nst > 0) {
    load(jb.a0, lda, A_KC, jb.mlim, 0, ra);
    load(jb.b0, ldb, B_KC, jb.nlim, 0, rb);
    store(As[0], A_KC, ra);
    store(Bs[0], B_KC, rb);
  }
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int cur = st & 1;
    const bool more = st + 1 < nst;
    if (more) {
      load(jb.a0, lda, A_KC, jb.mlim, (st + 1) * kKS, ra);
      load(jb.b0, ldb, B_KC, jb.nlim, (st + 1) * kKS, rb);
    }
#pragma unroll
    for (int kk = 0; kk < kKS / 4; ++kk) {
      double av[F], bv[F];
#pragma unroll
      for (int i = 0; i < F; ++i) av[i] = As[cur][4 * kk + lane / 16][wm + 16 * i + lane % 16];
#pragma unroll
      for (int j = 0; j < F; ++j) bv[j] = Bs[cur][4 * kk + lane / 16][wn + 16 * j + lane % 16];
#pragma unroll
      for (int i = 0; i < F; ++i)
#pragma unroll
        for (int j = 0; j < F; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      store(As[cur ^ 1], A_KC, ra);
      store(Bs[cur ^ 1], B_KC, rb);
    }
    __syncthreads();
  }

  // Epilogue: lane holds rows (lane / 16) + 4 e, column lane % 16 of each block.
  const double alpha = g.alpha, beta = g.beta;
#pragma unroll
  for (int i = 0; i < F; ++i)
#pragma unroll
    for (int j = 0; j < F; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = wm + 16 * i + lane / 16 + 4 * e, n = wn + 16 * j + lane % 16;
        if (m < jb.mlim && n < jb.nlim) {
          double* p = C_T ? jb.c0 + (int64_t)n * g.ldc + m : jb.c0 + (int64_t)m * g.ldc + n;
          const double v = alpha * acc[i][j][e];
          *p = beta != 0.0 ? fma(beta, *p, v) : v;
        }
      }
}

template <int TILE, bool A_KC, bool B_KC, int MAP, bool C_T = false>
hipError_t gemm64(dim3 grid, const GArgs& g, hipStream_t st) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm64_kernel<TILE, A_KC, B_KC, MAP, C_T>), grid, dim3(kThreads), 0, st, g);
  return hipGetLastError();
}

// ---- Hessian of the reversed, scaled inputs --------------------------------
// Xc[t][i] = X[t0 + t][K-1-i] / s[K-1-i] in fp64 for t < rows and i < K; zero
// elsewhere (padding rows up to a stage multiple, padding columns up to Kp).
template <typename S>
__global__ void xs_rev_kernel(const S* __restrict__ X, const float* __restrict__ s, int64_t K,
                              int64_t t0, int rows, int rows_pad, int64_t Kp,
                              double* __restrict__ Xc) {
  const int64_t total = (int64_t)rows_pad * Kp;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = idx / Kp, i = idx % Kp;
    double v = 0.0;
    if (t < rows && i < K) {
      const int64_t j = K - 1 - i;
      v = (double)to_f32(X[(t0 + t) * K + j]) / (double)s[j];
    }
    Xc[idx] = v;
  }
}

// Dead channels (zero diagonal: no input reaches them) get a diagonal of 1,
// then damp * mean(diag) is added to the K real diagonal entries; padding
// entries get exactly 1.  dead[j] flags channel j in natural order.
__global__ __launch_bounds__(kThreads) void damp_kernel(double* __restrict__ H, int64_t K,
                                                        int64_t Kp, double damp,
                                                        uint8_t* __restrict__ dead) {
  __shared__ double red[kThreads];
  double sum = 0.0;
  for (int64_t i = threadIdx.x; i < Kp; i += kThreads) {
    double* p = H + i * Kp + i;
    if (i >= K) {
      *p = 1.0;
      continue;
    }
    const bool z = *p == 0.0;
    if (z) *p = 1.0;
    dead[K - 1 - i] = z ? 1 : 0;
    sum += *p;
  }
  red[threadIdx.x] = sum;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const double lam = damp * (red[0] / (double)K);
  for (int64_t i = threadIdx.x; i < K; i += kThreads) H[i * Kp + i] += lam;
}

// ---- Cholesky of one diagonal block and its inverse --------------------------
// One wave; lane r owns row r of the 64x64 block (lower part read only).  The
// factor L_pp itself is never needed again (the panel below is solved with
// its inverse, the later updates use the solved panel), so the block is
// overwritten with L_pp^-1 (zeros above the diagonal).  Both halves are
// right-looking, so the dependent chain per column is short and the updates
// of the later entries are independent FMAs.
__global__ __launch_bounds__(64) void chol_diag_kernel(double* __restrict__ H, int64_t ld, int p) {
  __shared__ double col[kNb];
  __shared__ double rdiag[kNb];
  __shared__ double Ls[kNb][kNb + 1];
  const int r = threadIdx.x;
  double* blk = H + (int64_t)p * kNb * ld + (int64_t)p * kNb;
  double a[kNb];
#pragma unroll
  for (int k = 0; k < kNb; ++k) a[k] = k <= r ? blk[(int64_t)r * ld + k] : 0.0;
  // factorisation: column j is scaled by 1 / L_jj, then every later column updated
#pragma unroll
  for (int j = 0; j < kNb; ++j) {
    if (r == j) {
      const double d = sqrt(a[j]);
      a[j] = d;
      rdiag[j] = 1.0 / d;
    }
    __syncthreads();
    if (r > j) {
      a[j] *= rdiag[j];
      col[r] = a[j];
    }
    __syncthreads();
    if (r > j) {
#pragma unroll
      for (int k = j + 1; k < kNb; ++k)
        if (k <= r) a[k] = fma(-a[j], col[k], a[k]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < kNb; ++k) Ls[r][k] = k <= r ? a[k] : 0.0;
  __syncthreads();
  // inverse: lane c solves L x = e_c, each x_i pushed into the later rows at once
  const int c = r;
  double acc[kNb], x[kNb];
#pragma unroll
  for (int i = 0; i < kNb; ++i) acc[i] = 0.0;
#pragma unroll
  for (int i = 0; i < kNb; ++i) {
    x[i] = ((i == c ? 1.0 : 0.0) - acc[i]) * rdiag[i];
#pragma unroll
    for (int m = i + 1; m < kNb; ++m) acc[m] = fma(Ls[m][i], x[i], acc[m]);
  }
#pragma unroll
  for (int i = 0; i < kNb; ++i) blk[(int64_t)i * ld + c] = x[i];
}

// U[a][b] = Linv[K-1-a][K-1-b]: swap every entry of the leading K x K block
// with its point reflection (in place; the lower triangle moves to the upper).
__global__ void reverse_kernel(double* __restrict__ H, int64_t K, int64_t ld) {
  const int64_t total = K * K;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < (total + 1) / 2;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t mir = total - 1 - idx;
    if (idx >= mir) continue;
    const int64_t a = idx / K, b = idx % K, a2 = mir / K, b2 = mir % K;
    double* p = H + a * ld + b;
    double* q = H + a2 * ld + b2;
    const double t = *p;
    *p = *q;
    *q = t;
  }
}

// ---- weights in the scaled space ----------------------------------------------
// Wc[n][k] = fp32(W[n][k] * s[k]) widened to fp64; dead channels are zeroed.
template <typename S>
__global__ void scaled_weights_kernel(const S* __restrict__ W, const float* __restrict__ s,
                                      const uint8_t* __restrict__ dead, int64_t N, int64_t K,
                                      double* __restrict__ Wc) {
  const int64_t total = N * K;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t k = idx % K;
    const float v = to_f32(W[idx]) * s[k];
    Wc[idx] = dead[k] ? 0.0 : (double)v;
  }
}

// ---- the column loop over one block of 64 columns --------------------------------
// Lane = weight row.  The block's 64 current values live in registers and the
// block's 64 x 64 piece of U is staged in LDS once (every lane reads the same
// U entries: broadcasts), so the only latency left per column is the
// quantiser's short dependent chain.  A group's step and zero-point come from
// its current values when the loop reaches its first column: inside the block
// for groups of at most 64 columns, else from this block's registers and the
// later columns in Wc (which already carry every earlier error).  Quantiser
// in IEEE fp32, one rounding per operation, quotients correctly rounded
// (div_rn with the reciprocal taken once per group):
//   delta = max((mx - mn) / qmax, 1e-10), z = clamp(rint(-mn / delta)),
//   c = clamp(rint(w / delta) + z), q = (c - z) * delta,
// with w, mn, mx the fp64 current values rounded to fp32.  The fp64 error
// (w - q) / U[j][j] is formed with the reciprocal of U[j][j].
struct BlockState {
  double w[64];            // current values of the block's columns
  float delta, rdelta, z, qmax, rq;
  uint64_t pack8;          // codes of the current 8 columns
  d2 epair;                // errors of the current 2 columns
  bool valid;
  int ncols, c0, gw;        // gw: the group width
  int64_t row, K, ng;
  const double* wr;        // this row's block in Wc
  const double (*us)[64];  // the block of U in LDS
  float* scales;
  uint8_t* zeros;
  uint8_t* codes8;
  double* err;             // this row-block's errors, row stride lde
  int64_t lde;
};

// Column J of the block (J a compile-time index, so w stays in registers).
template <int G, int J>
__device__ __forceinline__ void column_step(BlockState& b) {
  if (J < b.ncols) {
    const bool gstart = G <= 64 ? (J % G == 0) : (J == 0 && b.c0 % b.gw == 0);
    if (gstart) {
      double mn = b.w[J], mx = b.w[J];
      constexpr int in_regs = G <= 64 ? G : 64 - J;
#pragma unroll
      for (int k = 1; k < in_regs; ++k) {
        mn = fmin(mn, b.w[J + k]);
        mx = fmax(mx, b.w[J + k]);
      }
      if (G > 64 && b.valid) {
#pragma unroll 8
        for (int k = 64; k < b.gw; ++k) {
          const double v = b.wr[k];
          mn = fmin(mn, v);
          mx = fmax(mx, v);
        }
      }
      const float mn32 = (float)mn, mx32 = (float)mx;
      b.delta = fmaxf(div_rn(mx32 - mn32, b.qmax, b.rq), kDeltaMin);
      b.rdelta = 1.0f / b.delta;
      b.z = fminf(fmaxf(__builtin_rintf(div_rn(-mn32, b.delta, b.rdelta)), 0.0f), b.qmax);
      if (b.valid) {
        const int64_t gi = b.row * b.ng + (b.c0 + J) / b.gw;
        b.scales[gi] = b.delta;
        b.zeros[gi] = (uint8_t)b.z;
      }
    }
    const double* u = b.us[J];
    const double ru = 1.0 / u[J];
    const float w32 = (float)b.w[J];
    const float c = fminf(fmaxf(__builtin_rintf(div_rn(w32, b.delta, b.rdelta)) + b.z, 0.0f),
                          b.qmax);
    const float q = (c - b.z) * b.delta;
    b.pack8 |= (uint64_t)(uint32_t)c << (8 * (J % 8));
    const double e = (b.w[J] - (double)q) * ru;
    if (J % 2 == 0) b.epair.x = e; else b.epair.y = e;
#pragma unroll
    for (int k = J + 1; k < 64; ++k) b.w[k] = fma(-e, u[k], b.w[k]);
    if (J % 8 == 7 && b.valid) {
      *(uint64_t*)(b.codes8 + b.row * b.K + b.c0 + J - 7) = b.pack8;
      b.pack8 = 0;
    }
    if (J % 2 == 1 && b.valid) *(d2*)(b.err + b.row * b.lde + J - 1) = b.epair;
  }
}

template <int G, int J>
struct Columns {
  static __device__ __forceinline__ void run(BlockState& b) {
    column_step<G, J>(b);
    Columns<G, J + 1>::run(b);
  }
};
template <int G>
struct Columns<G, 64> {
  static __device__ __forceinline__ void run(BlockState&) {}
};

// G: the group width when it is 32 or 64 (groups start inside the block);
// 128 stands for every width of at least 128 (groups start at block starts).
template <int G>
__global__ __launch_bounds__(64) void gptq_block_kernel(
    const double* __restrict__ Wc, int64_t N, int64_t K, const double* __restrict__ U,
    int64_t ldu, int c0, int bits, int group, float* __restrict__ scales,
    uint8_t* __restrict__ zeros,
    uint8_t* __restrict__ codes8, double* __restrict__ err, int64_t lde) {
  __shared__ __attribute__((aligned(16))) double us[64][64];
  // U[c0 + r][c0 + l] -> us[r][l]: one coalesced 512-byte row per load
  {
    const int l = threadIdx.x;
    const double* src = U + (int64_t)c0 * ldu + c0 + l;
#pragma unroll 16
    for (int r = 0; r < 64; ++r) us[r][l] = src[(int64_t)r * ldu];
  }
  __syncthreads();
  BlockState b;
  b.us = us;
  b.row = (int64_t)blockIdx.x * 64 + threadIdx.x;
  b.valid = b.row < N;
  b.ncols = K - c0 < 64 ? (int)(K - c0) : 64;
  b.c0 = c0;
  b.K = K;
  b.gw = group;
  b.ng = K / group;
  b.qmax = (float)((1 << bits) - 1);
  b.rq = 1.0f / b.qmax;
  b.wr = Wc + b.row * K + c0;
  b.scales = scales;
  b.zeros = zeros;
  b.codes8 = codes8;
  b.err = err;
  b.lde = lde;
#pragma unroll
  for (int j = 0; j < 64; j += 2) {
    d2 v = d2{0.0, 0.0};
    if (b.valid && j < b.ncols) v = *(const d2*)(b.wr + j);
    b.w[j] = v.x;
    b.w[j + 1] = v.y;
  }
  b.delta = 1.0f;
  b.z = 0.0f;
  if (G > 64 && c0 % group != 0 && b.valid) {
    const int64_t gi = b.row * b.ng + c0 / group;
    b.delta = scales[gi];
    b.z = (float)zeros[gi];
  }
  b.rdelta = 1.0f / b.delta;
  b.pack8 = 0;
  b.epair = d2{0.0, 0.0};
  Columns<G, 0>::run(b);
}

// Pack uint8 codes [N][K] into each row's little-endian bitstream.
__global__ void pack_codes_kernel(const uint8_t* __restrict__ codes8, int64_t N, int64_t K,
                                  int bits, uint32_t* __restrict__ out) {
  const int64_t chunks = K / 32;
  const int64_t total = N * chunks;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = idx / chunks, ch = idx % chunks;
    const uint8_t* src = codes8 + n * K + ch * 32;
    uint32_t* dst = out + n * (K * bits / 32) + ch * bits;
    uint64_t acc = 0;
    int have = 0, wo = 0;
    for (int j = 0; j < 32; ++j) {
      acc |= (uint64_t)src[j] << have;
      have += bits;
      if (have >= 32) {
        dst[wo++] = (uint32_t)acc;
        acc >>= 32;
        have -= 32;
      }
    }
  }
}

int grid_for(int64_t total, int per_block = 256) {
  int64_t g = (total + per_block - 1) / per_block;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

#define RET_IF(e)                         \
  do {                                    \
    hipError_t err_ = (e);                \
    if (err_ != hipSuccess) return err_;  \
  } while (0)

}  // namespace

GptqLayout gptq_layout(int64_t N, int64_t K, int64_t T) {
  GptqLayout L;
  L.Kp = (K + 127) / 128 * 128;
  const int64_t tr = (T + kKS - 1) / kKS * kKS;
  L.chunk_rows = (int)(tr < 2048 ? tr : 2048);
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t off = 0;
  L.h_off = off;
  off += al((size_t)L.Kp * L.Kp * 8);
  L.xc_off = off;
  off += al((size_t)L.chunk_rows * L.Kp * 8);
  L.wc_off = off;
  off += al((size_t)N * K * 8);
  L.err_off = off;
  off += al((size_t)N * kSuper * 8);
  L.codes_off = off;
  off += al((size_t)N * K);
  L.dead_off = off;
  off += al((size_t)K);
  L.bytes = off;
  return L;
}

hipError_t launch_gptq(const void* W, const void* X, awq_dtype_t dt, int64_t N, int64_t K,
                       int64_t T, const float* s, int bits, int group, double damp,
                       uint32_t* codes, float* scales, uint8_t* zeros, void* ws, hipStream_t st) {
  const GptqLayout L = gptq_layout(N, K, T);
  char* base = (char*)ws;
  double* H = (double*)(base + L.h_off);
  double* Xc = (double*)(base + L.xc_off);
  double* Wc = (double*)(base + L.wc_off);
  double* E = (double*)(base + L.err_off);
  uint8_t* C8 = (uint8_t*)(base + L.codes_off);
  uint8_t* dead = (uint8_t*)(base + L.dead_off);
  const int64_t Kp = L.Kp;
  const int nblk = (int)(Kp / kNb);

  // 1. H of the reversed scaled inputs, lower tiles only, chunk by chunk
  {
    ProfScope ps("awq_gptq_hessian", st);
    const int r = (int)(Kp / 128);
    for (int64_t t0 = 0; t0 < T; t0 += L.chunk_rows) {
      const int rows = (int)std::min<int64_t>(L.chunk_rows, T - t0);
      const int rows_pad = (rows + kKS - 1) / kKS * kKS;
      const int gx = grid_for((int64_t)rows_pad * Kp);
      if (dt == AWQ_F16)
        hipLaunchKernelGGL(xs_rev_kernel<_Float16>, dim3(gx), dim3(256), 0, st,
                           (const _Float16*)X, s, K, t0, rows, rows_pad, Kp, Xc);
      else if (dt == AWQ_BF16)
        hipLaunchKernelGGL(xs_rev_kernel<__bf16>, dim3(gx), dim3(256), 0, st,
                           (const __bf16*)X, s, K, t0, rows, rows_pad, Kp, Xc);
      else
        hipLaunchKernelGGL(xs_rev_kernel<float>, dim3(gx), dim3(256), 0, st, (const float*)X,
                           s, K, t0, rows, rows_pad, Kp, Xc);
      RET_IF(hipGetLastError());
      GArgs g{};
      g.a = Xc;
      g.b = Xc;
      g.c = H;
      g.lda = g.ldb = Kp;
      g.ldc = Kp;
      g.depth = rows_pad;
      g.off = 0;
      g.r = r;
      g.alpha = 1.0;
      g.beta = t0 == 0 ? 0.0 : 1.0;
      RET_IF((gemm64<128, false, false, kLower>(dim3(r * (r + 1) / 2), g, st)));
    }
  }
  // 2. damping and dead channels; the scaled weights
  {
    ProfScope ps("awq_gptq_prep", st);
    hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(kThreads), 0, st, H, K, Kp, damp, dead);
    RET_IF(hipGetLastError());
    const int gx = grid_for(N * K);
    if (dt == AWQ_F16)
      hipLaunchKernelGGL(scaled_weights_kernel<_Float16>, dim3(gx), dim3(256), 0, st,
                         (const _Float16*)W, s, dead, N, K, Wc);
    else if (dt == AWQ_BF16)
      hipLaunchKernelGGL(scaled_weights_kernel<__bf16>, dim3(gx), dim3(256), 0, st,
                         (const __bf16*)W, s, dead, N, K, Wc);
    else
      hipLaunchKernelGGL(scaled_weights_kernel<float>, dim3(gx), dim3(256), 0, st,
                         (const float*)W, s, dead, N, K, Wc);
    RET_IF(hipGetLastError());
  }
  // 3. blocked Cholesky of the reversed H (lower), diagonal blocks inverted
  {
    ProfScope ps("awq_gptq_cholesky", st);
    for (int p = 0; p < nblk; ++p) {
      hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(64), 0, st, H, Kp, p);
      RET_IF(hipGetLastError());
      const int rest = nblk - p - 1;
      if (rest == 0) break;
      double* panel = H + (int64_t)(p + 1) * kNb * Kp + (int64_t)p * kNb;
      double* dinv = H + (int64_t)p * kNb * Kp + (int64_t)p * kNb;
      GArgs g{};
      // panel solve: A[i][p] <- A[i][p] Linv_pp^T (in place, per 64-row tile)
      g.a = panel;
      g.b = dinv;
      g.c = panel;
      g.lda = g.ldb = g.ldc = Kp;
      g.M = (int64_t)rest * kNb;
      g.Nn = kNb;
      g.depth = kNb;
      g.alpha = 1.0;
      g.beta = 0.0;
      RET_IF((gemm64<64, true, true, kRect>(dim3(1, rest), g, st)));
      // trailing update of the lower tiles: A[i][j] -= A[i][p] A[j][p]^T
      GArgs u{};
      u.a = H + (int64_t)p * kNb;
      u.b = H + (int64_t)p * kNb;
      u.c = H;
      u.lda = u.ldb = u.ldc = Kp;
      u.depth = kNb;
      u.off = p + 1;
      u.r = rest;
      u.alpha = -1.0;
      u.beta = 1.0;
      RET_IF((gemm64<64, true, true, kLower>(dim3(rest * (rest + 1) / 2), u, st)));
    }
  }
  // 4. L^-1 bottom-up: blocks of width 2h from two inverted halves
  {
    ProfScope ps("awq_gptq_inverse", st);
    for (int h = 1; h < nblk; h *= 2) {
      const int nsub = (nblk + 2 * h - 1) / (2 * h);
      GArgs g{};
      g.a = H;
      g.c = H;
      g.lda = g.ldb = g.ldc = Kp;
      g.h = h;
      g.nblk = nblk;
      g.alpha = 1.0;
      g.beta = 0.0;
      RET_IF((gemm64<64, true, false, kInvT1, true>(dim3(h, h, nsub), g, st)));
      g.alpha = -1.0;
      RET_IF((gemm64<64, true, true, kInvT2>(dim3(h, h, nsub), g, st)));
    }
    hipLaunchKernelGGL(reverse_kernel, dim3(grid_for((K * K + 1) / 2)), dim3(256), 0, st, H, K, Kp);
    RET_IF(hipGetLastError());
  }
  // 5. the column loop, 64 columns per step; each step's errors go to the rest
  //    of its super-block at once and to the columns beyond once per super-block
  {
    ProfScope ps("awq_gptq_columns", st);
    const int gb = (int)((N + 63) / 64);
    for (int64_t s0 = 0; s0 < K; s0 += kSuper) {
      const int64_t s1 = std::min<int64_t>(s0 + kSuper, K);
      for (int64_t c0 = s0; c0 < s1; c0 += 64) {
        double* eb = E + (c0 - s0);
#define AWQ_GPTQ_BLOCK(G)                                                                   \
  hipLaunchKernelGGL(gptq_block_kernel<G>, dim3(gb), dim3(64), 0, st, Wc, N, K, H, Kp, (int)c0, \
                     bits, group, scales, zeros, C8, eb, (int64_t)kSuper)
        switch (group) {
          case 32: AWQ_GPTQ_BLOCK(32); break;
          case 64: AWQ_GPTQ_BLOCK(64); break;
          default: AWQ_GPTQ_BLOCK(128); break;
        }
#undef AWQ_GPTQ_BLOCK
        RET_IF(hipGetLastError());
        const int64_t rest = s1 - c0 - 64;
        if (rest <= 0) continue;
        GArgs g{};
        g.a = eb;
        g.lda = kSuper;
        g.b = H + c0 * Kp + c0 + 64;
        g.ldb = Kp;
        g.c = Wc + c0 + 64;
        g.ldc = K;
        g.M = N;
        g.Nn = rest;
        g.depth = 64;
        g.alpha = -1.0;
        g.beta = 1.0;
        const dim3 grid((unsigned)((rest + 63) / 64), (unsigned)((N + 63) / 64));
        RET_IF((gemm64<64, true, false, kRect>(grid, g, st)));
      }
      const int64_t rest = K - s1;
      if (rest <= 0) break;
      GArgs g{};
      g.a = E;
      g.lda = kSuper;
      g.b = H + s0 * Kp + s1;
      g.ldb = Kp;
      g.c = Wc + s1;
      g.ldc = K;
      g.M = N;
      g.Nn = rest;
      g.depth = (int)(s1 - s0);
      g.alpha = -1.0;
      g.beta = 1.0;
      const dim3 grid((unsigned)((rest + 127) / 128), (unsigned)((N + 127) / 128));
      RET_IF((gemm64<128, true, false, kRect>(grid, g, st)));
    }
  }
  // 6. packed codes
  {
    ProfScope ps("awq_gptq_pack", st);
    hipLaunchKernelGGL(pack_codes_kernel, dim3(grid_for(N * (K / 32))), dim3(256), 0, st, C8, N,
                       K, bits, codes);
    RET_IF(hipGetLastError());
  }
  return hipSuccess;
}

}  // namespace awq
