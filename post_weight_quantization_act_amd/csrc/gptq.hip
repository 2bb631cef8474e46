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
  kStrict = 4,   // tiles (i, j), 0 <= j < i < r: the lower triangle without its diagonal
  kDiag = 5,     // the three lower TILE-tiles of each diagonal 2 TILE block d < r
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
  } else if constexpr (MAP == kLower || MAP == kStrict || MAP == kDiag) {
    int ti, tj;
    if constexpr (MAP == kDiag) {
      const int d = (int)blockIdx.x / 3, sub = (int)blockIdx.x % 3;
      ti = 2 * d + (sub > 0);
      tj = 2 * d + (sub == 2);
    } else {
      tri_index((int)blockIdx.x, ti, tj);
      if constexpr (MAP == kStrict) ++ti;
    }
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
__global__ __launch_bounds__(kThreads, 2) void gemm64_kernel(GArgs g) {
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

  // Two register sets keep the global loads of the next two stages in flight
  // while a stage multiplies out of LDS (double-buffered): stage st + 1 goes
  // to LDS at the end of stage st, stage st + 2 is loaded into the set that
  // stage st has just vacated.
  d2 ra0[PER / 2], rb0[PER / 2], ra1[PER / 2], rb1[PER / 2];
  const int nst = jb.nk / kKS;
  if (nst > 0) {
    load(jb.a0, lda, A_KC, jb.mlim, 0, ra0);
    load(jb.b0, ldb, B_KC, jb.nlim, 0, rb0);
  }
  if (nst > 1) {
    load(jb.a0, lda, A_KC, jb.mlim, kKS, ra1);
    load(jb.b0, ldb, B_KC, jb.nlim, kKS, rb1);
  }
  if (nst > 0) {
    store(As[0], A_KC, ra0);
    store(Bs[0], B_KC, rb0);
  }
  __syncthreads();
  auto step = [&](int st, d2* ra_free, d2* rb_free, const d2* ra_next, const d2* rb_next) {
    const int cur = st & 1;
    if (st + 2 < nst) {
      load(jb.a0, lda, A_KC, jb.mlim, (st + 2) * kKS, ra_free);
      load(jb.b0, ldb, B_KC, jb.nlim, (st + 2) * kKS, rb_free);
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
    if (st + 1 < nst) {
      store(As[cur ^ 1], A_KC, ra_next);
      store(Bs[cur ^ 1], B_KC, rb_next);
    }
    __syncthreads();
  };
  for (int st = 0; st < nst; st += 2) {
    step(st, ra0, rb0, ra1, rb1);
    if (st + 1 < nst) step(st + 1, ra1, rb1, ra0, rb0);
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
// Sixteen waves share the 64x64 block: lane r of every wave stands for row r,
// wave q owns the four columns 4q..4q+3 of that row in registers (lower part
// read only).  The factor L_pp itself is never needed again (the panel below
// is solved with its inverse, the later updates use the solved panel), so the
// block is overwritten with L_pp^-1 (zeros above the diagonal).
//
// Both halves go four columns per step, the steps unrolled by template
// recursion so every register index is static (a rolled loop would move the
// row to scratch memory).  Factorisation step JB: the wave owning columns
// JB..JB+3 gathers the 4x4 diagonal block by readlane and factors it in every
// lane (1/sqrt from the hardware estimate and two Newton steps), the rows
// below solve their four entries against it and the four columns are
// published in LDS (row-major L, one 32-byte write per lane); after one
// barrier every wave updates its own later columns with four FMAs each.
// Inverse step IB: lane c now stands for column c of L^-1 and wave q owns its
// rows 4q..4q+3; the wave owning rows IB..IB+3 solves the 4x4 block for
// x_IB..x_IB+3, publishes them in LDS and every wave pushes them into its own
// later rows.  Each entry sees the same operations in the same order as in a
// one-wave sweep of the whole row, so the split changes no bit of the result.
__device__ __forceinline__ double readlane64(double v, int lane) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)b, lane);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), lane);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// 1/sqrt(x) for x > 0 to a few ulps: the hardware estimate, then two Newton
// steps y <- y + y (1/2 - (x/2) y^2), each doubling the correct bits.
__device__ __forceinline__ double rsqrt64(double x) {
  double y = __builtin_amdgcn_rsq(x);
  const double h = 0.5 * x;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const double e = fma(-h * y, y, 0.5);
    y = fma(y, e, y);
  }
  return y;
}

constexpr int kCq = 4;               // columns (rows, in the inverse) per wave
constexpr int kQw = kNb / kCq;       // waves per block
typedef double LRow[kNb + 2];

// Columns i0..kCq-1 of this wave (global column kCq q + i) take the rank-4 update
// by the new columns JB..JB+3; w holds this row's own four new entries.
template <int I0>
__device__ __forceinline__ void chol_update(double* a, int kbase, int JB, d2 w0, d2 w1,
                                            const LRow* Lr) {
#pragma unroll
  for (int i = I0; i < kCq; ++i) {
    const int k = kbase + i;
    const d2 u0 = *(const d2*)&Lr[k][JB], u1 = *(const d2*)&Lr[k][JB + 2];
    double v = a[i];
    v = fma(-w0.x, u0.x, v);
    v = fma(-w0.y, u0.y, v);
    v = fma(-w1.x, u1.x, v);
    v = fma(-w1.y, u1.y, v);
    a[i] = v;
  }
}

template <int JB>
__device__ __forceinline__ void chol_step(double* a, int r, int q, LRow* Lr, double* rdiag) {
  if constexpr (JB < kNb) {
    constexpr int qo = JB / kCq, li = JB % kCq;
    if (q == qo) {
      double b[4][4], l[4][4], rr[4], x[4];
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int t = 0; t <= p; ++t) b[p][t] = readlane64(a[li + t], JB + p);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        double d = b[t][t];
#pragma unroll
        for (int s = 0; s < t; ++s) d = fma(-l[t][s], l[t][s], d);
        rr[t] = rsqrt64(d);
        l[t][t] = d * rr[t];
#pragma unroll
        for (int p = t + 1; p < 4; ++p) {
          double v = b[p][t];
#pragma unroll
          for (int s = 0; s < t; ++s) v = fma(-l[p][s], l[t][s], v);
          l[p][t] = v * rr[t];
        }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        double v = a[li + t];
#pragma unroll
        for (int s = 0; s < t; ++s) v = fma(-x[s], l[t][s], v);
        x[t] = v * rr[t];
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        double inblk = 0.0;
#pragma unroll
        for (int p = t; p < 4; ++p) inblk = r == JB + p ? l[p][t] : inblk;
        a[li + t] = r >= JB + 4 ? x[t] : inblk;
      }
      *(d2*)&Lr[r][JB] = d2{a[li], a[li + 1]};
      *(d2*)&Lr[r][JB + 2] = d2{a[li + 2], a[li + 3]};
      if (r == 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) rdiag[JB + t] = rr[t];
      }
    }
    __syncthreads();
    if (q == qo) {
      if constexpr (li + 4 < kCq)
        chol_update<li + 4>(a, qo * kCq, JB, d2{a[li], a[li + 1]}, d2{a[li + 2], a[li + 3]}, Lr);
    } else if (q > qo) {
      chol_update<0>(a, q * kCq, JB, *(const d2*)&Lr[r][JB], *(const d2*)&Lr[r][JB + 2], Lr);
    }
    chol_step<JB + 4>(a, r, q, Lr, rdiag);
  }
}

// Rows i0..kCq-1 of this wave (global row kCq q + i) of column c take the four
// new entries x_IB..x_IB+3.
template <int I0>
__device__ __forceinline__ void inv_update(double* a, int mbase, int IB, const double* x,
                                           const LRow* Lr) {
#pragma unroll
  for (int i = I0; i < kCq; ++i) {
    const int m = mbase + i;
    const d2 u0 = *(const d2*)&Lr[m][IB], u1 = *(const d2*)&Lr[m][IB + 2];
    double v = a[i];
    v = fma(u0.x, x[0], v);
    v = fma(u0.y, x[1], v);
    v = fma(u1.x, x[2], v);
    v = fma(u1.y, x[3], v);
    a[i] = v;
  }
}

template <int IB>
__device__ __forceinline__ void inv_step(double* a, int c, int q, const LRow* Lr,
                                         const double* rdiag, double (*Xs)[kNb], double* blk,
                                         int64_t ld) {
  if constexpr (IB < kNb) {
    constexpr int qo = IB / kCq, li = IB % kCq;
    if (q == qo) {
      double x[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        double v = (IB + t == c ? 1.0 : 0.0) - a[li + t];
#pragma unroll
        for (int s = 0; s < t; ++s) v = fma(-Lr[IB + t][IB + s], x[s], v);
        x[t] = v * rdiag[IB + t];
        blk[(int64_t)(IB + t) * ld + c] = x[t];
        if constexpr (qo + 1 < kQw) Xs[IB + t][c] = x[t];
      }
      if constexpr (li + 4 < kCq) inv_update<li + 4>(a, qo * kCq, IB, x, Lr);
    }
    if constexpr (qo + 1 < kQw) {
      __syncthreads();
      if (q > qo) {
        double x[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) x[t] = Xs[IB + t][c];
        inv_update<0>(a, q * kCq, IB, x, Lr);
      }
    }
    inv_step<IB + 4>(a, c, q, Lr, rdiag, Xs, blk, ld);
  }
}

__global__ __launch_bounds__(kNb * kQw) void chol_diag_kernel(double* __restrict__ H, int64_t ld,
                                                               int p) {
  __shared__ __attribute__((aligned(16))) LRow Lr[kNb];
  __shared__ double rdiag[kNb];
  __shared__ double Xs[kNb][kNb];
  const int r = threadIdx.x % kNb;
  const int q = __builtin_amdgcn_readfirstlane(threadIdx.x / kNb);
  double* blk = H + (int64_t)p * kNb * ld + (int64_t)p * kNb;
  double a[kCq];
#pragma unroll
  for (int i = 0; i < kCq; ++i) {
    const int k = q * kCq + i;
    a[i] = k <= r ? blk[(int64_t)r * ld + k] : 0.0;
  }
  chol_step<0>(a, r, q, Lr, rdiag);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kCq; ++i) a[i] = 0.0;
  inv_step<0>(a, r, q, Lr, rdiag, Xs, blk, ld);
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
// Lane = weight row; 64 rows per workgroup (one wave).  The block's piece of
// U (transposed, so a column of U is a contiguous LDS row) and the rows'
// current values are staged in LDS.  The 64 columns go in sub-blocks of 16:
// a sub-block's values sit in registers and are quantised one column at a
// time, each error pushed into the sub-block's later columns at once; then
// the sub-block's 16 errors are pushed into the block's later columns (16
// FMAs per column, a rolled loop).  Loops stay rolled where they can:
// straight-line code run once per launch spends its time fetching
// instructions.
//
// A group's step and zero-point come from its current values when the loop
// reaches its first column: from LDS for groups of at most 64 columns, else
// from LDS and the later columns in Wc (which already carry every earlier
// error).  Quantiser in IEEE fp32, one rounding per operation, quotients
// correctly rounded (div_rn with the reciprocal taken once per group):
//   delta = max((mx - mn) / qmax, 1e-10), z = clamp(rint(-mn / delta)),
//   c = clamp(rint(w / delta) + z), q = (c - z) * delta,
// with w, mn, mx the fp64 current values rounded to fp32.  The fp64 error
// (w - q) / U[j][j] is formed with the reciprocal of U[j][j].
constexpr int kSub = 16;

// G: the group width when it is 32 or 64 (groups start inside the block);
// 128 stands for every width of at least 128 (groups start at block starts).
template <int G>
__global__ __launch_bounds__(kThreads) void gptq_block_kernel(
    const double* __restrict__ Wc, int64_t N, int64_t K, const double* __restrict__ U,
    int64_t ldu, int c0, int bits, int group, float* __restrict__ scales,
    uint8_t* __restrict__ zeros, uint8_t* __restrict__ codes8, double* __restrict__ err,
    int64_t lde) {
  __shared__ __attribute__((aligned(16))) double ut[64][66];   // ut[k][j] = U[c0 + j][c0 + k]
  __shared__ double wl[64][64];                                // wl[k][r]: current values of row r
  __shared__ double es[kSub][64];                              // a sub-block's errors
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int ncols = K - c0 < 64 ? (int)(K - c0) : 64;
  const int64_t ng = K / group;
  const float qmax = (float)((1 << bits) - 1), rq = 1.0f / qmax;
  {
    // thread t stages 16 entries of U's block and 16 current values of row
    // t / 4, all loads in flight at once
    const int j = t >> 2, k0 = (t & 3) * 16;
    const double* us = U + (int64_t)(c0 + j) * ldu + c0 + k0;
    const int64_t rr = r0 + j;
    const bool vr = rr < N;
    const double* ws = Wc + rr * K + c0 + k0;
    d2 u[8], w[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      u[v] = *(const d2*)(us + 2 * v);
      w[v] = vr && k0 + 2 * v < ncols ? *(const d2*)(ws + 2 * v) : d2{0.0, 0.0};
    }
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      ut[k0 + 2 * v][j] = u[v].x;
      ut[k0 + 2 * v + 1][j] = u[v].y;
      wl[k0 + 2 * v][j] = w[v].x;
      wl[k0 + 2 * v + 1][j] = w[v].y;
    }
  }
  __syncthreads();
  const int64_t row = r0 + lane;
  const bool valid = row < N;
  const double* wr = Wc + row * K + c0;
  float delta = 1.0f, z = 0.0f;
  if (G > 64 && c0 % group != 0 && valid) {
    const int64_t gi = row * ng + c0 / group;
    delta = scales[gi];
    z = (float)zeros[gi];
  }
  float rdelta = 1.0f / delta;
#pragma unroll 1
  for (int s0 = 0; s0 < ncols; s0 += kSub) {
    if (wave == 0) {
      const bool gstart = G <= 64 ? (s0 % G == 0) : (s0 == 0 && c0 % group == 0);
      if (gstart) {
        const int gend = G <= 64 ? s0 + G : 64;
        double mn = wl[s0][lane], mx = mn;
#pragma unroll 4
        for (int k = s0 + 1; k < gend; ++k) {
          const double v = wl[k][lane];
          mn = fmin(mn, v);
          mx = fmax(mx, v);
        }
        if (G > 64 && valid) {
#pragma unroll 8
          for (int k = 64; k < group; ++k) {
            const double v = wr[k];
            mn = fmin(mn, v);
            mx = fmax(mx, v);
          }
        }
        const float mn32 = (float)mn, mx32 = (float)mx;
        delta = fmaxf(div_rn(mx32 - mn32, qmax, rq), kDeltaMin);
        rdelta = 1.0f / delta;
        z = fminf(fmaxf(__builtin_rintf(div_rn(-mn32, delta, rdelta)), 0.0f), qmax);
        if (valid) {
          const int64_t gi = row * ng + (c0 + s0) / group;
          scales[gi] = delta;
          zeros[gi] = (uint8_t)z;
        }
      }
      double w[kSub], e[kSub];
#pragma unroll
      for (int jj = 0; jj < kSub; ++jj) w[jj] = wl[s0 + jj][lane];
      uint64_t pk[2] = {0, 0};
#pragma unroll
      for (int jj = 0; jj < kSub; ++jj) {
        const double ru = 1.0 / ut[s0 + jj][s0 + jj];
        const float w32 = (float)w[jj];
        const float c =
            fminf(fmaxf(__builtin_rintf(div_rn(w32, delta, rdelta)) + z, 0.0f), qmax);
        const float q = (c - z) * delta;
        pk[jj / 8] |= (uint64_t)(uint32_t)c << (8 * (jj % 8));
        e[jj] = (w[jj] - (double)q) * ru;
        es[jj][lane] = e[jj];
#pragma unroll
        for (int j2 = jj + 1; j2 < kSub; ++j2) w[j2] = fma(-e[jj], ut[s0 + j2][s0 + jj], w[j2]);
      }
      if (valid) {
        uint64_t* cp = (uint64_t*)(codes8 + row * K + c0 + s0);
        cp[0] = pk[0];
        cp[1] = pk[1];
        double* ep = err + row * lde + s0;
#pragma unroll
        for (int jj = 0; jj < kSub; jj += 2) *(d2*)(ep + jj) = d2{e[jj], e[jj + 1]};
      }
    }
    __syncthreads();
    // the sub-block's errors into the block's later columns, columns split
    // between the four waves
    double e[kSub];
#pragma unroll
    for (int jj = 0; jj < kSub; ++jj) e[jj] = es[jj][lane];
#pragma unroll 2
    for (int k = s0 + kSub + wave; k < ncols; k += 4) {
      double v = wl[k][lane];
      const double* uk = &ut[k][s0];
#pragma unroll
      for (int jj = 0; jj < kSub; ++jj) v = fma(-e[jj], uk[jj], v);
      wl[k][lane] = v;
    }
    __syncthreads();
  }
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
      // The r (r - 1) / 2 tiles below the diagonal as 128-tiles (two per CU fit at once, so
      // this count stays within one round where the full triangle would spill a few tiles
      // into a second), the diagonal blocks as three 64-tiles each in a second launch.
      RET_IF((gemm64<128, false, false, kStrict>(dim3(r * (r - 1) / 2), g, st)));
      RET_IF((gemm64<64, false, false, kDiag>(dim3(3 * r), g, st)));
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
      hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(kNb * kQw), 0, st, H, Kp, p);
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
  hipLaunchKernelGGL(gptq_block_kernel<G>, dim3(gb), dim3(kThreads), 0, st, Wc, N, K, H, Kp,     \
                     (int)c0,                                                                 \
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
      // 64-tiles: four fit on a CU at once, so the launch fills the chip in even rounds
      // (128-tiles, two per CU, left most of a second round idle at these sizes)
      const dim3 grid((unsigned)((rest + 63) / 64), (unsigned)((N + 63) / 64));
      RET_IF((gemm64<64, true, false, kRect>(grid, g, st)));
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
