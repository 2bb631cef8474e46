// Per-input-channel activation magnitude a_j = mean_t |X[t, j]|.
//
// AWQ reading notes ("AWQ: Activation-Aware Weight Quantization For On-Device
// LLM Compression AND Acceleration"), section "Measures": the importance
// statistic is the average absolute activation of every input channel,
// gathered on calibration data.
//
// X is row-major [T, K]; the reduction runs down the columns, so a wavefront
// reads rows: 32 lanes cover 512 contiguous bytes of one row and the 2 lane
// sets of a wave read 2 rows.  Every lane accumulates its columns in fp64.
// Pass 1 sums a fixed chunk of rows per workgroup into fp64 partials
// [chunks, K]; pass 2 adds each column's chunks in a fixed order (8 lanes per
// column, each a strided share of the chunks, then a fixed tree in LDS) and
// divides by T, so the result does not depend on scheduling.
#include "common.h"

namespace awq {
namespace {

constexpr int kThreads = 256;
constexpr int kColThreads = 32;
constexpr int kRowThreads = kThreads / kColThreads;
constexpr int kTargetBlocks = 2048;   // ~8 workgroups per CU on 256 CUs
constexpr int kMinRowsPerChunk = 64;

// Chunking depends only on (T, K) so the workspace query needs no dtype.
void chunking(int64_t T, int64_t K, int64_t* chunks, int64_t* rows_per_chunk) {
  int64_t gx_ref = (K + 255) / 256;
  int64_t c = (kTargetBlocks + gx_ref - 1) / gx_ref;
  int64_t cmax = (T + kMinRowsPerChunk - 1) / kMinRowsPerChunk;
  if (c > cmax) c = cmax;
  if (c < 1) c = 1;
  int64_t rpc = (T + c - 1) / c;
  *rows_per_chunk = rpc;
  *chunks = (T + rpc - 1) / rpc;
}

template <typename S>
__device__ __forceinline__ void load_vec(const S* p, float (&v)[16 / sizeof(S)]) {
  constexpr int E = 16 / sizeof(S);
  i32x4 raw = *reinterpret_cast<const i32x4*>(p);
  const S* e = reinterpret_cast<const S*>(&raw);
#pragma unroll
  for (int i = 0; i < E; ++i) v[i] = to_f32(e[i]);
}

template <typename S, bool kVector>
__global__ __launch_bounds__(kThreads) void act_stats_partial(const S* __restrict__ X, int64_t T,
                                                              int64_t K, int64_t rpc,
                                                              double* __restrict__ part) {
  constexpr int E = 16 / sizeof(S);           // elements per lane per row
  constexpr int CB = kColThreads * E;         // columns per workgroup
  __shared__ double red[kRowThreads][CB];

  const int tx = threadIdx.x % kColThreads;
  const int ty = threadIdx.x / kColThreads;
  const int64_t col0 = (int64_t)blockIdx.x * CB + tx * E;
  const int64_t r_begin = (int64_t)blockIdx.y * rpc;
  int64_t r_end = r_begin + rpc;
  if (r_end > T) r_end = T;

  double acc[E];
#pragma unroll
  for (int i = 0; i < E; ++i) acc[i] = 0.0;

  if (kVector) {
    if (col0 < K) {
      const S* p = X + r_begin * K + col0;
      int64_t r = r_begin + ty;
      // eight rows in flight per lane (four measured 13% slower on 32 MB inputs,
      // the same on large ones); the additions stay in row order
      for (; r + 7 * kRowThreads < r_end; r += 8 * kRowThreads) {
        float v[8][E];
        const S* q = p + (r - r_begin) * K;
#pragma unroll
        for (int u = 0; u < 8; ++u) load_vec(q + u * kRowThreads * K, v[u]);
#pragma unroll
        for (int i = 0; i < E; ++i) {
#pragma unroll
          for (int u = 0; u < 8; ++u) acc[i] += (double)fabsf(v[u][i]);
        }
      }
      for (; r < r_end; r += kRowThreads) {
        float v[E];
        load_vec(p + (r - r_begin) * K, v);
#pragma unroll
        for (int i = 0; i < E; ++i) acc[i] += (double)fabsf(v[i]);
      }
    }
  } else {
    for (int64_t r = r_begin + ty; r < r_end; r += kRowThreads) {
#pragma unroll
      for (int i = 0; i < E; ++i) {
        if (col0 + i < K) acc[i] += (double)fabsf(to_f32(X[r * K + col0 + i]));
      }
    }
  }

#pragma unroll
  for (int i = 0; i < E; ++i) red[ty][tx * E + i] = acc[i];
  __syncthreads();
  if (threadIdx.x < CB) {
    double s = 0.0;
#pragma unroll
    for (int r = 0; r < kRowThreads; ++r) s += red[r][threadIdx.x];
    const int64_t c = (int64_t)blockIdx.x * CB + threadIdx.x;
    if (c < K) part[(int64_t)blockIdx.y * K + c] = s;
  }
}

// One workgroup per 32 columns: lane group q (8 lanes per column) sums chunks
// q, q + 8, q + 16, ... of its column, then the 8 sums are added in a fixed
// tree through LDS.
constexpr int kFinCols = 32;
constexpr int kFinSplit = kThreads / kFinCols;

__global__ __launch_bounds__(kThreads) void act_stats_finish(const double* __restrict__ part,
                                                             int64_t chunks, int64_t K, int64_t T,
                                                             float* __restrict__ a) {
  __shared__ double red[kFinSplit][kFinCols];
  const int c = threadIdx.x % kFinCols, q = threadIdx.x / kFinCols;
  const int64_t j = (int64_t)blockIdx.x * kFinCols + c;
  // Two running sums: s0 takes chunks q, q + 16, q + 32, ..., s1 chunks
  // q + 8, q + 24, ...  A batch of the lane's chunks is loaded before any is
  // added (the partials sit in L2 or the MALL: the round trips, not the
  // bandwidth, are the cost), then added in that order.
  constexpr int kFinBatch = 16;
  double s0 = 0.0, s1 = 0.0;
  if (j < K) {
    for (int64_t b = q; b < chunks; b += kFinBatch * kFinSplit) {
      double v[kFinBatch];
#pragma unroll
      for (int u = 0; u < kFinBatch; ++u) {
        const int64_t i = b + (int64_t)u * kFinSplit;
        v[u] = i < chunks ? part[i * K + j] : 0.0;
      }
#pragma unroll
      for (int u = 0; u < kFinBatch; ++u) {
        if (b + (int64_t)u * kFinSplit >= chunks) break;
        if (u % 2 == 0) s0 += v[u];
        else s1 += v[u];
      }
    }
  }
  red[q][c] = s0 + s1;
  __syncthreads();
#pragma unroll
  for (int w = kFinSplit / 2; w >= 1; w >>= 1) {
    if (q < w) red[q][c] += red[q + w][c];
    __syncthreads();
  }
  if (q == 0 && j < K) a[j] = (float)(red[0][c] / (double)T);
}

template <typename S>
hipError_t run(const void* X, int64_t T, int64_t K, float* a, void* ws, hipStream_t st) {
  constexpr int E = 16 / sizeof(S);
  constexpr int CB = kColThreads * E;
  int64_t chunks, rpc;
  chunking(T, K, &chunks, &rpc);
  const bool vec = (K % E == 0) && ((uintptr_t)X % 16 == 0);
  dim3 grid((unsigned)((K + CB - 1) / CB), (unsigned)chunks);
  double* part = static_cast<double*>(ws);
  {
    ProfScope p("awq_act_stats_partial", st);
    if (vec)
      act_stats_partial<S, true><<<grid, kThreads, 0, st>>>(static_cast<const S*>(X), T, K, rpc,
                                                            part);
    else
      act_stats_partial<S, false><<<grid, kThreads, 0, st>>>(static_cast<const S*>(X), T, K,
                                                             rpc, part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope p("awq_act_stats_finish", st);
    act_stats_finish<<<(unsigned)((K + kFinCols - 1) / kFinCols), kThreads, 0, st>>>(part, chunks, K,
                                                                                   T, a);
  }
  return hipGetLastError();
}

}  // namespace

size_t act_stats_ws_bytes(int64_t T, int64_t K) {
  int64_t chunks, rpc;
  chunking(T, K, &chunks, &rpc);
  return (size_t)chunks * (size_t)K * sizeof(double);
}

hipError_t launch_act_stats(const void* X, awq_dtype_t dt, int64_t T, int64_t K, float* a,
                            void* ws, hipStream_t st) {
  switch (dt) {
    case AWQ_F32: return run<float>(X, T, K, a, ws, st);
    case AWQ_F16: return run<_Float16>(X, T, K, a, ws, st);
    default: return run<__bf16>(X, T, K, a, ws, st);
  }
}

}  // namespace awq
