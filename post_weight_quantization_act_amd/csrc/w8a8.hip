// SmoothQuant: 8-bit weights and activations.
//
// "52 · AWQ, GPTQ và SmoothQuant", section 5: to run the layer's product in
// INT8, divide each activation channel by a factor and multiply the matching
// weights by it (the product is unchanged), with the factor balancing the two
// sides, s_j = sqrt(max|X_j| / max|W_j|); both sides then have moderate
// ranges and both are quantised to INT8.
//
// Kernels: the channel maxima of X and W (an atomic max on the fp32 bit
// patterns, which order like the values for non-negative numbers, so the
// result does not depend on scheduling); the scales; and a row quantiser
// (one workgroup per row: the row's maximum magnitude after smoothing, then
// symmetric 127-level codes) that writes either row-major codes or the tiled
// layout of the MFMA GEMM, byte pairs standing for its 2-byte elements.
// Arithmetic is IEEE fp32 with correctly rounded division and square root:
//   s_j = sqrt(ax_j / aw_j) (1 when either maximum is 0);
//   v = x / s_j (activations) or w * s_j (weights);
//   step = max|v| / 127 over the row (1 for an all-zero row);
//   q = clamp(rint(v / step), -127, 127).
#include "common.h"

namespace awq {
namespace {

constexpr int kRowThreads = 256;
constexpr int kColRows = 256;       // rows per workgroup of the channel-maximum pass
constexpr float kQMax = 127.0f;

__global__ void fill_zero_kernel(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// out[j] = max(out[j], max over this workgroup's rows of |A[r][j]|), as fp32 bits.
template <typename S>
__global__ __launch_bounds__(256) void colmax_kernel(const S* __restrict__ A, int64_t R, int64_t K,
                                                     uint32_t* __restrict__ out) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= K) return;
  const int64_t r0 = (int64_t)blockIdx.y * kColRows;
  const int64_t r1 = r0 + kColRows < R ? r0 + kColRows : R;
  float m = 0.0f;
  for (int64_t r = r0; r < r1; ++r) m = fmaxf(m, fabsf(to_f32(A[r * K + j])));
  atomicMax(out + j, __float_as_uint(m));
}

__global__ void smooth_scale_kernel(const float* __restrict__ ax, const float* __restrict__ aw,
                                    int64_t K, float* __restrict__ s) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= K) return;
  const float x = ax[j], w = aw[j];
  s[j] = (x > 0.0f && w > 0.0f) ? sqrtf(x / w) : 1.0f;
}

template <typename S>
__device__ __forceinline__ void load16(const S* p, float (&v)[16]) {
  if constexpr (sizeof(S) == 4) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 a = reinterpret_cast<const f32x4*>(p)[q];
      v[4 * q] = a.x;
      v[4 * q + 1] = a.y;
      v[4 * q + 2] = a.z;
      v[4 * q + 3] = a.w;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const i32x4 raw = reinterpret_cast<const i32x4*>(p)[q];
      const S* e = reinterpret_cast<const S*>(&raw);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[8 * q + i] = to_f32(e[i]);
    }
  }
}

// The smoothed values of 16 consecutive elements of a row.
template <typename S, bool kMul>
__device__ __forceinline__ void smoothed16(const S* row, const float* s, int64_t k0,
                                           float (&v)[16]) {
  load16(row + k0, v);
  if (s) {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = kMul ? v[i] * s[k0 + i] : v[i] / s[k0 + i];
  }
}

// One workgroup per row r < Rw.  Rows R <= r < Rw (padding of the tiled
// layout) get zero codes.  K is a multiple of 64.
template <typename S, bool kMul, bool kTiled>
__global__ __launch_bounds__(kRowThreads) void quant_rows_kernel(
    const S* __restrict__ A, int64_t R, int64_t K, const float* __restrict__ s,
    int8_t* __restrict__ q, float* __restrict__ step_out) {
  __shared__ float red[kRowThreads / 64];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t chunks = K / 16;
  auto dst = [&](int64_t c) -> i32x4* {
    if (kTiled) return reinterpret_cast<i32x4*>(q + 2 * tiled_index(r, 8 * c, K / 2));
    return reinterpret_cast<i32x4*>(q + r * K + 16 * c);
  };
  if (r >= R) {
    for (int64_t c = tid; c < chunks; c += kRowThreads) *dst(c) = i32x4{0, 0, 0, 0};
    return;
  }
  const S* row = A + r * K;
  float m = 0.0f;
  for (int64_t c = tid; c < chunks; c += kRowThreads) {
    float v[16];
    smoothed16<S, kMul>(row, s, 16 * c, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < kRowThreads / 64; ++w) m = fmaxf(m, red[w]);
  const float step = m > 0.0f ? m / kQMax : 1.0f;
  if (tid == 0) step_out[r] = step;
  for (int64_t c = tid; c < chunks; c += kRowThreads) {
    float v[16];
    smoothed16<S, kMul>(row, s, 16 * c, v);
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float cq = fminf(fmaxf(__builtin_rintf(v[i] / step), -kQMax), kQMax);
      w[i / 4] |= ((uint32_t)(int)cq & 0xffu) << (8 * (i % 4));
    }
    *dst(c) = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
  }
}

template <typename S>
hipError_t colmax(const void* A, int64_t R, int64_t K, uint32_t* out, hipStream_t st) {
  const dim3 grid((unsigned)((K + 255) / 256), (unsigned)((R + kColRows - 1) / kColRows));
  hipLaunchKernelGGL(colmax_kernel<S>, grid, dim3(256), 0, st, static_cast<const S*>(A), R, K,
                     out);
  return hipGetLastError();
}

template <typename S>
hipError_t quant_rows(const void* A, int64_t R, int64_t Rw, int64_t K, const float* s, bool mul,
                      bool tiled, int8_t* q, float* step, hipStream_t st) {
  const S* a = static_cast<const S*>(A);
  const dim3 grid((unsigned)Rw), block(kRowThreads);
  if (mul && tiled)
    hipLaunchKernelGGL((quant_rows_kernel<S, true, true>), grid, block, 0, st, a, R, K, s, q, step);
  else if (mul)
    hipLaunchKernelGGL((quant_rows_kernel<S, true, false>), grid, block, 0, st, a, R, K, s, q, step);
  else if (tiled)
    hipLaunchKernelGGL((quant_rows_kernel<S, false, true>), grid, block, 0, st, a, R, K, s, q, step);
  else
    hipLaunchKernelGGL((quant_rows_kernel<S, false, false>), grid, block, 0, st, a, R, K, s, q, step);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_smooth_scales(const void* X, const void* W, awq_dtype_t dt, int64_t T,
                                int64_t N, int64_t K, float* absmax, float* s, hipStream_t st) {
  ProfScope p("awq_smooth_scales", st);
  uint32_t* bits = reinterpret_cast<uint32_t*>(absmax);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((2 * K + 255) / 256)), dim3(256), 0, st,
                     bits, 2 * K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dt == AWQ_F16) {
    e = colmax<_Float16>(X, T, K, bits, st);
    if (e == hipSuccess) e = colmax<_Float16>(W, N, K, bits + K, st);
  } else if (dt == AWQ_BF16) {
    e = colmax<__bf16>(X, T, K, bits, st);
    if (e == hipSuccess) e = colmax<__bf16>(W, N, K, bits + K, st);
  } else {
    e = colmax<float>(X, T, K, bits, st);
    if (e == hipSuccess) e = colmax<float>(W, N, K, bits + K, st);
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(smooth_scale_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st,
                     absmax, absmax + K, K, s);
  return hipGetLastError();
}

hipError_t launch_quant_rows_int8(const void* A, awq_dtype_t dt, int64_t R, int64_t Rw,
                                  int64_t K, const float* s, bool multiply, bool tiled,
                                  int8_t* q, float* step, hipStream_t st) {
  ProfScope p("awq_quant_rows_int8", st);
  if (dt == AWQ_F16) return quant_rows<_Float16>(A, R, Rw, K, s, multiply, tiled, q, step, st);
  if (dt == AWQ_BF16) return quant_rows<__bf16>(A, R, Rw, K, s, multiply, tiled, q, step, st);
  return quant_rows<float>(A, R, Rw, K, s, multiply, tiled, q, step, st);
}

}  // namespace awq
