// Internal declarations shared by the HIP translation units of the AWQ
// scale-search library (gfx950 only).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/awq.h"

namespace awq {

// ---- vector types -----------------------------------------------------------
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

// Element tags: storage type of W / X / W_hat.
struct F32T { typedef float storage; static constexpr int size = 4; };
struct F16T { typedef _Float16 storage; static constexpr int size = 2; };
struct BF16T { typedef __bf16 storage; static constexpr int size = 2; };
// Two int8 values stored as one 2-byte element of the tiled layout.
struct I8Pair {
  int8_t lo, hi;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(_Float16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

// Round-to-nearest-even conversions out of fp32.
template <typename S> __device__ __forceinline__ S from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float x) { return (_Float16)x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// RN(a/b) from y = RN(1/b) in 5 fp32 operations (Markstein: after the first
// correction q is within an ulp of a/b, so the residual a - b q is exact and
// the second correction rounds correctly).  Needs the intermediate values
// normal, which holds for the quantiser's quotients (b = delta >= 1e-10, and
// a quotient small enough to be at risk only ever feeds rint).  Callers must
// be compiled without contraction so that a * y is one rounding.
__device__ __forceinline__ float div_rn(float a, float b, float y) {
  float q = a * y;
  float r = fmaf(-b, q, a);
  q = fmaf(r, y, q);
  r = fmaf(-b, q, a);
  return fmaf(r, y, q);
}

// ---- tiled operand layout of the MFMA GEMM --------------------------------------
// fp16/bf16 GEMM operands are stored tile by tile so that every global -> LDS
// transfer of the GEMM is a contiguous 1 KB block holding whole 128-byte lines:
// rows are padded to a multiple of 256 (padding rows are zero) and K is split in
// stages of 32 elements.  Block (tile t, stage s) is 256 rows x 64 bytes at byte
// ((t * (K / 32)) + s) * 16384; row r of the block occupies bytes [64 r, 64 r + 64)
// and its 16-byte chunk c (k = 32 s + 8 c .. 32 s + 8 c + 7) sits at chunk
// c ^ ((r >> 1) & 3), the LDS swizzle the GEMM's fragment reads expect.
constexpr int kTileRows = 256;
constexpr int kStageK = 32;
constexpr int kBlockBytes = kTileRows * kStageK * 2;

__host__ __device__ constexpr int64_t padded_rows(int64_t rows) {
  return (rows + kTileRows - 1) / kTileRows * kTileRows;
}
__host__ __device__ __forceinline__ int swizzle_chunk(int r, int c) { return c ^ ((r >> 1) & 3); }
// Element offset of (row, k) in the tiled layout of a [rows, K] matrix (2-byte elements).
__host__ __device__ __forceinline__ int64_t tiled_index(int64_t row, int64_t k, int64_t K) {
  const int64_t t = row / kTileRows, r = row % kTileRows, s = k / kStageK;
  const int c = (int)((k % kStageK) / 8);
  return ((t * (K / kStageK) + s) * kTileRows + r) * kStageK + 8 * swizzle_chunk((int)r, c) + k % 8;
}

// ---- launch plumbing ----------------------------------------------------------
// Optional per-launch event timing (see awq_profile_* in the public header).
// prof_begin returns a token (or -1 when profiling is off) to hand to prof_end.
int prof_begin(const char* kernel, hipStream_t stream);
void prof_end(int token, hipStream_t stream);

struct ProfScope {
  int tok;
  hipStream_t st;
  ProfScope(const char* name, hipStream_t s) : tok(prof_begin(name, s)), st(s) {}
  ~ProfScope() { prof_end(tok, st); }
};

// ---- launchers (each returns hipSuccess or the launch error) ---------------------
// act_stats.hip
size_t act_stats_ws_bytes(int64_t T, int64_t K);
hipError_t launch_act_stats(const void* X, awq_dtype_t dt, int64_t T, int64_t K, float* a,
                            void* ws, hipStream_t st);

// quant.hip
struct AlphaChunk {
  int n;
  float v[64];
};
// s_out [al.n, K]; rs_out (may be null) [al.n, K] = RN(1 / s).
hipError_t launch_scale_table(const float* a, int64_t K, const AlphaChunk& al, float* s_out,
                              float* rs_out, hipStream_t st);
// s [n_s, K]; rs (may be null) its elementwise RN(1 / s).  out: n_s consecutive
// [N, K] row-major matrices, or (tiled = true, fp16/bf16 only) n_s consecutive
// tiled [padded_rows(N), K] matrices with zero padding rows.
// keep (tiled only, may be null): columns with keep[j] != 0 stay at full
// precision and are left out of their group's range.
hipError_t launch_fake_quant(const void* W, awq_dtype_t dt, int64_t N, int64_t K,
                             const float* s, const float* rs, int n_s, int bits, int group,
                             bool delta_form, bool tiled, void* out, hipStream_t st,
                             const uint8_t* keep = nullptr);
// keep[j] = 1 for the n_keep largest scores (ties: lower index first), else 0.
hipError_t launch_keep_mask(const float* score, int64_t K, int64_t n_keep, uint8_t* keep,
                            hipStream_t st);
// Copy a row-major [R, K] fp16/bf16 matrix into the tiled layout (zero padding rows).
hipError_t launch_tile_rows(const void* src, int64_t R, int64_t K, void* dst, hipStream_t st);
hipError_t launch_quantize_pack(const void* W, awq_dtype_t dt, int64_t N, int64_t K,
                                const float* s, int bits, int group, uint32_t* codes,
                                float* scales, uint8_t* zeros, hipStream_t st);

// lowbit.hip: the low-bit layer on repacked codes (layout in lowbit.hip)
hipError_t launch_lowbit_repack(const uint32_t* codes, const float* scales, const uint8_t* zeros,
                                int64_t N, int64_t K, int bits, int group, uint32_t* codes_t,
                                void* meta_t, hipStream_t st);
size_t lowbit_gemv_ws_bytes(awq_dtype_t dt, int64_t M, int64_t N, int64_t K);
hipError_t launch_lowbit_gemv(const void* X, awq_dtype_t dt, int64_t M, int64_t K,
                              const uint32_t* codes_t, const void* meta_t, int64_t N, int bits,
                              int group, float* Y, void* ws, hipStream_t st);
// Device address of this GPU's static scratch array for the allocation-free
// GEMV (AWQ_LOWBIT_STATIC_SCRATCH_BYTES), looked up on the first call per device.
hipError_t lowbit_static_scratch(void** out);
// fp16/bf16 activations only; K a multiple of the group, group >= 32.
hipError_t launch_lowbit_gemm(const void* X, awq_dtype_t dt, int64_t M, int64_t K,
                              const uint32_t* codes_t, const void* meta_t, int64_t N, int bits,
                              int group, float* Y, hipStream_t st);

// gptq.hip: GPTQ error feedback after the scaling (all fp64 but the quantiser)
struct GptqLayout {
  int64_t Kp;          // K rounded up to 128: leading dimension of the factor matrix
  int chunk_rows;      // calibration rows per Hessian chunk (a multiple of 16)
  size_t h_off;        // fp64 [Kp][Kp]: reversed H -> L -> L^-1 -> U (upper triangle)
  size_t xc_off;       // fp64 [chunk_rows][Kp]: one chunk of reversed X diag(s)^-1
  size_t wc_off;       // fp64 [N][K]: current scaled weights
  size_t err_off;      // fp64 [N][512]: one super-block's scaled errors
  size_t codes_off;    // uint8 [N][K]: codes before packing
  size_t dead_off;     // uint8 [K]: channels no calibration input reaches
  size_t bytes;
};
GptqLayout gptq_layout(int64_t N, int64_t K, int64_t T);
hipError_t launch_gptq(const void* W, const void* X, awq_dtype_t dt, int64_t N, int64_t K,
                       int64_t T, const float* s, int bits, int group, double damp,
                       uint32_t* codes, float* scales, uint8_t* zeros, void* ws, hipStream_t st);

// w8a8.hip: SmoothQuant scales and the INT8 row quantiser
// absmax [2K]: max|X_j| then max|W_j| (fp32); s [K] = sqrt(max|X_j| / max|W_j|).
hipError_t launch_smooth_scales(const void* X, const void* W, awq_dtype_t dt, int64_t T,
                                int64_t N, int64_t K, float* absmax, float* s, hipStream_t st);
// Rows r < R of A [R, K] (K a multiple of 64): smoothed by s (multiplied or
// divided; s may be null), symmetric 127-level codes and steps.  tiled: codes
// in the tiled layout of the MFMA GEMM with Rw (padded) rows, the padding rows
// zero; else row-major [R, K] (Rw = R).
hipError_t launch_quant_rows_int8(const void* A, awq_dtype_t dt, int64_t R, int64_t Rw,
                                  int64_t K, const float* s, bool multiply, bool tiled,
                                  int8_t* q, float* step, hipStream_t st);

// gemm_sse.hip
// GEMM epilogues.  kStore writes y row-major [T][N].  kRefOut writes the
// reference output that a later kSseRef launch reads: on the fp16/bf16/int8
// matrix-core path in the accumulator-fragment layout (frag_index below), on
// the fp32 path row-major.  kSseRef sums (Y_ref - y)^2, kSseDelta sums y^2.
enum class Epi { kStore = 0, kSseRef = 1, kSseDelta = 2, kRefOut = 3 };
// Fragment layout of a matrix-core GEMM's fp32 output: the 256 x 256 tile
// (tm, tn) is 64 K floats at float offset (tm * tiles_n + tn) * 65536; inside
// it wave w (8 waves, 2 x 4 over 128 x 64 blocks), 16 x 16 block (i, j)
// (8 x 4 per wave) and lane l hold the float4 at float4 offset
// (w * 32 + i * 4 + j) * 64 + l, whose component r is output
// (tm * 256 + (w / 4) * 128 + i * 16 + (l / 16) * 4 + r,
//  tn * 256 + (w % 4) * 64 + j * 16 + l % 16).
// A wave's 16-byte pieces of one block are 1 KB contiguous.  Outputs past T or
// N are written (as the product of the zero padding) and never read back.
struct GemmTiles {
  int tile_m, tile_n;
};
GemmTiles gemm_tiles(awq_dtype_t dt);
// Workgroups of a persistent fp16/bf16 GEMM launch on the current device (its
// compute units rounded down to a multiple of 8); a launch of more tiles
// runs them in rounds of this many.
int gemm_grid();
// C[t, n] = sum_k X[t, k] * B_b[n, k] over nb weight matrices.
//   fp16/bf16: X is tiled (padded_rows(T) rows); B is tiled with nb matrices of
//   padded_rows(N) rows each (b_tiled = true) or row-major [N, K] (b_tiled =
//   false, nb = 1).  fp32: both row-major, B_b = B + b*N*K.
//   kStore:    Y[t, n] = C (nb must be 1)
//   kSseRef:   partials[(a0 + b)][tm][tn] = sum over the tile of (Y - C)^2
//   kSseDelta: partials[(a0 + b)][tm][tn] = sum over the tile of C^2
// An fp16/bf16 launch may run part of the batch: logical tiles [tile0,
// tile0 + ntiles) of its nb * tiles_m * tiles_n, numbered candidate by
// candidate and, within a candidate, in the raster order of groups of 8 token
// tiles (ntiles < 0: every tile from tile0 on).  fp32 launches run the whole
// batch.
hipError_t launch_gemm(Epi epi, awq_dtype_t dt, const void* X, const void* B, bool b_tiled,
                       int nb, int64_t T, int64_t N, int64_t K, float* Y, double* partials,
                       int a0, hipStream_t st, int tile0 = 0, int ntiles = -1);
// INT8 GEMM on tiled operands (Xq [padded T][K], Wq [padded N][K] int8, K a
// multiple of 64, in the tiled layout of the 2-byte case with byte pairs as
// elements): kStore writes Y = fp32(fp32(fp32(acc) sx[t]) sw[n]); kSseRef
// writes per-tile sums of (Y_ref - that)^2 to partials (Y holds Y_ref).
hipError_t launch_gemm_w8a8(Epi epi, const void* Xq, const void* Wq, int64_t T, int64_t N,
                            int64_t K, const float* sx, const float* sw, float* Y,
                            double* partials, hipStream_t st);
hipError_t launch_loss_argmin(const double* partials, int n_alpha, int64_t tiles_per_alpha,
                              double inv_count, const float* s_table, int64_t K,
                              double* losses, int32_t* best, float* s_best, hipStream_t st);

}  // namespace awq
