// Scale table, group-wise fake quantisation and final packing.
//
// AWQ Q&A page (aivaro.ru), sections 5 and 9: the scaled weights are
// quantised round-to-nearest per group, asymmetric (zero_point), group size
// q_group_size, w_bit bits.  AWQ reading notes, section "Measures": for each
// candidate exponent alpha the scales are s = a^alpha, the weights are scaled
// per input channel, quantised group-wise and dequantised, and the chosen
// scales' codes are saved with their per-group metadata.
//
// This file is compiled with -ffp-contract=off and -fno-honor-nans (inputs are
// finite; without NaNs min/max need no canonicalising moves and fuse with
// their DPP operands).  Every quantiser operation is
// a single IEEE fp32 operation with round-to-nearest-even (rint is
// v_rndne_f32, denormals are kept), in the order: w' = w*s; mx, mn over the
// group; delta = (mx - mn)/qmax floored at 1e-10; z = clamp(rint(-mn/delta));
// c = clamp(rint(w'/delta) + z); W_hat = ((c - z)*delta)/s.  So codes, steps
// and zero-points match any other IEEE evaluation of that order bit for bit.
//
// Every quotient is the correctly rounded one, computed from a reciprocal
// taken once and reused: with y = RN(1/b) (a correctly rounded division),
// q = RN(a*y) followed by two corrections q = fma(fma(-b, q, a), y, q) gives
// exactly RN(a/b) (Markstein's theorem: after the first correction q is
// within an ulp of a/b, so the residual a - b*q is exact and the second
// correction rounds correctly), in 5 VALU operations instead of the ~12 of
// the division sequence.  The theorem needs the intermediate values to stay
// normal; the quantiser's quotients by delta always do (delta >= 1e-10, and
// a tiny quotient only ever feeds rint), and for W_hat = deq/s a wave falls
// back to true divisions whenever one of its scales lies outside
// [2^-60, 2^60].
#include "common.h"

namespace awq {
namespace {

constexpr float kAMin = 1e-8f;
constexpr float kDeltaMin = 1e-10f;

// ---------------------------------------------------------------------------
// min / max across the `lanes` consecutive lanes that hold one group (a power
// of two; groups start at multiples of it; the branches are wave-uniform).
// The steps inside a 16-lane DPP row use quad permutes and the half-row / row
// mirrors; wider groups finish with cross-row swizzles.  Every lane ends with the group's
// min and max.
// ---------------------------------------------------------------------------
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, true));
}

__device__ __forceinline__ void group_minmax(float& mn, float& mx, int lanes) {
  if (lanes >= 2) {
    mn = fminf(mn, dpp<0xB1>(mn));   // quad_perm [1,0,3,2]
    mx = fmaxf(mx, dpp<0xB1>(mx));
  }
  if (lanes >= 4) {
    mn = fminf(mn, dpp<0x4E>(mn));   // quad_perm [2,3,0,1]
    mx = fmaxf(mx, dpp<0x4E>(mx));
  }
  if (lanes >= 8) {
    mn = fminf(mn, dpp<0x141>(mn));  // row_half_mirror
    mx = fmaxf(mx, dpp<0x141>(mx));
  }
  if (lanes >= 16) {
    mn = fminf(mn, dpp<0x140>(mn));  // row_mirror
    mx = fmaxf(mx, dpp<0x140>(mx));
  }
  if (lanes >= 32) {
    mn = fminf(mn, __shfl_xor(mn, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
  }
  if (lanes >= 64) {
    mn = fminf(mn, __shfl_xor(mn, 32));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
  }
}

// div_rn (common.h): RN(a/b) from y = RN(1/b), see the file header.

struct GroupQ {
  float delta, rdelta, z;   // step, RN(1 / step), zero-point
};

// qmax and rq = RN(1/qmax) are per-launch constants.
__device__ __forceinline__ GroupQ group_params(float mn, float mx, float qmax, float rq) {
  GroupQ g;
  g.delta = fmaxf(div_rn(mx - mn, qmax, rq), kDeltaMin);
  g.rdelta = 1.0f / g.delta;
  g.z = __builtin_amdgcn_fmed3f(__builtin_rintf(div_rn(-mn, g.delta, g.rdelta)), 0.0f, qmax);
  return g;
}

__device__ __forceinline__ float code_of(float wp, const GroupQ& g, float qmax) {
  return __builtin_amdgcn_fmed3f(__builtin_rintf(div_rn(wp, g.delta, g.rdelta)) + g.z, 0.0f, qmax);
}

// c - z for c = clamp(rint(q) + z, 0, qmax), formed as clamp(rint(q), -z, qmax - z).
// The two agree exactly: the integers involved are exact in fp32 unless
// |rint(q)| >= 2^24, and then both clamp to the same bound.
__device__ __forceinline__ float code_minus_z(float wp, const GroupQ& g, float qmax) {
  return __builtin_amdgcn_fmed3f(__builtin_rintf(div_rn(wp, g.delta, g.rdelta)), -g.z, qmax - g.z);
}

constexpr float kRecipSafeLo = 0x1p-60f, kRecipSafeHi = 0x1p60f;

template <typename S>
__device__ __forceinline__ void load8(const S* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <typename S>
__device__ __forceinline__ void load8(const S* p, float (&v)[8]) {
  i32x4 raw = *reinterpret_cast<const i32x4*>(p);
  const S* e = reinterpret_cast<const S*>(&raw);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = to_f32(e[i]);
}

template <typename S>
__device__ __forceinline__ void store8(S* p, const float (&v)[8]);
template <>
__device__ __forceinline__ void store8<float>(float* p, const float (&v)[8]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}
template <typename S>
__device__ __forceinline__ void store8(S* p, const float (&v)[8]) {
  i32x4 raw;
  S* e = reinterpret_cast<S*>(&raw);
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = from_f32<S>(v[i]);
  *reinterpret_cast<i32x4*>(p) = raw;
}

// ---------------------------------------------------------------------------
// s[k][j] = fp32(pow(fp64(max(a_j, 1e-8)), fp64(alpha_k))), and optionally
// rs[k][j] = RN(1 / s[k][j]) for the fake-quantisation kernel.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void scale_table_kernel(const float* __restrict__ a, int64_t K,
                                                          AlphaChunk al, float* __restrict__ s,
                                                          float* __restrict__ rs) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int k = blockIdx.y;
  if (j >= K || k >= al.n) return;
  const double x = (double)fmaxf(a[j], kAMin);
  const float v = (float)pow(x, (double)al.v[k]);
  s[(int64_t)k * K + j] = v;
  if (rs) rs[(int64_t)k * K + j] = 1.0f / v;
}

// ---------------------------------------------------------------------------
// Fake quantisation of W diag(s_k) for n_s scale vectors in one pass over W.
//
// A workgroup owns a tile of 32 rows x 512 columns.  Each wave covers one
// 512-column row segment per step (8 consecutive columns per lane, 16-byte
// loads), so the tile is read from HBM once into registers (8 rows x 8
// values per lane) and reused for every scale vector; only the 8 scales of
// the lane's columns are fetched per vector, with their reciprocals (read from
// rs when the caller has them, else computed) shared by the 8 rows.  A group of G channels lives in
// G/8 consecutive lanes and is reduced with DPP.  Output k is written to
// out + k*out_rows*K, row-major or in the GEMM's tiled layout (16-byte chunks
// land on their swizzled slot; padding rows up to a multiple of 256 get zeros).
// ---------------------------------------------------------------------------
constexpr int kFqThreads = 256;
constexpr int kFqCols = 512;                  // columns per workgroup (one wave-row)
constexpr int kFqRowSteps = 8;                // rows per wave
constexpr int kFqRows = kFqRowSteps * (kFqThreads / 64);

// kLanes = G/8 lanes per group, or 0 to take it from lanes_rt.
// kKeep: columns with keep[j] != 0 stay at full precision (output W, or 0 in
// the delta form) and take no part in their group's min / max.
template <typename S, typename O, bool kDelta, bool kTiled, int kLanes, bool kKeep = false>
__global__ __launch_bounds__(kFqThreads) void fake_quant_kernel(
    const S* __restrict__ W, int64_t N, int64_t K, const float* __restrict__ s,
    const float* __restrict__ rs, int n_s, float qmax, int lanes_rt, int64_t out_rows,
    O* __restrict__ out, const uint8_t* __restrict__ keep = nullptr) {
  const int lanes = kLanes ? kLanes : lanes_rt;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t col = (int64_t)blockIdx.x * kFqCols + lane * 8;
  const int64_t row0 = (int64_t)blockIdx.y * kFqRows + wave;
  const bool col_ok = col < K;

  float w[kFqRowSteps][8];
  bool row_ok[kFqRowSteps];
#pragma unroll
  for (int p = 0; p < kFqRowSteps; ++p) {
    const int64_t r = row0 + (int64_t)p * (kFqThreads / 64);
    row_ok[p] = r < N;
    if (col_ok && row_ok[p]) {
      load8(W + r * K + col, w[p]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) w[p][i] = 0.0f;
    }
  }

  bool kept[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) kept[i] = kKeep && col_ok && keep[col + i] != 0;

  const float rq = 1.0f / qmax;
  for (int k = 0; k < n_s; ++k) {
    float sv[8], ys[8];
    if (col_ok) {
      load8(s + (int64_t)k * K + col, sv);
      if (rs) load8(rs + (int64_t)k * K + col, ys);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) sv[i] = ys[i] = 1.0f;
    }
    bool extreme = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (!rs) ys[i] = 1.0f / sv[i];
      extreme |= !(fabsf(sv[i]) >= kRecipSafeLo && fabsf(sv[i]) <= kRecipSafeHi);
    }
    const bool exact_div = __builtin_amdgcn_ballot_w64(extreme) != 0;   // wave-uniform
    O* outk = out + (int64_t)k * out_rows * K;
#pragma unroll
    for (int p = 0; p < kFqRowSteps; ++p) {
      float wp[8];
      float mn, mx;
#pragma unroll
      for (int i = 0; i < 8; ++i) wp[i] = w[p][i] * sv[i];
      if (kKeep) {
        mn = kept[0] ? __builtin_inff() : wp[0];
        mx = kept[0] ? -__builtin_inff() : wp[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) {
          mn = fminf(mn, kept[i] ? __builtin_inff() : wp[i]);
          mx = fmaxf(mx, kept[i] ? -__builtin_inff() : wp[i]);
        }
      } else {
        mn = wp[0];
        mx = wp[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) {
          mn = fminf(mn, wp[i]);
          mx = fmaxf(mx, wp[i]);
        }
      }
      group_minmax(mn, mx, lanes);
      const GroupQ g = group_params(mn, mx, qmax, rq);
      float o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float deq = code_minus_z(wp[i], g, qmax) * g.delta;
        const float what = exact_div ? deq / sv[i] : div_rn(deq, sv[i], ys[i]);
        o[i] = kDelta ? (w[p][i] - what) : what;
        if (kKeep && kept[i]) o[i] = kDelta ? 0.0f : w[p][i];
      }
      const int64_t r = row0 + (int64_t)p * (kFqThreads / 64);
      if (kTiled) {
        // padding rows of the tiled layout are written as zeros
        if (col_ok && r < out_rows) {
          if (!row_ok[p]) {
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = 0.0f;
          }
          store8(outk + tiled_index(r, col, K), o);
        }
      } else if (col_ok && row_ok[p]) {
        store8(outk + r * K + col, o);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Final quantisation + packing for one scale vector.
//
// One lane owns 32 consecutive columns of kPackRows rows: it loads the 32
// scales once, then per row loads the 32 weights, reduces its share of the
// group (G/32 lanes per group, DPP), computes the 32 codes and writes them as
// `bits` uint32 words -- exactly its slice of the row's little-endian
// bitstream (32 codes x bits bits).  The first lane of each group writes the
// group's step and zero-point.  Consecutive lanes own consecutive column
// chunks (a group never straddles a wave: K/32 is a multiple of G/32).
// ---------------------------------------------------------------------------
constexpr int kPackRows = 4;

template <typename S, int BITS>
__global__ __launch_bounds__(256) void quantize_pack_kernel(
    const S* __restrict__ W, int64_t N, int64_t K, const float* __restrict__ s, int group,
    int lanes, uint32_t* __restrict__ codes, float* __restrict__ scales,
    uint8_t* __restrict__ zeros) {
  const int64_t chunks_per_row = K / 32;
  const int64_t row_blocks = (N + kPackRows - 1) / kPackRows;
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool ok = q < row_blocks * chunks_per_row;
  const int64_t rb = ok ? q / chunks_per_row : 0;
  const int64_t cc = ok ? q % chunks_per_row : 0;
  const int64_t col0 = cc * 32;
  const float qmax = (float)((1 << BITS) - 1);
  const float rq = 1.0f / qmax;

  float sv[32];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    float v[8];
    if (ok) {
      load8(s + col0 + h * 8, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 1.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) sv[h * 8 + i] = v[i];
  }

  for (int r = 0; r < kPackRows; ++r) {
    const int64_t row = rb * kPackRows + r;
    const bool row_ok = ok && row < N;      // uniform across a group's lanes
    float wp[32];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float v[8];
      if (row_ok) {
        load8(W + row * K + col0 + h * 8, v);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) wp[h * 8 + i] = v[i] * sv[h * 8 + i];
    }
    float mn = wp[0], mx = wp[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) {
      mn = fminf(mn, wp[i]);
      mx = fmaxf(mx, wp[i]);
    }
    group_minmax(mn, mx, lanes);
    const GroupQ g = group_params(mn, mx, qmax, rq);

    // 32 codes of `bits` bits -> `bits` words; bit p of the slice is bit
    // p%32 of word p/32.
    uint32_t words[BITS];
#pragma unroll
    for (int i = 0; i < BITS; ++i) words[i] = 0u;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint32_t c = (uint32_t)code_of(wp[j], g, qmax);
      const int p = BITS * j;               // compile-time after unrolling
      const int wi = p >> 5, sh = p & 31;
      words[wi] |= c << sh;
      if (sh + BITS > 32) words[wi + 1] |= c >> (32 - sh);   // BITS <= 8: two words at most
    }
    if (row_ok) {
      uint32_t* dst = codes + row * (chunks_per_row * BITS) + cc * BITS;
#pragma unroll
      for (int t = 0; t < BITS; ++t) dst[t] = words[t];
      if ((cc % lanes) == 0) {
        const int64_t gi = row * (K / group) + col0 / group;
        scales[gi] = g.delta;
        zeros[gi] = (uint8_t)g.z;
      }
    }
  }
}

template <typename S, typename O, bool kDelta>
hipError_t fq_dispatch(const void* W, int64_t N, int64_t K, const float* s, const float* rs,
                       int n_s, int bits, int group, bool tiled, const uint8_t* keep, void* out,
                       hipStream_t st) {
  const int64_t out_rows = tiled ? padded_rows(N) : N;
  dim3 grid((unsigned)((K + kFqCols - 1) / kFqCols), (unsigned)((out_rows + kFqRows - 1) / kFqRows));
  const float qmax = (float)((1 << bits) - 1);
  const S* w = static_cast<const S*>(W);
  O* o = static_cast<O*>(out);
  const int lanes = group / 8;
  ProfScope p("awq_fake_quant", st);
  if (!tiled) {
    if (keep) return hipErrorInvalidValue;
    fake_quant_kernel<S, O, kDelta, false, 0><<<grid, kFqThreads, 0, st>>>(w, N, K, s, rs, n_s,
                                                                           qmax, lanes, out_rows, o);
    return hipGetLastError();
  }
  // the search's launch: the group width is a compile-time constant
#define AWQ_FQ_TILED(L)                                                                          \
  if (keep)                                                                                      \
    fake_quant_kernel<S, O, kDelta, true, L, true><<<grid, kFqThreads, 0, st>>>(                  \
        w, N, K, s, rs, n_s, qmax, L, out_rows, o, keep);                                         \
  else                                                                                           \
    fake_quant_kernel<S, O, kDelta, true, L><<<grid, kFqThreads, 0, st>>>(w, N, K, s, rs, n_s,    \
                                                                          qmax, L, out_rows, o)
  switch (lanes) {
    case 4: AWQ_FQ_TILED(4); break;
    case 8: AWQ_FQ_TILED(8); break;
    case 16: AWQ_FQ_TILED(16); break;
    case 32: AWQ_FQ_TILED(32); break;
    default: AWQ_FQ_TILED(64); break;
  }
#undef AWQ_FQ_TILED
  return hipGetLastError();
}

template <typename S>
hipError_t pack_dispatch(const void* W, int64_t N, int64_t K, const float* s, int bits, int group,
                         uint32_t* codes, float* scales, uint8_t* zeros, hipStream_t st) {
  const int64_t threads = (N + kPackRows - 1) / kPackRows * (K / 32);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  const S* w = static_cast<const S*>(W);
  ProfScope p("awq_quantize_pack", st);
  const int lanes = group / 32;
  switch (bits) {
    case 2: quantize_pack_kernel<S, 2><<<blocks, 256, 0, st>>>(w, N, K, s, group, lanes, codes, scales, zeros); break;
    case 3: quantize_pack_kernel<S, 3><<<blocks, 256, 0, st>>>(w, N, K, s, group, lanes, codes, scales, zeros); break;
    case 4: quantize_pack_kernel<S, 4><<<blocks, 256, 0, st>>>(w, N, K, s, group, lanes, codes, scales, zeros); break;
    case 5: quantize_pack_kernel<S, 5><<<blocks, 256, 0, st>>>(w, N, K, s, group, lanes, codes, scales, zeros); break;
    case 6: quantize_pack_kernel<S, 6><<<blocks, 256, 0, st>>>(w, N, K, s, group, lanes, codes, scales, zeros); break;
    case 7: quantize_pack_kernel<S, 7><<<blocks, 256, 0, st>>>(w, N, K, s, group, lanes, codes, scales, zeros); break;
    default: quantize_pack_kernel<S, 8><<<blocks, 256, 0, st>>>(w, N, K, s, group, lanes, codes, scales, zeros); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scale_table(const float* a, int64_t K, const AlphaChunk& al, float* s_out,
                              float* rs_out, hipStream_t st) {
  ProfScope p("awq_scale_table", st);
  scale_table_kernel<<<dim3((unsigned)((K + 255) / 256), (unsigned)al.n), 256, 0, st>>>(a, K, al, s_out,
                                                                                     rs_out);
  return hipGetLastError();
}

hipError_t launch_fake_quant(const void* W, awq_dtype_t dt, int64_t N, int64_t K, const float* s,
                             const float* rs, int n_s, int bits, int group, bool delta_form,
                             bool tiled, void* out, hipStream_t st, const uint8_t* keep) {
  switch (dt) {
    case AWQ_F32:
      if (tiled || keep) return hipErrorInvalidValue;
      return delta_form
                 ? fq_dispatch<float, float, true>(W, N, K, s, rs, n_s, bits, group, false, nullptr, out, st)
                 : fq_dispatch<float, float, false>(W, N, K, s, rs, n_s, bits, group, false, nullptr, out, st);
    case AWQ_F16:
      return delta_form
                 ? fq_dispatch<_Float16, _Float16, true>(W, N, K, s, rs, n_s, bits, group, tiled, keep, out, st)
                 : fq_dispatch<_Float16, _Float16, false>(W, N, K, s, rs, n_s, bits, group, tiled, keep, out, st);
    default:
      return delta_form
                 ? fq_dispatch<__bf16, __bf16, true>(W, N, K, s, rs, n_s, bits, group, tiled, keep, out, st)
                 : fq_dispatch<__bf16, __bf16, false>(W, N, K, s, rs, n_s, bits, group, tiled, keep, out, st);
  }
}

// keep[j] = 1 for the n_keep channels with the largest score (ties: lower index).
__global__ __launch_bounds__(256) void keep_mask_kernel(const float* __restrict__ score, int64_t K,
                                                        int64_t n_keep, uint8_t* __restrict__ keep) {
  __shared__ float tile[1024];
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const float sj = j < K ? score[j] : 0.0f;
  int64_t rank = 0;                       // channels ranked before j
  for (int64_t base = 0; base < K; base += 1024) {
    const int64_t n = K - base < 1024 ? K - base : 1024;
    __syncthreads();
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) tile[i] = score[base + i];
    __syncthreads();
    for (int64_t i = 0; i < n; ++i) {
      const float si = tile[i];
      rank += (si > sj || (si == sj && base + i < j)) ? 1 : 0;
    }
  }
  if (j < K) keep[j] = rank < n_keep ? 1 : 0;
}

hipError_t launch_keep_mask(const float* score, int64_t K, int64_t n_keep, uint8_t* keep,
                            hipStream_t st) {
  ProfScope p("awq_keep_mask", st);
  keep_mask_kernel<<<(unsigned)((K + 255) / 256), 256, 0, st>>>(score, K, n_keep, keep);
  return hipGetLastError();
}

hipError_t launch_quantize_pack(const void* W, awq_dtype_t dt, int64_t N, int64_t K,
                                const float* s, int bits, int group, uint32_t* codes,
                                float* scales, uint8_t* zeros, hipStream_t st) {
  switch (dt) {
    case AWQ_F32: return pack_dispatch<float>(W, N, K, s, bits, group, codes, scales, zeros, st);
    case AWQ_F16: return pack_dispatch<_Float16>(W, N, K, s, bits, group, codes, scales, zeros, st);
    default: return pack_dispatch<__bf16>(W, N, K, s, bits, group, codes, scales, zeros, st);
  }
}

}  // namespace awq
