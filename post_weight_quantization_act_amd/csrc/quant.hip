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

// ---------------------------------------------------------------------------
// Rounding decision of the code without the exact quotient.
//
// The oracle's code is c = clamp(rint(RN(w'/delta)) + z, 0, qmax).  With
// y = RN(1/delta) (a correctly rounded division, once per group) the kernel
// forms t = RN(w' * y + z) (one fma).  Let Q = w'/delta and V = RN(Q) + z.
// Then |t - V| <= 2^-24 (3 |Q| + z) + 2^-149: y and the fma each round once
// (relative 2^-24) and RN(Q) is within 2^-24 |Q| of Q.  If t lies farther than
// that from every half-integer, V rounds to the same integer as t and is no
// tie, so rint(t) = rint(RN(Q)) + z exactly (z is an integer) and
// c = clamp(rint(t), 0, qmax).  The group-wide bound uses M = max(-mn, mx)
// >= |w'|:
//   lim = 1/2 - (M y 2^-21 + (z + 1) 2^-23)
// 2^-21 covers 3 * 2^-24 |Q| with room for the roundings of the bound itself,
// and (z + 1) 2^-23 covers 2^-24 z plus the rounding of lim (at most 2^-25)
// and the underflow term.  A code is safe when |t - rint(t)| < lim (t - rint(t)
// is exact); otherwise, or when lim <= 0, the wave recomputes the row's
// quotients exactly.  Clamping t to [-1/4, qmax + 1/4] before the test leaves
// it valid: a t beyond those bounds gets code 0 or qmax whichever way its
// exact value rounds, and the clamped t is 1/4 from its rounding.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float safe_limit(float mn, float mx, float y, float z) {
  const float m = fmaxf(-mn, mx);
  return 0.5f - (m * y * 0x1p-21f + (z + 1.0f) * 0x1p-23f);
}

constexpr float kRecipSafeLo = 0x1p-60f, kRecipSafeHi = 0x1p60f;

// ---------------------------------------------------------------------------
// Group parameters of four rows at once, for groups of 16 lanes (one DPP row).
//
// Every lane of a group needs the same step, reciprocal, zero-point and safety
// bound, so forming them in all 16 lanes repeats the same work 16 times.
// Instead the lanes' partial min / max of four rows are reduced so that each
// quad of the group ends with one row's group-wide values (a reduce-scatter),
// each lane forms the parameters of that one row, and they are broadcast back
// per row with ds_swizzle (LDS crossbar, no vector-ALU issue).
//   step 1: row_mirror pairs lane j with 15 - j (opposite bit 3); a lane with
//           bit 3 clear keeps rows 0, 1 and sends rows 2, 3, the other way round
//           for its partner;
//   step 2: row_half_mirror pairs j with the lane of opposite bit 2 in its half
//           row; bit 2 clear keeps the lower of its two rows;
//   steps 3, 4: the four lanes of a quad hold the same row and all-reduce.
// Lane j then holds row (j >> 2) & 3 reduced over all 16 lanes (the four
// lanes of quad q cover {q', 7 - q', 8 + q', 15 - q'} for its four q', whose
// union is the whole row).  min / max are exact, so the result does not depend
// on the order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void minmax_scatter4(const float (&mn)[4], const float (&mx)[4],
                                                int lane, float& omn, float& omx) {
  const bool b3 = (lane & 8) != 0, b2 = (lane & 4) != 0;
  float kn[2], kx[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float keep_n = b3 ? mn[2 + i] : mn[i], send_n = b3 ? mn[i] : mn[2 + i];
    const float keep_x = b3 ? mx[2 + i] : mx[i], send_x = b3 ? mx[i] : mx[2 + i];
    kn[i] = fminf(keep_n, dpp<0x140>(send_n));   // row_mirror
    kx[i] = fmaxf(keep_x, dpp<0x140>(send_x));
  }
  const float keep_n = b2 ? kn[1] : kn[0], send_n = b2 ? kn[0] : kn[1];
  const float keep_x = b2 ? kx[1] : kx[0], send_x = b2 ? kx[0] : kx[1];
  omn = fminf(keep_n, dpp<0x141>(send_n));       // row_half_mirror
  omx = fmaxf(keep_x, dpp<0x141>(send_x));
  omn = fminf(omn, dpp<0x4E>(omn));              // quad_perm [2,3,0,1]
  omx = fmaxf(omx, dpp<0x4E>(omx));
  omn = fminf(omn, dpp<0xB1>(omn));              // quad_perm [1,0,3,2]
  omx = fmaxf(omx, dpp<0xB1>(omx));
}

// The same reduce-scatter for groups of 8 lanes (half a DPP row): the half-row
// mirror pairs lane j with 7 - j (opposite bit 2), the quad permute [2,3,0,1]
// pairs lanes of opposite bit 1, and [1,0,3,2] finishes; lane j then holds
// row (j >> 1) & 3 reduced over its 8 lanes ({j', 7 - j', j' ^ 2, 7 - (j' ^ 2)}
// for both lanes j' of the pair cover all 8).
__device__ __forceinline__ void minmax_scatter4_8(const float (&mn)[4], const float (&mx)[4],
                                                  int lane, float& omn, float& omx) {
  const bool b2 = (lane & 4) != 0, b1 = (lane & 2) != 0;
  float kn[2], kx[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float keep_n = b2 ? mn[2 + i] : mn[i], send_n = b2 ? mn[i] : mn[2 + i];
    const float keep_x = b2 ? mx[2 + i] : mx[i], send_x = b2 ? mx[i] : mx[2 + i];
    kn[i] = fminf(keep_n, dpp<0x141>(send_n));   // row_half_mirror
    kx[i] = fmaxf(keep_x, dpp<0x141>(send_x));
  }
  const float keep_n = b1 ? kn[1] : kn[0], send_n = b1 ? kn[0] : kn[1];
  const float keep_x = b1 ? kx[1] : kx[0], send_x = b1 ? kx[0] : kx[1];
  omn = fminf(keep_n, dpp<0x4E>(send_n));        // quad_perm [2,3,0,1]
  omx = fmaxf(keep_x, dpp<0x4E>(send_x));
  omn = fminf(omn, dpp<0xB1>(omn));              // quad_perm [1,0,3,2]
  omx = fmaxf(omx, dpp<0xB1>(omx));
}

// Value of lane 2 p of the lane's 8-lane group (source lane (lane & 0x18) | 2 p).
template <int P>
__device__ __forceinline__ float from_pair(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), ((2 * P) << 5) | 0x18));
}

// Value of lane 4 p of the lane's 16-lane group (ds_swizzle bitmask mode within
// 32 lanes: source lane = (lane & 0x10) | 4 p).
template <int P>
__device__ __forceinline__ float from_quad(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), ((4 * P) << 5) | 0x10));
}

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
  for (int i = 0; i < 8; ++i) {
    // The value is rounded to fp32 first and then converted.  The empty asm
    // keeps the compiler from folding the conversion into the fma that
    // produced the value: its mixed-precision fma with an fp16 result does not
    // round as the two steps do (it resolved fp16 ties differently).
    float x = v[i];
    asm("" : "+v"(x));
    e[i] = from_f32<S>(x);
  }
  *reinterpret_cast<i32x4*>(p) = raw;
}

// 8 consecutive elements of a row in their storage type (16 bytes; 32 for fp32).
template <typename S>
struct WRow {
  i32x4 v[sizeof(S) / 2];
};
template <typename S>
__device__ __forceinline__ WRow<S> load_wrow(const S* p) {
  WRow<S> r;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(S) / 2); ++i) r.v[i] = reinterpret_cast<const i32x4*>(p)[i];
  return r;
}
template <typename S>
__device__ __forceinline__ void widen_wrow(const WRow<S>& r, float (&v)[8]) {
  const S* e = reinterpret_cast<const S*>(&r.v[0]);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = to_f32(e[i]);
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
// G/8 consecutive lanes and is reduced with DPP; for G = 128 (16 lanes) the
// rows are taken four at a time and each row's group parameters are formed
// once per group (minmax_scatter4) instead of in all 16 lanes.  Output k is written to
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
template <typename S, typename O, bool kDelta, bool kTiled, int kLanes, bool kKeep = false,
          bool kRs = true>
__global__ __launch_bounds__(kFqThreads) void fake_quant_kernel(
    const S* __restrict__ W, int64_t N, int64_t K, const float* __restrict__ s,
    const float* __restrict__ rs, int n_s, float qmax, int lanes_rt, int64_t out_rows,
    O* __restrict__ out, const uint8_t* __restrict__ keep = nullptr) {
  const int lanes = kLanes ? kLanes : lanes_rt;
  // groups of 16 lanes (G = 128) form their parameters once per row and group
  constexpr bool kShare = kLanes == 16 && !kKeep;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t col = (int64_t)blockIdx.x * kFqCols + lane * 8;
  const int64_t row0 = (int64_t)blockIdx.y * kFqRows + wave;
  const bool col_ok = col < K;

  // The tile stays in registers in its storage type (8 16-bit values in four
  // registers per row), widened to fp32 per scale vector: half the registers
  // of an fp32 copy, for one shift or conversion per element (two on the
  // shared-parameter path, which widens again where a row is finished).
  WRow<S> wraw[kFqRowSteps];
  bool row_ok[kFqRowSteps];
#pragma unroll
  for (int p = 0; p < kFqRowSteps; ++p) {
    const int64_t r = row0 + (int64_t)p * (kFqThreads / 64);
    row_ok[p] = r < N;
    if (col_ok && row_ok[p]) {
      wraw[p] = load_wrow(W + r * K + col);
    } else {
#pragma unroll
      for (int i = 0; i < (int)(sizeof(S) / 2); ++i) wraw[p].v[i] = i32x4{0, 0, 0, 0};
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
      if (kRs) load8(rs + (int64_t)k * K + col, ys);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) sv[i] = ys[i] = 1.0f;
    }
    bool extreme = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (!kRs) ys[i] = 1.0f / sv[i];
      // kept in a register: left alone the compiler may recompute the
      // division in every row rather than hold the eight reciprocals
      asm("" : "+v"(ys[i]));
      extreme |= !(fabsf(sv[i]) >= kRecipSafeLo && fabsf(sv[i]) <= kRecipSafeHi);
    }
    const bool exact_div = __builtin_amdgcn_ballot_w64(extreme) != 0;   // wave-uniform
    O* outk = out + (int64_t)k * out_rows * K;

    // Codes, dequantisation, division by s and the store of row step p, given
    // the row's group step, its reciprocal, the clamp bounds lo = -z - 1/4 and
    // hi = qmax - z + 1/4 and the safety bound lim.
    // c - z for c = clamp(rint(w' / delta) + z, 0, qmax) is formed as
    // clamp(rint(w' / delta), -z, qmax - z): the two agree exactly, as the
    // integers involved are exact in fp32 unless |rint| >= 2^24, and then both
    // clamp to the same bound.  It is decided from t = RN(w' y)
    // (the bound of safe_limit holds with z = 0 in the fma, so it holds here);
    // t is clamped to [lo, hi] and rounded to the nearest integer, ties to
    // even (v_rndne); t - rint(t) is exact (the two lie within a factor 2 of
    // each other unless rint(t) = 0).  A risky lane sends the wave to the exact
    // quotients.  z = -lo - 1/4 exactly (z <= 255).
    auto finish_row = [&](int p, const float (&wp)[8], float delta, float rdelta, float lo,
                          float hi, float lim) {
      // an opaque copy, so that the compiler widens again here instead of
      // keeping the first widening live
      WRow<S> raw = wraw[p];
#pragma unroll
      for (int i = 0; i < (int)(sizeof(S) / 2); ++i) asm("" : "+v"(raw.v[i]));
      float w[8];
      widen_wrow(raw, w);
      float cmz[8];
      bool risky = false;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float t = __builtin_amdgcn_fmed3f(wp[i] * rdelta, lo, hi);
        cmz[i] = __builtin_rintf(t);
        risky |= !(fabsf(t - cmz[i]) < lim);
      }
      if (__builtin_amdgcn_ballot_w64(risky) != 0) {       // wave-uniform
        const float z = -lo - 0.25f, nz = -z, qz = qmax - z;   // as group_params gave them
#pragma unroll
        for (int i = 0; i < 8; ++i)
          cmz[i] = __builtin_amdgcn_fmed3f(__builtin_rintf(div_rn(wp[i], delta, rdelta)), nz, qz);
      }
      // W_hat = deq / s from the reciprocal; a wave with an extreme scale
      // redoes the row with true divisions (one wave-uniform branch per row,
      // not one per element)
      float deq[8], what[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        deq[i] = cmz[i] * delta;
        what[i] = div_rn(deq[i], sv[i], ys[i]);
      }
      if (exact_div) {
#pragma unroll
        for (int i = 0; i < 8; ++i) what[i] = deq[i] / sv[i];
      }
      float o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        o[i] = kDelta ? (w[i] - what[i]) : what[i];
        if (kKeep && kept[i]) o[i] = kDelta ? 0.0f : w[i];
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
    };

    if constexpr (kShare) {
      // Four rows at a time: partial min / max, one reduce-scatter, the group
      // parameters once per (row, group), broadcast back per row.
#pragma unroll
      for (int h = 0; h < kFqRowSteps; h += 4) {
        // w' of the four rows is kept; w is widened again where the row is
        // finished (one instruction per element, against 32 registers that
        // would cost a wave per SIMD).
        float wp[4][8], mn[4], mx[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float w[8];
          widen_wrow(wraw[h + q], w);
#pragma unroll
          for (int i = 0; i < 8; ++i) wp[q][i] = w[i] * sv[i];
          mn[q] = wp[q][0];
          mx[q] = wp[q][0];
#pragma unroll
          for (int i = 1; i < 8; ++i) {
            mn[q] = fminf(mn[q], wp[q][i]);
            mx[q] = fmaxf(mx[q], wp[q][i]);
          }
        }
        float gmn, gmx;
        minmax_scatter4(mn, mx, lane, gmn, gmx);
        const GroupQ g = group_params(gmn, gmx, qmax, rq);
        const float lim = safe_limit(gmn, gmx, g.rdelta, g.z);
        const float lo = -g.z - 0.25f, hi = qmax - g.z + 0.25f;
        finish_row(h + 0, wp[0], from_quad<0>(g.delta), from_quad<0>(g.rdelta),
                   from_quad<0>(lo), from_quad<0>(hi), from_quad<0>(lim));
        finish_row(h + 1, wp[1], from_quad<1>(g.delta), from_quad<1>(g.rdelta),
                   from_quad<1>(lo), from_quad<1>(hi), from_quad<1>(lim));
        finish_row(h + 2, wp[2], from_quad<2>(g.delta), from_quad<2>(g.rdelta),
                   from_quad<2>(lo), from_quad<2>(hi), from_quad<2>(lim));
        finish_row(h + 3, wp[3], from_quad<3>(g.delta), from_quad<3>(g.rdelta),
                   from_quad<3>(lo), from_quad<3>(hi), from_quad<3>(lim));
      }
    } else {
#pragma unroll
      for (int p = 0; p < kFqRowSteps; ++p) {
        float w[8], wp[8];
        float mn, mx;
        widen_wrow(wraw[p], w);
#pragma unroll
        for (int i = 0; i < 8; ++i) wp[i] = w[i] * sv[i];
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
        const float lim = safe_limit(mn, mx, g.rdelta, g.z);
        finish_row(p, wp, g.delta, g.rdelta, -g.z - 0.25f, qmax - g.z + 0.25f, lim);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Final quantisation + packing for one scale vector.
//
// A wave owns 1024 consecutive columns (16 per lane: two 16-byte loads of a
// 16-bit row) of kPackRows rows.  Its 16 scales are loaded once; all
// kPackRows rows are loaded up front, so a lane has that many rows of
// transfers in flight, and then handled row by row: scale, group min / max
// over the group's G/16 lanes (DPP), step, reciprocal and zero-point, the 16
// codes, and the packing.  Two neighbouring lanes hold 32 consecutive codes,
// i.e. exactly `bits` words of the row's little-endian bitstream: each lane
// places its 16 codes (16 * bits bits) at bit offset 16 * bits * (lane % 2)
// of the pair's stream, the pair ORs its words together (DPP), and lane j
// stores the words w with w % 2 == j.  The first lane of each group writes the
// group's step and zero-point.  The codes take the rounding decision above.
// ---------------------------------------------------------------------------
constexpr int kPackLaneCols = 16;                  // columns per lane
constexpr int kPackCols = 64 * kPackLaneCols;      // columns per wave
constexpr int kPackRows = 4;                       // rows per wave
constexpr int kPackWaves = 4;                      // waves per workgroup

// 16 consecutive elements of a row, as raw 16-byte loads (four for fp32).
template <typename S>
struct Raw16 {
  i32x4 v[sizeof(S)];
};
template <typename S>
__device__ __forceinline__ Raw16<S> load_raw16(const S* p) {
  Raw16<S> r;
#pragma unroll
  for (int i = 0; i < (int)sizeof(S); ++i) r.v[i] = reinterpret_cast<const i32x4*>(p)[i];
  return r;
}
template <typename S>
__device__ __forceinline__ void unpack16(const Raw16<S>& r, float (&v)[16]) {
  const S* e = reinterpret_cast<const S*>(&r.v[0]);
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = to_f32(e[i]);
}

__device__ __forceinline__ uint32_t pair_or(uint32_t v) {
  return v | (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, true);   // [1,0,3,2]
}

// Word wi of a bit stream that holds `f` (NW words, little-endian) shifted left by SH bits.
template <int NW, int SH>
__device__ __forceinline__ uint32_t shifted_word(const uint32_t (&f)[NW], int wi) {
  const int q = SH / 32, r = SH % 32;
  const int src = wi - q;
  const uint32_t lo = (src >= 0 && src < NW) ? f[src] : 0u;
  if (r == 0) return lo;
  const uint32_t below = (src - 1 >= 0 && src - 1 < NW) ? f[src - 1] : 0u;
  return (lo << r) | (below >> (32 - r));
}

// Sizes arrive precomputed (no integer division in the kernel): col_blocks =
// ceil(K / 1024) waves per row block, group_shift = log2(group), lanes =
// group / 16 (a power of two, at least 2).
// kShare: groups of 128 columns (8 lanes); the four rows' group parameters are
// formed once per row and group (minmax_scatter4_8) and broadcast.
template <typename S, int BITS, bool kShare>
__global__ __launch_bounds__(64 * kPackWaves) void quantize_pack_kernel(
    const S* __restrict__ W, int N, int K, const float* __restrict__ s, int group_shift,
    int lanes, int col_blocks, uint32_t* __restrict__ codes, float* __restrict__ scales,
    uint8_t* __restrict__ zeros) {
  constexpr int NW = (16 * BITS + 31) / 32;                // words of one lane's 16 codes
  const int lane = threadIdx.x & 63;
  const int wave_id = __builtin_amdgcn_readfirstlane(blockIdx.x * kPackWaves + (threadIdx.x >> 6));
  const int rb = wave_id / col_blocks;                     // scalar
  const int cb = wave_id - rb * col_blocks;
  const int row0 = rb * kPackRows;
  if (row0 >= N) return;                                   // wave-uniform
  const int col = cb * kPackCols + lane * kPackLaneCols;
  const bool col_ok = col < K;                             // whole groups of lanes
  const float qmax = (float)((1 << BITS) - 1);
  const float rq = 1.0f / qmax;

  float sv[16];
  if (col_ok) {
    float a[8], b[8];
    load8(s + col, a);
    load8(s + col + 8, b);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sv[i] = a[i];
      sv[8 + i] = b[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) sv[i] = 1.0f;
  }
  const S* wrow = W + (int64_t)row0 * K + col;
  Raw16<S> raw[kPackRows];
#pragma unroll
  for (int p = 0; p < kPackRows; ++p) {
    if (col_ok && row0 + p < N) {
      raw[p] = load_raw16(wrow + (int64_t)p * K);
    } else {
#pragma unroll
      for (int i = 0; i < (int)sizeof(S); ++i) raw[p].v[i] = i32x4{0, 0, 0, 0};
    }
  }
  const int j = lane & 1;                                  // position in the pair
  const int words_per_row = (K >> 5) * BITS;
  const int groups_per_row = K >> group_shift;
  uint32_t* dst = codes + (int64_t)row0 * words_per_row + (col >> 5) * BITS;
  const int64_t g0 = (int64_t)row0 * groups_per_row + (col >> group_shift);
  const bool group_lead = (lane & (lanes - 1)) == 0;
  // Codes, packing and stores of row step p from its w' and its group's step,
  // reciprocal, zero-point and safety bound.
  auto finish_row = [&](int p, const float (&wp)[16], float delta, float rdelta, float zf,
                        float lim) {
    const GroupQ g{delta, rdelta, zf};
    // Code = clamp(rint(t), 0, qmax).  t is first clamped to [-1/4, qmax + 1/4]
    // (beyond, the clamp decides the code whatever the rounding); adding 2^23
    // then rounds it to the nearest integer, ties to even (2^23 is even, and
    // just below 2^23 the tie at -1/4 goes up to 2^23), leaving rint(t) in
    // the low mantissa bits; the difference to t is exact.
    uint32_t code[16];
    bool risky = false;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float t = __builtin_amdgcn_fmed3f(fmaf(wp[i], g.rdelta, g.z), -0.25f, qmax + 0.25f);
      const float u = t + 0x1p23f;
      risky |= !(fabsf(t - (u - 0x1p23f)) < lim);
      code[i] = __float_as_uint(u) - 0x4B000000u;        // bits of 2^23
    }
    if (__builtin_amdgcn_ballot_w64(risky) != 0) {         // wave-uniform
#pragma unroll
      for (int i = 0; i < 16; ++i)
        code[i] = (uint32_t)__builtin_amdgcn_fmed3f(
            __builtin_rintf(div_rn(wp[i], g.delta, g.rdelta)) + g.z, 0.0f, qmax);
    }
    // the lane's 16 codes as NW words, bit BITS * i + b of code i at stream bit BITS * i + b
    uint32_t f[NW];
#pragma unroll
    for (int q = 0; q < NW; ++q) f[q] = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t c = code[i];
      const int pos = BITS * i;                            // compile-time after unrolling
      f[pos >> 5] |= c << (pos & 31);
      if ((pos & 31) + BITS > 32) f[(pos >> 5) + 1] |= c >> (32 - (pos & 31));
    }
    // the pair's BITS words: lane 0's codes at bit 0, lane 1's at bit 16 * BITS
    uint32_t word[BITS];
#pragma unroll
    for (int wi = 0; wi < BITS; ++wi)
      word[wi] = pair_or(j ? shifted_word<NW, 16 * BITS>(f, wi) : shifted_word<NW, 0>(f, wi));
    if (col_ok) {
#pragma unroll
      for (int wi = 0; wi < BITS; ++wi)
        if ((wi & 1) == j) dst[(int64_t)p * words_per_row + wi] = word[wi];
      if (group_lead) {
        scales[g0 + (int64_t)p * groups_per_row] = g.delta;
        zeros[g0 + (int64_t)p * groups_per_row] = (uint8_t)g.z;
      }
    }
  };
  if constexpr (kShare) {
    float wp[kPackRows][16], mn[kPackRows], mx[kPackRows];
#pragma unroll
    for (int p = 0; p < kPackRows; ++p) {
      float w[16];
      unpack16(raw[p], w);
#pragma unroll
      for (int i = 0; i < 16; ++i) wp[p][i] = w[i] * sv[i];
      mn[p] = wp[p][0];
      mx[p] = wp[p][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) {
        mn[p] = fminf(mn[p], wp[p][i]);
        mx[p] = fmaxf(mx[p], wp[p][i]);
      }
    }
    float gmn, gmx;
    minmax_scatter4_8(mn, mx, lane, gmn, gmx);
    const GroupQ g = group_params(gmn, gmx, qmax, rq);
    const float lim = safe_limit(gmn, gmx, g.rdelta, g.z);
    static_assert(kPackRows == 4, "four rows per reduce-scatter");
    // rows past N (wave-uniform) are skipped; their zero rows took part harmlessly
    if (row0 + 0 < N)
      finish_row(0, wp[0], from_pair<0>(g.delta), from_pair<0>(g.rdelta), from_pair<0>(g.z),
                 from_pair<0>(lim));
    if (row0 + 1 < N)
      finish_row(1, wp[1], from_pair<1>(g.delta), from_pair<1>(g.rdelta), from_pair<1>(g.z),
                 from_pair<1>(lim));
    if (row0 + 2 < N)
      finish_row(2, wp[2], from_pair<2>(g.delta), from_pair<2>(g.rdelta), from_pair<2>(g.z),
                 from_pair<2>(lim));
    if (row0 + 3 < N)
      finish_row(3, wp[3], from_pair<3>(g.delta), from_pair<3>(g.rdelta), from_pair<3>(g.z),
                 from_pair<3>(lim));
  } else {
#pragma unroll
    for (int p = 0; p < kPackRows; ++p) {
      if (row0 + p >= N) break;                              // wave-uniform
      float w[16], wp[16];
      unpack16(raw[p], w);
#pragma unroll
      for (int i = 0; i < 16; ++i) wp[i] = w[i] * sv[i];
      float mn = wp[0], mx = wp[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) {
        mn = fminf(mn, wp[i]);
        mx = fmaxf(mx, wp[i]);
      }
      group_minmax(mn, mx, lanes);
      const GroupQ g = group_params(mn, mx, qmax, rq);
      finish_row(p, wp, g.delta, g.rdelta, g.z, safe_limit(mn, mx, g.rdelta, g.z));
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
    // G = 128: group parameters shared across each group's lanes; kRs: the
    // reciprocals of s are read from rs rather than computed
#define AWQ_FQ_ROWS(L, R)                                                                        \
  fake_quant_kernel<S, O, kDelta, false, L, false, R><<<grid, kFqThreads, 0, st>>>(              \
      w, N, K, s, rs, n_s, qmax, lanes, out_rows, o)
    if (lanes == 16) {
      if (rs) AWQ_FQ_ROWS(16, true); else AWQ_FQ_ROWS(16, false);
    } else {
      if (rs) AWQ_FQ_ROWS(0, true); else AWQ_FQ_ROWS(0, false);
    }
#undef AWQ_FQ_ROWS
    return hipGetLastError();
  }
  if (!rs) return hipErrorInvalidValue;   // the search's launches pass RN(1 / s)
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
  // the caller keeps N and K below 2^31 (operands below 4 GiB), so do the wave counts
  const int col_blocks = (int)((K + kPackCols - 1) / kPackCols);
  const int64_t waves = (int64_t)col_blocks * ((N + kPackRows - 1) / kPackRows);
  if (waves > INT32_MAX - kPackWaves) return hipErrorInvalidValue;
  const unsigned blocks = (unsigned)((waves + kPackWaves - 1) / kPackWaves);
  const S* w = static_cast<const S*>(W);
  const int lanes = group / kPackLaneCols;
  const int group_shift = __builtin_ctz((unsigned)group);
  ProfScope p("awq_quantize_pack", st);
  // G = 128 (8 lanes a group): group parameters shared across the group's lanes
#define AWQ_PACK_K(B, SH)                                                                         \
  quantize_pack_kernel<S, B, SH><<<blocks, 64 * kPackWaves, 0, st>>>(                             \
      w, (int)N, (int)K, s, group_shift, lanes, col_blocks, codes, scales, zeros)
#define AWQ_PACK(B)                                                                               \
  if (lanes == 8) AWQ_PACK_K(B, true); else AWQ_PACK_K(B, false)
  switch (bits) {
    case 2: AWQ_PACK(2); break;
    case 3: AWQ_PACK(3); break;
    case 4: AWQ_PACK(4); break;
    case 5: AWQ_PACK(5); break;
    case 6: AWQ_PACK(6); break;
    case 7: AWQ_PACK(7); break;
    default: AWQ_PACK(8); break;
  }
#undef AWQ_PACK
#undef AWQ_PACK_K
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
