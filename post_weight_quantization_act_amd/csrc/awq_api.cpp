// C ABI of the AWQ scale-search library: argument validation, workspace
// layout, the order of launches on the caller's stream, error reporting and
// optional per-launch timing.  All arithmetic runs in the HIP kernels of
// act_stats.hip, quant.hip and gemm_sse.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

namespace {

thread_local std::string g_last_error;

awq_status_t fail(awq_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

awq_status_t hip_fail(hipError_t e, const char* what) {
  return fail(AWQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr uint64_t kMaxBufferBytes = 0xFFFFFF00ull;  // byte offsets inside kernels are 32-bit
constexpr int kMaxAlpha = 4096;
constexpr int kLaunchRounds = 4;      // candidate-GEMM rounds of the persistent grid per launch
constexpr int64_t kGptqMaxK = 32768;   // the fp64 factor matrix is K^2 * 8 bytes
constexpr int64_t kLowbitGemmMaxM = 65535ll * 128;  // activation-row tiles on grid y
constexpr int64_t kLowbitGemmMaxK = 1ll << 22;       // a 256-row activation tile in 32-bit offsets

int esize(awq_dtype_t dt) { return dt == AWQ_F32 ? 4 : 2; }

bool valid_dtype(int dt) { return dt == AWQ_F32 || dt == AWQ_F16 || dt == AWQ_BF16; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// Checks shared by the quantiser entry points.
awq_status_t check_quant_args(awq_dtype_t dt, int64_t N, int64_t K, int bits, int group) {
  if (!valid_dtype(dt)) return fail(AWQ_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  if (N < 1 || K < 1) return fail(AWQ_ERR_INVALID_ARG, "N and K must be >= 1 (N=%lld K=%lld)",
                                  (long long)N, (long long)K);
  if (bits < 2 || bits > 8) return fail(AWQ_ERR_UNSUPPORTED, "bits=%d outside [2, 8]", bits);
  if (group < 32 || group > 512 || (group & (group - 1)) != 0)
    return fail(AWQ_ERR_UNSUPPORTED, "group=%d must be a power of two in [32, 512]", group);
  if (K % group != 0)
    return fail(AWQ_ERR_INVALID_ARG, "K=%lld is not a multiple of group=%d", (long long)K, group);
  if ((uint64_t)awq::padded_rows(N) * (uint64_t)K * (uint64_t)esize(dt) > kMaxBufferBytes ||
      N > INT32_MAX)
    return fail(AWQ_ERR_UNSUPPORTED, "W [%lld, %lld] exceeds the 4 GiB operand limit",
                (long long)N, (long long)K);
  return AWQ_OK;
}

// ---------------------------------------------------------------------------
// Workspace layout of the search.
// ---------------------------------------------------------------------------
awq_status_t compute_layout(awq_dtype_t dt, int64_t N, int64_t K, int64_t T, int n_alpha,
                            uint32_t flags, size_t ws_bytes, awq_search_layout_t* L) {
  const awq::GemmTiles gt = awq::gemm_tiles(dt);
  const bool delta = (flags & AWQ_SEARCH_REFERENCE_OUTPUT) == 0;
  std::memset(L, 0, sizeof(*L));
  L->tile_m = gt.tile_m;
  L->tile_n = gt.tile_n;
  // the flattened GEMM grid (tiles of every candidate of a batch) is an int
  const int64_t tm = (T + gt.tile_m - 1) / gt.tile_m, tn = (N + gt.tile_n - 1) / gt.tile_n;
  if (tm > INT32_MAX / 2 || tn > INT32_MAX / 2 || tm * tn > INT32_MAX / 2)
    return fail(AWQ_ERR_UNSUPPORTED, "%lld x %lld output tiles of one candidate exceed the GEMM's "
                "range", (long long)tm, (long long)tn);
  L->tiles_m = (int32_t)tm;
  L->tiles_n = (int32_t)tn;
  size_t off = 0;
  L->s_table_offset = off;   // s [n_alpha][K], then RN(1/s) [n_alpha][K]
  off = align_up(off + 2 * (size_t)n_alpha * (size_t)K * 4);
  L->partials_offset = off;
  off = align_up(off + (size_t)n_alpha * (size_t)L->tiles_m * (size_t)L->tiles_n * 8);
  if (delta) {
    L->y_ref_offset = SIZE_MAX;
  } else {
    // fp16/bf16: whole 256 x 256 tiles in the GEMM's fragment layout
    const bool frag = dt != AWQ_F32;
    L->y_ref_offset = off;
    off = align_up(off + (frag ? (size_t)awq::padded_rows(T) * (size_t)awq::padded_rows(N)
                               : (size_t)T * (size_t)N) * 4);
  }
  const bool tiled = dt != AWQ_F32;   // the MFMA path reads tiled operands
  if (tiled) {
    L->x_tiled_offset = off;
    off = align_up(off + (size_t)awq::padded_rows(T) * (size_t)K * 2);
  } else {
    L->x_tiled_offset = SIZE_MAX;
  }
  L->w_hat_offset = off;
  const size_t rows = tiled ? (size_t)awq::padded_rows(N) : (size_t)N;
  const size_t per_alpha = align_up(rows * (size_t)K * (size_t)esize(dt));
  int batch = n_alpha;
  if (ws_bytes != 0) {
    if (ws_bytes < off + per_alpha)
      return fail(AWQ_ERR_WORKSPACE, "workspace of %zu bytes is below the minimum %zu", ws_bytes,
                  off + per_alpha);
    const size_t fit = (ws_bytes - off) / per_alpha;
    if (fit < (size_t)batch) batch = (int)fit;
  }
  // keep the flattened GEMM grid within int range
  const int64_t tiles = (int64_t)L->tiles_m * L->tiles_n;
  const int64_t max_batch = (int64_t)(INT32_MAX / 2) / (tiles > 0 ? tiles : 1);
  if (batch > max_batch) batch = (int)(max_batch > 0 ? max_batch : 1);
  L->alpha_batch = batch;
  L->total_bytes = off + (size_t)batch * per_alpha;
  return AWQ_OK;
}

// ---------------------------------------------------------------------------
// Per-launch event timing.
// ---------------------------------------------------------------------------
struct ProfRec {
  std::string name;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
std::vector<ProfRec> g_prof;
std::atomic<bool> g_prof_on{false};
std::string g_prof_prefix;   // guarded by g_prof_mu

// ---------------------------------------------------------------------------
// Mixed-precision ablation: keep the top channels, round the rest to nearest.
// Workspace: the search layout for one candidate (alpha = 0, weight-delta
// form), then the keep mask [K] uint8, the argmin index and a [K] fp32 copy
// of the unit scales.
// ---------------------------------------------------------------------------
struct KeepLayout {
  awq_search_layout_t search;
  size_t keep_offset, best_offset, s_copy_offset, total_bytes;
};

awq_status_t keep_layout(awq_dtype_t dt, int64_t N, int64_t K, int64_t T, KeepLayout* L) {
  awq_status_t st = compute_layout(dt, N, K, T, 1, AWQ_SEARCH_WEIGHT_DELTA, 0, &L->search);
  if (st != AWQ_OK) return st;
  size_t off = align_up(L->search.total_bytes);
  L->keep_offset = off;
  off = align_up(off + (size_t)K);
  L->best_offset = off;
  off = align_up(off + 4);
  L->s_copy_offset = off;
  off = align_up(off + (size_t)K * 4);
  L->total_bytes = off;
  return AWQ_OK;
}

}  // namespace

namespace awq {

int prof_begin(const char* kernel, hipStream_t stream) {
  if (!g_prof_on.load(std::memory_order_relaxed)) return -1;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_prefix.empty() && std::strncmp(kernel, g_prof_prefix.c_str(), g_prof_prefix.size()) != 0)
    return -1;
  ProfRec r;
  r.name = kernel;
  if (hipEventCreate(&r.start) != hipSuccess) return -1;
  if (hipEventCreate(&r.stop) != hipSuccess) {
    (void)hipEventDestroy(r.start);
    return -1;
  }
  (void)hipEventRecord(r.start, stream);
  g_prof.push_back(r);
  return (int)g_prof.size() - 1;
}

void prof_end(int token, hipStream_t stream) {
  if (token < 0) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if ((size_t)token < g_prof.size()) (void)hipEventRecord(g_prof[token].stop, stream);
}

}  // namespace awq

#define AWQ_GUARD_BEGIN try {
#define AWQ_GUARD_END                                                  \
  }                                                                    \
  catch (...) {                                                        \
    return fail(AWQ_ERR_HIP, "unexpected C++ exception in the library"); \
  }

extern "C" {

const char* awq_version(void) { return "awq-mi355x 0.1"; }

const char* awq_last_error(void) { return g_last_error.c_str(); }

size_t awq_act_stats_workspace_size(int64_t T, int64_t K) {
  if (T < 1 || K < 1) return 0;
  return align_up(awq::act_stats_ws_bytes(T, K));
}

awq_status_t awq_act_stats(const void* X, awq_dtype_t x_dtype, int64_t T, int64_t K, float* a_out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  AWQ_GUARD_BEGIN
  if (!valid_dtype(x_dtype)) return fail(AWQ_ERR_INVALID_ARG, "unknown dtype %d", (int)x_dtype);
  if (T < 1 || K < 1) return fail(AWQ_ERR_INVALID_ARG, "T and K must be >= 1");
  if (!X || !a_out) return fail(AWQ_ERR_INVALID_ARG, "null X or a_out");
  const size_t need = awq_act_stats_workspace_size(T, K);
  if (!workspace || workspace_bytes < need)
    return fail(AWQ_ERR_WORKSPACE, "act_stats needs %zu workspace bytes, got %zu", need,
                workspace_bytes);
  if (!aligned(workspace, 8)) return fail(AWQ_ERR_WORKSPACE, "workspace must be 8-byte aligned");
  hipError_t e = awq::launch_act_stats(X, x_dtype, T, K, a_out, workspace, stream);
  if (e != hipSuccess) return hip_fail(e, "act_stats launch");
  return AWQ_OK;
  AWQ_GUARD_END
}

awq_status_t awq_scale_table(const float* a, int64_t K, const float* alphas, int n_alpha,
                             float* s_out, hipStream_t stream) {
  AWQ_GUARD_BEGIN
  if (!a || !alphas || !s_out) return fail(AWQ_ERR_INVALID_ARG, "null pointer");
  if (K < 1 || n_alpha < 1 || n_alpha > kMaxAlpha)
    return fail(AWQ_ERR_INVALID_ARG, "K=%lld n_alpha=%d", (long long)K, n_alpha);
  for (int k = 0; k < n_alpha; ++k)
    if (!std::isfinite(alphas[k])) return fail(AWQ_ERR_INVALID_ARG, "alpha[%d] is not finite", k);
  for (int c0 = 0; c0 < n_alpha; c0 += 64) {
    awq::AlphaChunk ch;
    ch.n = std::min(64, n_alpha - c0);
    for (int i = 0; i < ch.n; ++i) ch.v[i] = alphas[c0 + i];
    hipError_t e = awq::launch_scale_table(a, K, ch, s_out + (size_t)c0 * K, nullptr, stream);
    if (e != hipSuccess) return hip_fail(e, "scale_table launch");
  }
  return AWQ_OK;
  AWQ_GUARD_END
}

awq_status_t awq_fake_quant(const void* W, awq_dtype_t w_dtype, int64_t N, int64_t K,
                            const float* s, int n_s, int bits, int group, uint32_t flags,
                            void* out, awq_dtype_t out_dtype, hipStream_t stream) {
  AWQ_GUARD_BEGIN
  awq_status_t st = check_quant_args(w_dtype, N, K, bits, group);
  if (st != AWQ_OK) return st;
  if (!W || !s || !out) return fail(AWQ_ERR_INVALID_ARG, "null pointer");
  if (n_s < 1) return fail(AWQ_ERR_INVALID_ARG, "n_s must be >= 1");
  if (flags & ~AWQ_FQ_WEIGHT_DELTA) return fail(AWQ_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if (out_dtype != w_dtype)
    return fail(AWQ_ERR_UNSUPPORTED, "out_dtype must equal w_dtype");
  if (!aligned(W, 16) || !aligned(s, 16) || !aligned(out, 16))
    return fail(AWQ_ERR_UNSUPPORTED, "W, s and out must be 16-byte aligned");
  hipError_t e = awq::launch_fake_quant(W, w_dtype, N, K, s, nullptr, n_s, bits, group,
                                        (flags & AWQ_FQ_WEIGHT_DELTA) != 0, false, out, stream);
  if (e != hipSuccess) return hip_fail(e, "fake_quant launch");
  return AWQ_OK;
  AWQ_GUARD_END
}

awq_status_t awq_search_layout(awq_dtype_t dtype, int64_t N, int64_t K, int64_t T, int n_alpha,
                               uint32_t flags, size_t workspace_bytes,
                               awq_search_layout_t* layout_out) {
  AWQ_GUARD_BEGIN
  if (!layout_out) return fail(AWQ_ERR_INVALID_ARG, "null layout_out");
  if (!valid_dtype(dtype)) return fail(AWQ_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (N < 1 || K < 1 || T < 1 || n_alpha < 1 || n_alpha > kMaxAlpha)
    return fail(AWQ_ERR_INVALID_ARG, "sizes must be >= 1 and n_alpha <= %d", kMaxAlpha);
  if (flags & ~AWQ_SEARCH_REFERENCE_OUTPUT)
    return fail(AWQ_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  return compute_layout(dtype, N, K, T, n_alpha, flags, workspace_bytes, layout_out);
  AWQ_GUARD_END
}

size_t awq_search_workspace_size(int64_t N, int64_t K, int64_t T, int n_alpha) {
  if (N < 1 || K < 1 || T < 1 || n_alpha < 1 || n_alpha > kMaxAlpha) return 0;
  size_t most = 0;
  for (awq_dtype_t dt : {AWQ_F32, AWQ_F16, AWQ_BF16}) {
    awq_search_layout_t L;
    if (compute_layout(dt, N, K, T, n_alpha, AWQ_SEARCH_WEIGHT_DELTA, 0, &L) != AWQ_OK) return 0;
    most = std::max(most, L.total_bytes);
  }
  return most;
}

awq_status_t awq_search_scales(const void* W, const void* X, awq_dtype_t dtype, int64_t N,
                               int64_t K, int64_t T, const float* a, int bits, int group,
                               const float* alphas, int n_alpha, uint32_t flags,
                               double* losses_out, float* s_best_out, int32_t* best_idx_out,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  AWQ_GUARD_BEGIN
  awq_status_t st = check_quant_args(dtype, N, K, bits, group);
  if (st != AWQ_OK) return st;
  if (!W || !X || !a || !alphas || !losses_out || !s_best_out || !best_idx_out)
    return fail(AWQ_ERR_INVALID_ARG, "null pointer");
  if (T < 1) return fail(AWQ_ERR_INVALID_ARG, "T must be >= 1");
  if (n_alpha < 1 || n_alpha > kMaxAlpha)
    return fail(AWQ_ERR_INVALID_ARG, "n_alpha=%d outside [1, %d]", n_alpha, kMaxAlpha);
  if (flags & ~AWQ_SEARCH_REFERENCE_OUTPUT)
    return fail(AWQ_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if ((flags & AWQ_SEARCH_REFERENCE_OUTPUT) && dtype == AWQ_BF16)
    return fail(AWQ_ERR_UNSUPPORTED,
                "the reference-output form is not offered for bf16 (W_hat rounding exceeds the "
                "loss tolerance); use AWQ_SEARCH_WEIGHT_DELTA");
  for (int k = 0; k < n_alpha; ++k)
    if (!std::isfinite(alphas[k])) return fail(AWQ_ERR_INVALID_ARG, "alpha[%d] is not finite", k);
  if ((uint64_t)awq::padded_rows(T) * (uint64_t)K * (uint64_t)esize(dtype) > kMaxBufferBytes ||
      T > INT32_MAX)
    return fail(AWQ_ERR_UNSUPPORTED, "X [%lld, %lld] exceeds the 4 GiB operand limit",
                (long long)T, (long long)K);
  if (!aligned(W, 16) || !aligned(X, 16) || !aligned(a, 4) || !aligned(s_best_out, 4))
    return fail(AWQ_ERR_UNSUPPORTED, "W and X must be 16-byte aligned");
  if (!workspace) return fail(AWQ_ERR_WORKSPACE, "null workspace");
  if (!aligned(workspace, 256)) return fail(AWQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  awq_search_layout_t L;
  st = compute_layout(dtype, N, K, T, n_alpha, flags, workspace_bytes, &L);
  if (st != AWQ_OK) return st;
  if (workspace_bytes < L.total_bytes)
    return fail(AWQ_ERR_WORKSPACE, "workspace of %zu bytes is below %zu", workspace_bytes,
                L.total_bytes);

  char* ws = static_cast<char*>(workspace);
  float* s_table = reinterpret_cast<float*>(ws + L.s_table_offset);
  float* rs_table = s_table + (size_t)n_alpha * K;
  double* partials = reinterpret_cast<double*>(ws + L.partials_offset);
  const bool delta = (flags & AWQ_SEARCH_REFERENCE_OUTPUT) == 0;
  float* y_ref = delta ? nullptr : reinterpret_cast<float*>(ws + L.y_ref_offset);
  void* w_hat = ws + L.w_hat_offset;

  hipError_t e;
  // step 2: scale table
  for (int c0 = 0; c0 < n_alpha; c0 += 64) {
    awq::AlphaChunk ch;
    ch.n = std::min(64, n_alpha - c0);
    for (int i = 0; i < ch.n; ++i) ch.v[i] = alphas[c0 + i];
    e = awq::launch_scale_table(a, K, ch, s_table + (size_t)c0 * K, rs_table + (size_t)c0 * K,
                                stream);
    if (e != hipSuccess) return hip_fail(e, "scale_table launch");
  }
  // fp16/bf16: X in the GEMM's tiled layout, once per call
  const bool tiled = dtype != AWQ_F32;
  const void* gemm_x = X;
  if (tiled) {
    void* xt = ws + L.x_tiled_offset;
    e = awq::launch_tile_rows(X, T, K, xt, stream);
    if (e != hipSuccess) return hip_fail(e, "tile_rows launch");
    gemm_x = xt;
  }
  // reference output W X, once per layer (B = the caller's row-major W)
  if (!delta) {
    e = awq::launch_gemm(awq::Epi::kRefOut, dtype, gemm_x, W, false, 1, T, N, K, y_ref, nullptr, 0,
                         stream);
    if (e != hipSuccess) return hip_fail(e, "reference GEMM launch");
  }
  // steps 3-4 over the grid: alpha_batch candidates fake-quantised per pass (W
  // read once per pass); the pass's GEMM tiles (fp16/bf16) in launches of
  // kLaunchRounds full rounds of the persistent grid, the last launch taking
  // the rest.  Measured on the layer shapes: launches of a few rounds run 1-5%
  // faster than one launch per pass or per candidate, and a launch that ends
  // on a partly filled round leaves CUs idle, which is why the split is by
  // rounds and not by candidates.
  const int64_t cand_tiles = (int64_t)L.tiles_m * L.tiles_n;
  const int64_t chunk = (int64_t)kLaunchRounds * awq::gemm_grid();
  const awq::Epi epi = delta ? awq::Epi::kSseDelta : awq::Epi::kSseRef;
  for (int a0 = 0; a0 < n_alpha; a0 += L.alpha_batch) {
    const int nb = std::min(L.alpha_batch, n_alpha - a0);
    e = awq::launch_fake_quant(W, dtype, N, K, s_table + (size_t)a0 * K, rs_table + (size_t)a0 * K,
                               nb, bits, group, delta, tiled, w_hat, stream);
    if (e != hipSuccess) return hip_fail(e, "fake_quant launch");
    if (!tiled) {
      e = awq::launch_gemm(epi, dtype, gemm_x, w_hat, false, nb, T, N, K, y_ref, partials, a0,
                           stream);
      if (e != hipSuccess) return hip_fail(e, "candidate GEMM launch");
      continue;
    }
    const int64_t total = nb * cand_tiles;
    for (int64_t t0 = 0; t0 < total; t0 += chunk) {
      e = awq::launch_gemm(epi, dtype, gemm_x, w_hat, true, nb, T, N, K, y_ref, partials, a0,
                           stream, (int)t0, (int)std::min(chunk, total - t0));
      if (e != hipSuccess) return hip_fail(e, "candidate GEMM launch");
    }
  }
  // step 5: losses, argmin, best scales
  const int64_t tiles = (int64_t)L.tiles_m * L.tiles_n;
  e = awq::launch_loss_argmin(partials, n_alpha, tiles, 1.0 / ((double)T * (double)N), s_table, K,
                              losses_out, best_idx_out, s_best_out, stream);
  if (e != hipSuccess) return hip_fail(e, "loss/argmin launch");
  return AWQ_OK;
  AWQ_GUARD_END
}

size_t awq_salient_keep_workspace_size(awq_dtype_t dtype, int64_t N, int64_t K, int64_t T) {
  if (!valid_dtype(dtype) || N < 1 || K < 1 || T < 1) return 0;
  KeepLayout L;
  if (keep_layout(dtype, N, K, T, &L) != AWQ_OK) return 0;
  return L.total_bytes;
}

awq_status_t awq_salient_keep_loss(const void* W, const void* X, awq_dtype_t dtype, int64_t N,
                                   int64_t K, int64_t T, const float* score, int64_t n_keep,
                                   int bits, int group, double* loss_out, uint8_t* keep_out,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  AWQ_GUARD_BEGIN
  awq_status_t st = check_quant_args(dtype, N, K, bits, group);
  if (st != AWQ_OK) return st;
  if (dtype == AWQ_F32) return fail(AWQ_ERR_UNSUPPORTED, "the ablation runs on fp16/bf16 layers");
  if (T < 1) return fail(AWQ_ERR_INVALID_ARG, "T must be >= 1");
  if (n_keep < 0 || n_keep > K) return fail(AWQ_ERR_INVALID_ARG, "n_keep=%lld outside [0, K]",
                                            (long long)n_keep);
  if (!W || !X || !score || !loss_out) return fail(AWQ_ERR_INVALID_ARG, "null pointer");
  if (!aligned(W, 16) || !aligned(X, 16) || !aligned(score, 4))
    return fail(AWQ_ERR_UNSUPPORTED, "W and X must be 16-byte aligned, score 4-byte");
  if ((uint64_t)awq::padded_rows(T) * (uint64_t)K * 2 > kMaxBufferBytes)
    return fail(AWQ_ERR_UNSUPPORTED, "X exceeds the 4 GiB operand limit");
  if (!workspace) return fail(AWQ_ERR_WORKSPACE, "null workspace");
  if (!aligned(workspace, 256)) return fail(AWQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  KeepLayout L;
  st = keep_layout(dtype, N, K, T, &L);
  if (st != AWQ_OK) return st;
  if (workspace_bytes < L.total_bytes)
    return fail(AWQ_ERR_WORKSPACE, "workspace of %zu bytes is below %zu", workspace_bytes,
                L.total_bytes);
  char* ws = static_cast<char*>(workspace);
  float* s_table = reinterpret_cast<float*>(ws + L.search.s_table_offset);
  float* rs_table = s_table + K;
  double* partials = reinterpret_cast<double*>(ws + L.search.partials_offset);
  void* xt = ws + L.search.x_tiled_offset;
  void* d = ws + L.search.w_hat_offset;
  uint8_t* keep = keep_out ? keep_out : reinterpret_cast<uint8_t*>(ws + L.keep_offset);
  int32_t* best = reinterpret_cast<int32_t*>(ws + L.best_offset);
  float* s_copy = reinterpret_cast<float*>(ws + L.s_copy_offset);

  hipError_t e = awq::launch_keep_mask(score, K, n_keep, keep, stream);
  if (e != hipSuccess) return hip_fail(e, "keep mask launch");
  // unit scales (alpha = 0) and their reciprocals; the statistic only has to be finite
  awq::AlphaChunk ch;
  ch.n = 1;
  ch.v[0] = 0.0f;
  e = awq::launch_scale_table(score, K, ch, s_table, rs_table, stream);
  if (e != hipSuccess) return hip_fail(e, "scale table launch");
  e = awq::launch_tile_rows(X, T, K, xt, stream);
  if (e != hipSuccess) return hip_fail(e, "tile_rows launch");
  e = awq::launch_fake_quant(W, dtype, N, K, s_table, rs_table, 1, bits, group, true, true, d,
                             stream, keep);
  if (e != hipSuccess) return hip_fail(e, "fake_quant launch");
  e = awq::launch_gemm(awq::Epi::kSseDelta, dtype, xt, d, true, 1, T, N, K, nullptr, partials, 0,
                       stream);
  if (e != hipSuccess) return hip_fail(e, "candidate GEMM launch");
  const int64_t tiles = (int64_t)L.search.tiles_m * L.search.tiles_n;
  e = awq::launch_loss_argmin(partials, 1, tiles, 1.0 / ((double)T * (double)N), s_table, K,
                              loss_out, best, s_copy, stream);
  if (e != hipSuccess) return hip_fail(e, "loss launch");
  return AWQ_OK;
  AWQ_GUARD_END
}

// ---------------------------------------------------------------------------
// GPTQ error feedback after the scaling.
// ---------------------------------------------------------------------------
size_t awq_gptq_workspace_size(int64_t N, int64_t K, int64_t T) {
  if (N < 1 || K < 1 || T < 1) return 0;
  return awq::gptq_layout(N, K, T).bytes;
}

int64_t awq_gptq_factor_ld(int64_t K) { return K < 1 ? 0 : awq::gptq_layout(1, K, 1).Kp; }

awq_status_t awq_gptq_quantize(const void* W, const void* X, awq_dtype_t dtype, int64_t N,
                               int64_t K, int64_t T, const float* s, int bits, int group,
                               double damp, uint32_t* codes_out, float* scales_out,
                               uint8_t* zeros_out, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  AWQ_GUARD_BEGIN
  awq_status_t st = check_quant_args(dtype, N, K, bits, group);
  if (st != AWQ_OK) return st;
  if (T < 1) return fail(AWQ_ERR_INVALID_ARG, "T must be >= 1");
  if (K > kGptqMaxK) return fail(AWQ_ERR_UNSUPPORTED, "K=%lld above %lld", (long long)K,
                                 (long long)kGptqMaxK);
  if (!(damp >= 0.0) || !std::isfinite(damp))
    return fail(AWQ_ERR_INVALID_ARG, "damp must be finite and >= 0");
  if (!W || !X || !s || !codes_out || !scales_out || !zeros_out)
    return fail(AWQ_ERR_INVALID_ARG, "null pointer");
  if (!aligned(W, esize(dtype)) || !aligned(X, esize(dtype)) || !aligned(s, 4) ||
      !aligned(codes_out, 4) || !aligned(scales_out, 4))
    return fail(AWQ_ERR_UNSUPPORTED, "W, X element-aligned; s, codes, scales 4-byte aligned");
  if (!workspace) return fail(AWQ_ERR_WORKSPACE, "null workspace");
  if (!aligned(workspace, 256)) return fail(AWQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const size_t need = awq::gptq_layout(N, K, T).bytes;
  if (workspace_bytes < need)
    return fail(AWQ_ERR_WORKSPACE, "workspace of %zu bytes is below %zu", workspace_bytes, need);
  hipError_t e = awq::launch_gptq(W, X, dtype, N, K, T, s, bits, group, damp, codes_out,
                                  scales_out, zeros_out, workspace, stream);
  if (e != hipSuccess) return hip_fail(e, "gptq launch");
  return AWQ_OK;
  AWQ_GUARD_END
}

// ---------------------------------------------------------------------------
// SmoothQuant W8A8.
// ---------------------------------------------------------------------------
namespace {

struct W8a8Layout {
  size_t xq, wq, sx, sw, xt, yref, partials, scratch, bytes;
  int tiles_m, tiles_n;
};

W8a8Layout w8a8_layout(int64_t N, int64_t K, int64_t T) {
  W8a8Layout L;
  const int64_t Tp = awq::padded_rows(T), Np = awq::padded_rows(N);
  const awq::GemmTiles gt = awq::gemm_tiles(AWQ_F16);
  L.tiles_m = (int)((T + gt.tile_m - 1) / gt.tile_m);
  L.tiles_n = (int)((N + gt.tile_n - 1) / gt.tile_n);
  size_t off = 0;
  L.xq = off;
  off = align_up(off + (size_t)Tp * K);
  L.wq = off;
  off = align_up(off + (size_t)Np * K);
  L.sx = off;
  off = align_up(off + (size_t)Tp * 4);
  L.sw = off;
  off = align_up(off + (size_t)Np * 4);
  L.xt = off;
  off = align_up(off + (size_t)Tp * K * 2);
  L.yref = off;                                     // fragment layout: whole tiles
  off = align_up(off + (size_t)Tp * Np * 4);
  L.partials = off;
  off = align_up(off + (size_t)L.tiles_m * L.tiles_n * 8);
  L.scratch = off;                                  // argmin scratch: 2K floats and an index
  off = align_up(off + (size_t)K * 8 + 4);
  L.bytes = off;
  return L;
}

awq_status_t check_w8a8(awq_dtype_t dt, int64_t R, int64_t K) {
  if (!valid_dtype(dt)) return fail(AWQ_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  if (R < 1 || K < 1) return fail(AWQ_ERR_INVALID_ARG, "sizes must be >= 1");
  if (K % 64 != 0) return fail(AWQ_ERR_UNSUPPORTED, "K=%lld is not a multiple of 64", (long long)K);
  if (R > INT32_MAX) return fail(AWQ_ERR_UNSUPPORTED, "too many rows");
  return AWQ_OK;
}

}  // namespace

awq_status_t awq_smooth_scales(const void* X, const void* W, awq_dtype_t dtype, int64_t T,
                               int64_t N, int64_t K, float* absmax_out, float* s_out,
                               hipStream_t stream) {
  AWQ_GUARD_BEGIN
  awq_status_t st = check_w8a8(dtype, T, K);
  if (st != AWQ_OK) return st;
  if (N < 1 || N > INT32_MAX) return fail(AWQ_ERR_INVALID_ARG, "N must be >= 1");
  if (!X || !W || !absmax_out || !s_out) return fail(AWQ_ERR_INVALID_ARG, "null pointer");
  if (!aligned(absmax_out, 4) || !aligned(s_out, 4))
    return fail(AWQ_ERR_UNSUPPORTED, "absmax and s must be 4-byte aligned");
  hipError_t e = awq::launch_smooth_scales(X, W, dtype, T, N, K, absmax_out, s_out, stream);
  if (e != hipSuccess) return hip_fail(e, "smooth scales launch");
  return AWQ_OK;
  AWQ_GUARD_END
}

awq_status_t awq_quantize_rows_int8(const void* A, awq_dtype_t dtype, int64_t R, int64_t K,
                                    const float* s, int multiply, int8_t* q_out,
                                    float* step_out, hipStream_t stream) {
  AWQ_GUARD_BEGIN
  awq_status_t st = check_w8a8(dtype, R, K);
  if (st != AWQ_OK) return st;
  if (!A || !q_out || !step_out) return fail(AWQ_ERR_INVALID_ARG, "null pointer");
  if (!aligned(A, 16) || !aligned(q_out, 16) || !aligned(step_out, 4) || (s && !aligned(s, 4)))
    return fail(AWQ_ERR_UNSUPPORTED, "A and q 16-byte aligned, s and steps 4-byte");
  hipError_t e = awq::launch_quant_rows_int8(A, dtype, R, R, K, s, multiply != 0, false, q_out,
                                             step_out, stream);
  if (e != hipSuccess) return hip_fail(e, "int8 row quantiser launch");
  return AWQ_OK;
  AWQ_GUARD_END
}

size_t awq_w8a8_workspace_size(int64_t N, int64_t K, int64_t T) {
  if (N < 1 || K < 1 || T < 1) return 0;
  return w8a8_layout(N, K, T).bytes;
}

awq_status_t awq_w8a8_loss(const void* W, const void* X, awq_dtype_t dtype, int64_t N,
                           int64_t K, int64_t T, const float* s, double* loss_out, float* y_out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  AWQ_GUARD_BEGIN
  awq_status_t st = check_w8a8(dtype, T, K);
  if (st != AWQ_OK) return st;
  if (dtype == AWQ_F32) return fail(AWQ_ERR_UNSUPPORTED, "W8A8 runs on fp16/bf16 layers");
  if (N < 1 || N > INT32_MAX) return fail(AWQ_ERR_INVALID_ARG, "N must be >= 1");
  if (!W || !X || !loss_out) return fail(AWQ_ERR_INVALID_ARG, "null pointer");
  if (!aligned(W, 16) || !aligned(X, 16) || (s && !aligned(s, 4)) || (y_out && !aligned(y_out, 4)))
    return fail(AWQ_ERR_UNSUPPORTED, "W and X must be 16-byte aligned, s and Y 4-byte");
  if ((uint64_t)awq::padded_rows(T) * (uint64_t)K * 2 > kMaxBufferBytes ||
      (uint64_t)awq::padded_rows(N) * (uint64_t)K * 2 > kMaxBufferBytes)
    return fail(AWQ_ERR_UNSUPPORTED, "an operand exceeds the 4 GiB limit");
  if (!workspace) return fail(AWQ_ERR_WORKSPACE, "null workspace");
  if (!aligned(workspace, 256)) return fail(AWQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const W8a8Layout L = w8a8_layout(N, K, T);
  if (workspace_bytes < L.bytes)
    return fail(AWQ_ERR_WORKSPACE, "workspace of %zu bytes is below %zu", workspace_bytes, L.bytes);
  char* ws = static_cast<char*>(workspace);
  int8_t* xq = reinterpret_cast<int8_t*>(ws + L.xq);
  int8_t* wq = reinterpret_cast<int8_t*>(ws + L.wq);
  float* sx = reinterpret_cast<float*>(ws + L.sx);
  float* sw = reinterpret_cast<float*>(ws + L.sw);
  float* yref = reinterpret_cast<float*>(ws + L.yref);
  double* partials = reinterpret_cast<double*>(ws + L.partials);
  float* scratch = reinterpret_cast<float*>(ws + L.scratch);
  hipError_t e = awq::launch_quant_rows_int8(X, dtype, T, awq::padded_rows(T), K, s, false, true,
                                             xq, sx, stream);
  if (e != hipSuccess) return hip_fail(e, "int8 row quantiser launch");
  e = awq::launch_quant_rows_int8(W, dtype, N, awq::padded_rows(N), K, s, true, true, wq, sw,
                                  stream);
  if (e != hipSuccess) return hip_fail(e, "int8 row quantiser launch");
  e = awq::launch_tile_rows(X, T, K, ws + L.xt, stream);
  if (e != hipSuccess) return hip_fail(e, "tile launch");
  e = awq::launch_gemm(awq::Epi::kRefOut, dtype, ws + L.xt, W, false, 1, T, N, K, yref, nullptr, 0,
                       stream);
  if (e != hipSuccess) return hip_fail(e, "reference GEMM launch");
  e = awq::launch_gemm_w8a8(awq::Epi::kSseRef, xq, wq, T, N, K, sx, sw, yref, partials, stream);
  if (e != hipSuccess) return hip_fail(e, "int8 GEMM launch");
  e = awq::launch_loss_argmin(partials, 1, (int64_t)L.tiles_m * L.tiles_n,
                              1.0 / ((double)T * (double)N), scratch, K, loss_out,
                              reinterpret_cast<int32_t*>(scratch + 2 * K), scratch + K, stream);
  if (e != hipSuccess) return hip_fail(e, "loss launch");
  if (y_out) {
    e = awq::launch_gemm_w8a8(awq::Epi::kStore, xq, wq, T, N, K, sx, sw, y_out, nullptr, stream);
    if (e != hipSuccess) return hip_fail(e, "int8 GEMM launch");
  }
  return AWQ_OK;
  AWQ_GUARD_END
}

// ---------------------------------------------------------------------------
// The low-bit layer on the packed weights.
// ---------------------------------------------------------------------------
awq_status_t awq_lowbit_repack(const uint32_t* codes, const float* scales, const uint8_t* zeros,
                               int64_t N, int64_t K, int bits, int group, uint32_t* codes_t,
                               void* meta_t, hipStream_t stream) {
  AWQ_GUARD_BEGIN
  awq_status_t st = check_quant_args(AWQ_F16, N, K, bits, group);
  if (st != AWQ_OK) return st;
  if (!codes || !scales || !zeros || !codes_t || !meta_t)
    return fail(AWQ_ERR_INVALID_ARG, "null pointer");
  if (!aligned(codes, 4) || !aligned(scales, 4) || !aligned(codes_t, 4) || !aligned(meta_t, 8))
    return fail(AWQ_ERR_UNSUPPORTED, "codes, scales, codes_t 4-byte and meta_t 8-byte aligned");
  if ((uint64_t)N * (uint64_t)K / 32 * (uint64_t)bits * 4 > kMaxBufferBytes ||
      (uint64_t)N * (uint64_t)(K / group) * 8 > kMaxBufferBytes)
    return fail(AWQ_ERR_UNSUPPORTED, "packed layer exceeds the 4 GiB operand limit");
  hipError_t e = awq::launch_lowbit_repack(codes, scales, zeros, N, K, bits, group, codes_t,
                                           meta_t, stream);
  if (e != hipSuccess) return hip_fail(e, "lowbit repack launch");
  return AWQ_OK;
  AWQ_GUARD_END
}

size_t awq_lowbit_gemv_workspace_size(awq_dtype_t x_dtype, int64_t M, int64_t N, int64_t K) {
  if (!valid_dtype(x_dtype) || M < 1 || N < 1 || K < 32) return 0;
  return awq::lowbit_gemv_ws_bytes(x_dtype, M, N, K);
}

awq_status_t awq_lowbit_gemv(const void* X, awq_dtype_t x_dtype, int64_t M, int64_t K,
                             const uint32_t* codes_t, const void* meta_t, int64_t N, int bits,
                             int group, float* Y, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  AWQ_GUARD_BEGIN
  awq_status_t st = check_quant_args(x_dtype, N, K, bits, group);
  if (st != AWQ_OK) return st;
  if (M < 1) return fail(AWQ_ERR_INVALID_ARG, "M must be >= 1");
  if (!X || !codes_t || !meta_t || !Y) return fail(AWQ_ERR_INVALID_ARG, "null pointer");
  if (!aligned(X, 16) || !aligned(codes_t, 4) || !aligned(meta_t, 8) || !aligned(Y, 4))
    return fail(AWQ_ERR_UNSUPPORTED, "X 16-byte, codes_t and Y 4-byte, meta_t 8-byte aligned");
  const size_t need = awq::lowbit_gemv_ws_bytes(x_dtype, M, N, K);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(AWQ_ERR_WORKSPACE, "workspace of %zu bytes is below %zu", workspace_bytes, need);
  if (need > 0 && !aligned(workspace, 4))
    return fail(AWQ_ERR_WORKSPACE, "workspace must be 4-byte aligned");
  hipError_t e = awq::launch_lowbit_gemv(X, x_dtype, M, K, codes_t, meta_t, N, bits, group, Y,
                                         workspace, stream);
  if (e != hipSuccess) return hip_fail(e, "lowbit gemv launch");
  return AWQ_OK;
  AWQ_GUARD_END
}

awq_status_t awq_lowbit_gemv_noalloc(const void* X, awq_dtype_t x_dtype, int64_t M, int64_t K,
                                     const uint32_t* codes_t, const void* meta_t, int64_t N,
                                     int bits, int group, float* Y, hipStream_t stream) {
  AWQ_GUARD_BEGIN
  awq_status_t st = check_quant_args(x_dtype, N, K, bits, group);
  if (st != AWQ_OK) return st;
  if (M < 1) return fail(AWQ_ERR_INVALID_ARG, "M must be >= 1");
  if (!X || !codes_t || !meta_t || !Y) return fail(AWQ_ERR_INVALID_ARG, "null pointer");
  if (!aligned(X, 16) || !aligned(codes_t, 4) || !aligned(meta_t, 8) || !aligned(Y, 4))
    return fail(AWQ_ERR_UNSUPPORTED, "X 16-byte, codes_t and Y 4-byte, meta_t 8-byte aligned");
  const size_t need = awq::lowbit_gemv_ws_bytes(x_dtype, M, N, K);
  if (need > (size_t)AWQ_LOWBIT_STATIC_SCRATCH_BYTES)
    return fail(AWQ_ERR_UNSUPPORTED,
                "partial sums of %zu bytes exceed the static scratch of %u bytes (M=%lld N=%lld "
                "K=%lld); use awq_lowbit_gemv with a workspace",
                need, (unsigned)AWQ_LOWBIT_STATIC_SCRATCH_BYTES, (long long)M, (long long)N,
                (long long)K);
  void* ws = nullptr;
  if (need > 0) {
    hipError_t e = awq::lowbit_static_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "static scratch lookup");
  }
  hipError_t e = awq::launch_lowbit_gemv(X, x_dtype, M, K, codes_t, meta_t, N, bits, group, Y, ws,
                                         stream);
  if (e != hipSuccess) return hip_fail(e, "lowbit gemv launch");
  return AWQ_OK;
  AWQ_GUARD_END
}

awq_status_t awq_lowbit_gemm(const void* X, awq_dtype_t x_dtype, int64_t M, int64_t K,
                             const uint32_t* codes_t, const void* meta_t, int64_t N, int bits,
                             int group, float* Y, hipStream_t stream) {
  AWQ_GUARD_BEGIN
  awq_status_t st = check_quant_args(x_dtype, N, K, bits, group);
  if (st != AWQ_OK) return st;
  if (x_dtype != AWQ_F16 && x_dtype != AWQ_BF16)
    return fail(AWQ_ERR_UNSUPPORTED, "lowbit gemm takes fp16 or bf16 activations");
  if (M < 1) return fail(AWQ_ERR_INVALID_ARG, "M must be >= 1");
  if (M > kLowbitGemmMaxM)
    return fail(AWQ_ERR_UNSUPPORTED, "M=%lld above %lld", (long long)M, (long long)kLowbitGemmMaxM);
  if (K > kLowbitGemmMaxK)
    return fail(AWQ_ERR_UNSUPPORTED, "K=%lld above %lld", (long long)K, (long long)kLowbitGemmMaxK);
  if (!X || !codes_t || !meta_t || !Y) return fail(AWQ_ERR_INVALID_ARG, "null pointer");
  if (!aligned(X, 16) || !aligned(codes_t, 4) || !aligned(meta_t, 8) || !aligned(Y, 4))
    return fail(AWQ_ERR_UNSUPPORTED, "X 16-byte, codes_t and Y 4-byte, meta_t 8-byte aligned");
  hipError_t e = awq::launch_lowbit_gemm(X, x_dtype, M, K, codes_t, meta_t, N, bits, group, Y,
                                         stream);
  if (e != hipSuccess) return hip_fail(e, "lowbit gemm launch");
  return AWQ_OK;
  AWQ_GUARD_END
}

awq_status_t awq_quantize_pack(const void* W, awq_dtype_t w_dtype, int64_t N, int64_t K,
                               const float* s, int bits, int group, uint32_t* codes_out,
                               float* scales_out, uint8_t* zeros_out, hipStream_t stream) {
  AWQ_GUARD_BEGIN
  awq_status_t st = check_quant_args(w_dtype, N, K, bits, group);
  if (st != AWQ_OK) return st;
  if (!W || !s || !codes_out || !scales_out || !zeros_out)
    return fail(AWQ_ERR_INVALID_ARG, "null pointer");
  if (!aligned(W, 16) || !aligned(s, 16) || !aligned(codes_out, 4) || !aligned(scales_out, 4))
    return fail(AWQ_ERR_UNSUPPORTED, "W and s must be 16-byte aligned, codes and scales 4-byte");
  hipError_t e = awq::launch_quantize_pack(W, w_dtype, N, K, s, bits, group, codes_out, scales_out,
                                           zeros_out, stream);
  if (e != hipSuccess) return hip_fail(e, "quantize_pack launch");
  return AWQ_OK;
  AWQ_GUARD_END
}

awq_status_t awq_profile_enable(int enable) {
  g_prof_on.store(enable != 0);
  return AWQ_OK;
}

awq_status_t awq_profile_select(const char* prefix) {
  AWQ_GUARD_BEGIN
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_prefix = prefix ? prefix : "";
  return AWQ_OK;
  AWQ_GUARD_END
}

awq_status_t awq_profile_read(const char* prefix, int64_t* launches, double* total_ms) {
  AWQ_GUARD_BEGIN
  if (!launches || !total_ms) return fail(AWQ_ERR_INVALID_ARG, "null output");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  const size_t plen = prefix ? std::strlen(prefix) : 0;
  int64_t n = 0;
  double ms = 0.0;
  for (const ProfRec& r : g_prof) {
    if (plen && r.name.compare(0, plen, prefix) != 0) continue;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float t = 0.f;
    e = hipEventElapsedTime(&t, r.start, r.stop);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    ms += t;
    ++n;
  }
  *launches = n;
  *total_ms = ms;
  return AWQ_OK;
  AWQ_GUARD_END
}

awq_status_t awq_profile_reset(void) {
  AWQ_GUARD_BEGIN
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (ProfRec& r : g_prof) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_prof.clear();
  return AWQ_OK;
  AWQ_GUARD_END
}

}  // extern "C"
