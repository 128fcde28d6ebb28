// abi.cpp -- the C ABI of libdsa.so: argument validation, status codes and
// dispatch to the HIP launchers. Validation is pure host code and runs before
// any HIP call, so argument errors are reported even where no GPU exists.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "dsa.h"
#include "kernels.h"

static_assert(DSA_STATIC_SCRATCH_BYTES == dsa::kStaticScratchBytes,
              "the header's scratch size is the library's");

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#ifdef DSA_DEBUG
// Debug builds: wait for the call's kernels, then read (and clear) every
// kernel file's device check record; the first failure found is reported.
int debug_check(const char* fn) {
  const hipError_t se = hipDeviceSynchronize();
  if (se != hipSuccess)
    return fail(DSA_ERR_HIP, "%s: HIP error %d (%s) while running", fn, (int)se, hipGetErrorString(se));
  struct Src {
    const char* file;
    int (*take)(dsa::DebugRecord*);
  };
  const Src srcs[] = {{"attn_gather.hip", dsa::debug_take_attn_gather},
                      {"attn_prefill.hip", dsa::debug_take_attn_prefill},
                      {"index_fp8.hip", dsa::debug_take_index_fp8},
                      {"index_scores.hip", dsa::debug_take_index_scores},
                      {"prologue.hip", dsa::debug_take_prologue},
                      {"topk.hip", dsa::debug_take_topk}};
  int status = DSA_OK;
  for (const Src& s : srcs) {  // every record is read, so none carries over to the next call
    dsa::DebugRecord r;
    const int t = s.take(&r);
    if (status != DSA_OK) continue;
    if (t < 0) status = fail(DSA_ERR_HIP, "%s: reading the check record of %s failed", fn, s.file);
    if (t > 0)
      status = fail(DSA_ERR_CHECK, "%s: device check failed in %s line %d (values %lld, %lld); %u failed checks",
                    fn, s.file, r.line, r.a, r.b, r.count);
  }
  return status;
}
#endif

int hip_status(hipError_t e, const char* fn) {
  if (e != hipSuccess)
    return fail(DSA_ERR_HIP, "%s: HIP error %d (%s)", fn, (int)e, hipGetErrorString(e));
#ifdef DSA_DEBUG
  return debug_check(fn);
#else
  return DSA_OK;
#endif
}

bool finite_pos(float x) { return std::isfinite(x) && x > 0.0f; }

bool head_dim_ok(int d) { return d >= 16 && d <= DSA_MAX_HEAD_DIM && d % 16 == 0; }

// Query rows (B * S) any call takes: grids index rows (times a small factor)
// in 32 bits. 33.5 M rows is far beyond one GPU's HBM for these layers.
constexpr long long kMaxRows = DSA_MAX_ROWS;
bool rows_ok(int B, int S) { return (long long)B * S <= kMaxRows; }
// Attention heads: the prefill grid's second dimension holds one per head.
constexpr int kMaxHeads = DSA_MAX_HEADS;
// Keys and positions: kernels index keys in 32 bits with small offsets
// added, so T and past_len + S stay at or below 2^30 (2000x the longest
// context here).
constexpr int kMaxKeys = DSA_MAX_KEYS;
bool keys_ok(long long T) { return T <= kMaxKeys; }
// Index heads: products with the head count and dim stay in 32 bits.
constexpr int kMaxIndexHeads = DSA_MAX_INDEX_HEADS;

// Common checks of the attention entry points. Returns DSA_OK or a status.
int check_attn(const char* fn, const void* q, const void* k, const void* v, const void* gate,
               const void* out, int B, int S, int T, int H, int nope, int rope, int v_dim,
               float sm_scale, int gate_dim, int dtype) {
  if (!q || !k || !v || !out) return fail(DSA_ERR_INVALID_ARG, "%s: null input/output pointer", fn);
  if (B < 1 || S < 1 || T < 1 || H < 1)
    return fail(DSA_ERR_INVALID_ARG, "%s: B, S, T and H must be >= 1 (got %d, %d, %d, %d)", fn, B,
                S, T, H);
  if (nope < 0 || rope < 0 || nope + (long long)rope < 1 || v_dim < 1)
    return fail(DSA_ERR_INVALID_ARG, "%s: bad head dims (nope %d, rope %d, v %d)", fn, nope, rope,
                v_dim);
  if (nope > DSA_MAX_HEAD_DIM || rope > DSA_MAX_HEAD_DIM)  // (keeps nope + rope in range)
    return fail(DSA_ERR_UNSUPPORTED, "%s: head dims must be at most %d (nope %d, rope %d)", fn,
                DSA_MAX_HEAD_DIM, nope, rope);
  if (dtype != DSA_F32 && dtype != DSA_BF16)
    return fail(DSA_ERR_INVALID_ARG, "%s: dtype must be DSA_F32 or DSA_BF16 (got %d)", fn, dtype);
  if (!rows_ok(B, S))
    return fail(DSA_ERR_UNSUPPORTED, "%s: B*S above %lld", fn, kMaxRows);
  if (H > kMaxHeads) return fail(DSA_ERR_UNSUPPORTED, "%s: more than %d heads", fn, kMaxHeads);
  if (!keys_ok(T)) return fail(DSA_ERR_UNSUPPORTED, "%s: more than %d keys", fn, kMaxKeys);
  if (!finite_pos(sm_scale))
    return fail(DSA_ERR_INVALID_ARG, "%s: sm_scale must be finite and > 0", fn);
  if (gate_dim != 0 && gate_dim != 1 && gate_dim != v_dim)
    return fail(DSA_ERR_INVALID_ARG, "%s: gate_dim must be 0, 1 or v_dim (got %d)", fn, gate_dim);
  if (gate_dim != 0 && !gate) return fail(DSA_ERR_INVALID_ARG, "%s: gate is NULL", fn);
  if (!head_dim_ok(nope + rope) || !head_dim_ok(v_dim))
    return fail(DSA_ERR_UNSUPPORTED,
                "%s: head dims must be multiples of 16 in [16, %d] (qk %d, v %d)", fn,
                DSA_MAX_HEAD_DIM, nope + rope, v_dim);
  return DSA_OK;
}

int check_ws(const char* fn, void* ws, size_t have, size_t need) {
  if (need == 0) return DSA_OK;
  if (!ws || have < need)
    return fail(DSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given%s", fn, need, have,
                ws ? "" : " (NULL)");
  return DSA_OK;
}

// (the gather path lists the n_sink sinks as extra entries; the MFMA path
// runs them as extra key blocks and needs no more workspace)
// Path of a DSA prefill call. The dense-masked MFMA tiles cost in proportion
// to the keys each query can see (about T - S/2 when the caches end with the
// chunk); the row gather costs in proportion to the topk rows each query
// selects, at about 1 flop per byte. Measured on one MI355X (4096-query
// chunks, 32 heads, dims 192/128, topk 2048): 131072 cached keys 12.8 ms
// dense vs 23.7 ms gather, 262144 keys 25.8 vs 24.1 ms, 524288 keys 52.0 vs
// 25.8 ms; the ratio does not depend on the head count or dims. So the gather
// takes calls whose visible keys per query exceed 128 x topk. The rule reads
// only (S, T, topk) so that the size query and the call always agree.
constexpr double kGatherKeysPerSelected = 128.0;
bool prefill_uses_mfma(int dtype, int S, int T, int qk_dim, int v_dim, int topk) {
  if (!dsa::prefill_mfma_supported(dtype, S, qk_dim, v_dim)) return false;
  return (double)T - 0.5 * S < kGatherKeysPerSelected * topk;
}

size_t prefill_ws(int B, int S, int T, int H, int qk_dim, int v_dim, int topk, int dtype,
                  int n_sink) {
  if (prefill_uses_mfma(dtype, S, T, qk_dim, v_dim, topk))
    return dsa::prefill_mfma_workspace_bytes(B, S, T, H, v_dim);
  return dsa::gather_workspace_bytes((int64_t)B * S, H, v_dim, (int64_t)topk + n_sink);
}

size_t swa_ws(int B, int S, int H, int qk_dim, int v_dim, int window, int dtype, int n_sink) {
  if (dsa::prefill_mfma_supported(dtype, S, qk_dim, v_dim)) return 0;
  return dsa::gather_workspace_bytes((int64_t)B * S, H, v_dim, (int64_t)window + n_sink);
}

// Size queries return 0 for arguments their calls reject (those calls fail
// before they look at the workspace), and otherwise the exact requirement.
bool attn_sizes_ok(int B, int S, int H, int qk_dim, int v_dim, int n_sink, int dtype) {
  return B >= 1 && S >= 1 && H >= 1 && H <= kMaxHeads && rows_ok(B, S) && head_dim_ok(qk_dim) && head_dim_ok(v_dim) &&
         n_sink >= 0 && n_sink <= DSA_MAX_SINKS && (dtype == DSA_F32 || dtype == DSA_BF16);
}

int check_sinks(const char* fn, const void* sink_k, const void* sink_v, int n_sink) {
  if (n_sink < 0 || n_sink > DSA_MAX_SINKS)
    return fail(DSA_ERR_INVALID_ARG, "%s: n_sink must be in [0, %d] (got %d)", fn, DSA_MAX_SINKS,
                n_sink);
  if (n_sink > 0 && (!sink_k || !sink_v))
    return fail(DSA_ERR_INVALID_ARG, "%s: sink_k / sink_v is NULL with n_sink %d", fn, n_sink);
  return DSA_OK;
}

int prefill_impl(const char* fn, const void* q, const void* k_cache, const void* v_cache,
                 const void* sink_k, const void* sink_v, int n_sink, const int32_t* indices,
                 const void* gate, void* out, int B, int S, int T, int past_len, int H,
                 int qk_nope_dim, int qk_rope_dim, int v_dim, int topk, float sm_scale,
                 int gate_dim, int dtype, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  g_err.clear();
  int st = check_attn(fn, q, k_cache, v_cache, gate, out, B, S, T, H, qk_nope_dim, qk_rope_dim,
                      v_dim, sm_scale, gate_dim, dtype);
  if (st) return st;
  if ((st = check_sinks(fn, sink_k, sink_v, n_sink))) return st;
  if (!indices) return fail(DSA_ERR_INVALID_ARG, "%s: indices is NULL", fn);
  if (past_len < 0 || (long long)past_len + S > T)
    return fail(DSA_ERR_INVALID_ARG, "%s: need 0 <= past_len and past_len + S <= T", fn);
  if (topk < 1 || topk > T)
    return fail(DSA_ERR_INVALID_ARG, "%s: topk must be in [1, T] (topk %d, T %d)", fn, topk, T);
  if (topk > DSA_MAX_TOPK)
    return fail(DSA_ERR_UNSUPPORTED, "%s: topk %d > %d", fn, topk, DSA_MAX_TOPK);
  const int dqk = qk_nope_dim + qk_rope_dim;
  const bool mfma = prefill_uses_mfma(dtype, S, T, dqk, v_dim, topk);
  if (mfma && B > 65535) return fail(DSA_ERR_UNSUPPORTED, "%s: B > 65535", fn);
  if (!mfma && (long long)B * S > 0x7FFFFFFF / 64)
    return fail(DSA_ERR_UNSUPPORTED, "%s: B*S too large for the gather path", fn);
  st = check_ws(fn, workspace, workspace_bytes,
                prefill_ws(B, S, T, H, dqk, v_dim, topk, dtype, n_sink));
  if (st) return st;
  hipError_t e;
  if (mfma)
    e = dsa::launch_prefill_mfma(q, k_cache, v_cache, sink_k, sink_v, n_sink, indices, gate, out,
                                 B, S, T, past_len, 0, H, H, dqk, v_dim, topk, 0, sm_scale,
                                 gate_dim, workspace, stream);
  else
    e = dsa::launch_gather(q, k_cache, v_cache, sink_k, sink_v, n_sink, indices, gate, out, B, S,
                           T, past_len, 0, H, H, dqk, v_dim, topk, 0, sm_scale, gate_dim, dtype,
                           workspace, stream);
  return hip_status(e, fn);
}

int decode_impl(const char* fn, const void* q, const void* k_cache, const void* v_cache,
                const void* sink_k, const void* sink_v, int n_sink, const int32_t* indices,
                const void* gate, void* out, int B, int T, int H, int qk_nope_dim,
                int qk_rope_dim, int v_dim, int topk, float sm_scale, int gate_dim, int dtype,
                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  int st = check_attn(fn, q, k_cache, v_cache, gate, out, B, 1, T, H, qk_nope_dim, qk_rope_dim,
                      v_dim, sm_scale, gate_dim, dtype);
  if (st) return st;
  if ((st = check_sinks(fn, sink_k, sink_v, n_sink))) return st;
  if (!indices) return fail(DSA_ERR_INVALID_ARG, "%s: indices is NULL", fn);
  if (topk < 1 || topk > T)
    return fail(DSA_ERR_INVALID_ARG, "%s: topk must be in [1, T] (topk %d, T %d)", fn, topk, T);
  if (topk > DSA_MAX_TOPK)
    return fail(DSA_ERR_UNSUPPORTED, "%s: topk %d > %d", fn, topk, DSA_MAX_TOPK);
  st = check_ws(fn, workspace, workspace_bytes,
                dsa::gather_workspace_bytes(B, H, v_dim, (int64_t)topk + n_sink));
  if (st) return st;
  return hip_status(dsa::launch_gather(q, k_cache, v_cache, sink_k, sink_v, n_sink, indices, gate,
                                       out, B, 1, T, T - 1, 0, H, H, qk_nope_dim + qk_rope_dim, v_dim,
                                       topk, 0, sm_scale, gate_dim, dtype, workspace, stream),
                    fn);
}

int swa_impl(const char* fn, const void* q, const void* k_buf, const void* v_buf,
             const void* sink_k, const void* sink_v, int n_sink, const void* gate, void* out,
             int B, int S, int T_buf, int past_len, int kv_offset, int H, int H_kv,
             int qk_nope_dim, int qk_rope_dim, int v_dim, int window, float sm_scale,
             int gate_dim, int dtype, void* workspace, size_t workspace_bytes,
             hipStream_t stream) {
  g_err.clear();
  int st = check_attn(fn, q, k_buf, v_buf, gate, out, B, S, T_buf, H, qk_nope_dim, qk_rope_dim,
                      v_dim, sm_scale, gate_dim, dtype);
  if (st) return st;
  if (H_kv < 1 || H_kv > H || H % H_kv != 0)
    return fail(DSA_ERR_INVALID_ARG, "%s: kv heads must divide the query heads (H %d, H_kv %d)",
                fn, H, H_kv);
  if ((st = check_sinks(fn, sink_k, sink_v, n_sink))) return st;
  if (window < 1) return fail(DSA_ERR_INVALID_ARG, "%s: window must be >= 1", fn);
  if (past_len < 0 || kv_offset < 0)
    return fail(DSA_ERR_INVALID_ARG, "%s: past_len and kv_offset must be >= 0", fn);
  if (!keys_ok((long long)past_len + S))
    return fail(DSA_ERR_UNSUPPORTED, "%s: positions past_len + S above %d", fn, kMaxKeys);
  const long long lim = std::max(0LL, (long long)past_len - window + 1);
  if (kv_offset > lim)
    return fail(DSA_ERR_INVALID_ARG,
                "%s: kv_offset %d > max(0, past_len - window + 1) = %lld (window not in buffer)",
                fn, kv_offset, lim);
  if ((long long)T_buf != (long long)past_len + S - kv_offset)
    return fail(DSA_ERR_INVALID_ARG, "%s: T_buf (%d) must equal past_len + S - kv_offset (%lld)",
                fn, T_buf, (long long)past_len + S - kv_offset);
  const int dqk = qk_nope_dim + qk_rope_dim;
  const bool mfma = dsa::prefill_mfma_supported(dtype, S, dqk, v_dim);
  if (mfma && B > 65535) return fail(DSA_ERR_UNSUPPORTED, "%s: B > 65535", fn);
  if (!mfma && (long long)B * S > 0x7FFFFFFF / 64)
    return fail(DSA_ERR_UNSUPPORTED, "%s: B*S too large for the gather path", fn);
  // A window wider than the context selects the same keys as one of exactly
  // past_len + S: every query's window then starts at or before position 0.
  window = (int)std::min<long long>(window, (long long)past_len + S);
  st = check_ws(fn, workspace, workspace_bytes,
                swa_ws(B, S, H, dqk, v_dim, window, dtype, n_sink));
  if (st) return st;
  hipError_t e;
  if (mfma)
    e = dsa::launch_prefill_mfma(q, k_buf, v_buf, sink_k, sink_v, n_sink, nullptr, gate, out, B,
                                 S, T_buf, past_len, kv_offset, H, H_kv, dqk, v_dim, 0, window,
                                 sm_scale, gate_dim, nullptr, stream);
  else
    e = dsa::launch_gather(q, k_buf, v_buf, sink_k, sink_v, n_sink, nullptr, gate, out, B, S,
                           T_buf, past_len, kv_offset, H, H_kv, dqk, v_dim, 0, window, sm_scale,
                           gate_dim, dtype, workspace, stream);
  return hip_status(e, fn);
}

}  // namespace

extern "C" {

const char* dsa_status_string(int status) {
  switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
    case DSA_ERR_CHECK: return "DSA_ERR_CHECK";
    default: return "DSA_ERR_UNKNOWN";
  }
}

const char* dsa_last_error(void) { return g_err.c_str(); }

int dsa_debug_build(void) {
#ifdef DSA_DEBUG
  return 1;
#else
  return 0;
#endif
}

// Checks of the indexer's arguments (dsa_index_scores, dsa_index_topk).
static int check_index(const char* fn, const void* q_idx, const void* k_idx, const void* w,
                       const void* out, int B, int S, int T, int past_len, int n_idx_heads,
                       int idx_dim, float scale, int relu_mode, int dtype) {
  if (!q_idx || !k_idx || !w || !out) return fail(DSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (B < 1 || S < 1 || T < 1 || n_idx_heads < 1 || idx_dim < 1 || past_len < 0)
    return fail(DSA_ERR_INVALID_ARG, "%s: sizes must be >= 1 and past_len >= 0", fn);
  if ((long long)past_len + S > T)
    return fail(DSA_ERR_INVALID_ARG, "%s: T (%d) < past_len + S (%d + %d)", fn, T, past_len, S);
  if (!finite_pos(scale)) return fail(DSA_ERR_INVALID_ARG, "%s: scale must be finite and > 0", fn);
  if (relu_mode < DSA_RELU_PER_HEAD || relu_mode > DSA_RELU_POST_SUM)
    return fail(DSA_ERR_INVALID_ARG, "%s: bad relu_mode %d", fn, relu_mode);
  if (dtype != DSA_F32 && dtype != DSA_BF16)
    return fail(DSA_ERR_INVALID_ARG, "%s: bad dtype %d", fn, dtype);
  if (idx_dim != 32 && idx_dim != 64 && idx_dim != 128)
    return fail(DSA_ERR_UNSUPPORTED, "%s: idx_dim must be 32, 64 or 128 (got %d)", fn, idx_dim);
  if ((long long)B * S > 65535 && dtype == DSA_F32)
    return fail(DSA_ERR_UNSUPPORTED, "%s: fp32 path limited to B*S <= 65535", fn);
  if (!rows_ok(B, S)) return fail(DSA_ERR_UNSUPPORTED, "%s: B*S above %lld", fn, kMaxRows);
  if (n_idx_heads > kMaxIndexHeads)
    return fail(DSA_ERR_UNSUPPORTED, "%s: more than %d index heads", fn, kMaxIndexHeads);
  if (!keys_ok(T)) return fail(DSA_ERR_UNSUPPORTED, "%s: more than %d keys", fn, kMaxKeys);
  if (B > 65535) return fail(DSA_ERR_UNSUPPORTED, "%s: B > 65535", fn);
  return DSA_OK;
}

int dsa_index_scores(const void* q_idx, const void* k_idx, const void* w, float* scores, int B,
                     int S, int T, int past_len, int n_idx_heads, int idx_dim, float scale,
                     int relu_mode, int dtype, hipStream_t stream) {
  const char* fn = "dsa_index_scores";
  g_err.clear();
  const int st = check_index(fn, q_idx, k_idx, w, scores, B, S, T, past_len, n_idx_heads, idx_dim,
                             scale, relu_mode, dtype);
  if (st) return st;
  return hip_status(dsa::launch_index_scores(q_idx, k_idx, w, scores, B, S, T, past_len,
                                             n_idx_heads, idx_dim, scale, relu_mode, dtype,
                                             stream),
                    fn);
}

size_t dsa_index_topk_workspace_size(int B, int S, int T, int topk) {
  if (B < 1 || S < 1 || T < 1 || topk < 1 || topk > T || topk > DSA_MAX_TOPK || !rows_ok(B, S) ||
      !keys_ok(T))
    return 0;
  const size_t scores = ((size_t)B * S * T * sizeof(float) + 255) / 256 * 256;
  return scores + dsa::topk_workspace_bytes(B, S, T, topk);
}

int dsa_index_topk(const void* q_idx, const void* k_idx, const void* w, int32_t* indices, int B,
                   int S, int T, int past_len, int n_idx_heads, int idx_dim, float scale,
                   int relu_mode, int dtype, int topk, int sorted, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "dsa_index_topk";
  g_err.clear();
  int st = check_index(fn, q_idx, k_idx, w, indices, B, S, T, past_len, n_idx_heads, idx_dim,
                       scale, relu_mode, dtype);
  if (st) return st;
  if (topk < 1 || topk > T)
    return fail(DSA_ERR_INVALID_ARG, "%s: topk must be in [1, T] (topk %d, T %d)", fn, topk, T);
  if (topk > DSA_MAX_TOPK) return fail(DSA_ERR_UNSUPPORTED, "%s: topk %d > %d", fn, topk, DSA_MAX_TOPK);
  if (sorted != 0 && sorted != 1)
    return fail(DSA_ERR_INVALID_ARG, "%s: sorted must be 0 or 1 (got %d)", fn, sorted);
  st = check_ws(fn, workspace, workspace_bytes, dsa_index_topk_workspace_size(B, S, T, topk));
  if (st) return st;
  float* scores = (float*)workspace;
  void* tk = (char*)workspace + ((size_t)B * S * T * sizeof(float) + 255) / 256 * 256;
  // scores of t <= past_len + s only; the top-k reads no further
  const hipError_t e = dsa::launch_index_scores(q_idx, k_idx, w, scores, B, S, T, past_len,
                                                n_idx_heads, idx_dim, scale, relu_mode, dtype,
                                                stream, /*fill_masked=*/false);
  if (e != hipSuccess) return hip_status(e, fn);
  return hip_status(dsa::launch_topk(scores, indices, B, S, T, topk, tk, stream, sorted ? 0 : 1,
                                     past_len),
                    fn);
}

int dsa_index_quant_fp8(const void* x, uint8_t* codes, float* scales, long long rows, int dim,
                        int dtype, hipStream_t stream) {
  const char* fn = "dsa_index_quant_fp8";
  g_err.clear();
  if (!x || !codes || !scales) return fail(DSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (rows < 1 || dim < 1) return fail(DSA_ERR_INVALID_ARG, "%s: rows and dim must be >= 1", fn);
  if (dtype != DSA_F32 && dtype != DSA_BF16)
    return fail(DSA_ERR_INVALID_ARG, "%s: bad dtype %d", fn, dtype);
  if (dtype != DSA_BF16) return fail(DSA_ERR_UNSUPPORTED, "%s: bf16 input only", fn);
  if (dim != 32 && dim != 64 && dim != 128)
    return fail(DSA_ERR_UNSUPPORTED, "%s: dim must be 32, 64 or 128 (got %d)", fn, dim);
  return hip_status(dsa::launch_quant_fp8(x, codes, scales, rows, dim, stream), fn);
}

int dsa_index_scores_fp8(const uint8_t* q_codes, const float* q_scales, const uint8_t* k_codes,
                         const float* k_scales, const void* w, float* scores, int B, int S, int T,
                         int past_len, int n_idx_heads, int idx_dim, float scale, int relu_mode,
                         int dtype, hipStream_t stream) {
  const char* fn = "dsa_index_scores_fp8";
  g_err.clear();
  if (!q_codes || !q_scales || !k_codes || !k_scales || !w || !scores)
    return fail(DSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (B < 1 || S < 1 || T < 1 || n_idx_heads < 1 || idx_dim < 1 || past_len < 0)
    return fail(DSA_ERR_INVALID_ARG, "%s: sizes must be >= 1 and past_len >= 0", fn);
  if ((long long)past_len + S > T)
    return fail(DSA_ERR_INVALID_ARG, "%s: T (%d) < past_len + S (%d + %d)", fn, T, past_len, S);
  if (!finite_pos(scale)) return fail(DSA_ERR_INVALID_ARG, "%s: scale must be finite and > 0", fn);
  if (relu_mode < DSA_RELU_PER_HEAD || relu_mode > DSA_RELU_POST_SUM)
    return fail(DSA_ERR_INVALID_ARG, "%s: bad relu_mode %d", fn, relu_mode);
  if (dtype != DSA_F32 && dtype != DSA_BF16)
    return fail(DSA_ERR_INVALID_ARG, "%s: bad dtype %d", fn, dtype);
  if (dtype != DSA_BF16) return fail(DSA_ERR_UNSUPPORTED, "%s: bf16 weights only", fn);
  if (idx_dim != 128)
    return fail(DSA_ERR_UNSUPPORTED, "%s: idx_dim must be 128 (got %d)", fn, idx_dim);
  if (B > 65535) return fail(DSA_ERR_UNSUPPORTED, "%s: B > 65535", fn);
  if (!rows_ok(B, S)) return fail(DSA_ERR_UNSUPPORTED, "%s: B*S above %lld", fn, kMaxRows);
  if (n_idx_heads > kMaxIndexHeads)
    return fail(DSA_ERR_UNSUPPORTED, "%s: more than %d index heads", fn, kMaxIndexHeads);
  if (!keys_ok(T)) return fail(DSA_ERR_UNSUPPORTED, "%s: more than %d keys", fn, kMaxKeys);
  return hip_status(dsa::launch_index_scores_fp8(q_codes, q_scales, k_codes, k_scales, w, scores,
                                                 B, S, T, past_len, n_idx_heads, idx_dim, scale,
                                                 relu_mode, stream),
                    fn);
}

size_t dsa_indexer_prologue_workspace_size(int B, int S, int idx_dim) {
  if (B < 1 || S < 1 || (idx_dim != 64 && idx_dim != 128) || !rows_ok(B, S)) return 0;
  return (size_t)B * S * idx_dim * 2;  // the key projection before its LayerNorm (bf16)
}

int dsa_indexer_prologue(const void* q_lora, const void* hidden, const void* wq_b, const void* wk,
                         const void* k_norm_weight, const void* k_norm_bias,
                         const void* weights_proj, const float* rope_cos, const float* rope_sin,
                         void* q_idx, void* k_idx_cache, void* w, int B, int S, int T,
                         int past_len, int q_lora_rank, int hidden_dim, int n_idx_heads,
                         int idx_dim, int rope_dim, float ln_eps, int dtype, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "dsa_indexer_prologue";
  g_err.clear();
  if (!q_lora || !hidden || !wq_b || !wk || !k_norm_weight || !k_norm_bias || !weights_proj ||
      !q_idx || !k_idx_cache || !w)
    return fail(DSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (rope_dim > 0 && (!rope_cos || !rope_sin))
    return fail(DSA_ERR_INVALID_ARG, "%s: rope tables are NULL with rope_dim %d", fn, rope_dim);
  if (B < 1 || S < 1 || T < 1 || past_len < 0 || q_lora_rank < 1 || hidden_dim < 1 ||
      n_idx_heads < 1 || idx_dim < 1)
    return fail(DSA_ERR_INVALID_ARG, "%s: sizes must be >= 1 and past_len >= 0", fn);
  if ((long long)past_len + S > T)
    return fail(DSA_ERR_INVALID_ARG, "%s: T (%d) < past_len + S (%d + %d)", fn, T, past_len, S);
  if (rope_dim < 0 || rope_dim > idx_dim || rope_dim % 2 != 0)
    return fail(DSA_ERR_INVALID_ARG, "%s: rope_dim must be even and in [0, idx_dim]", fn);
  if (!(ln_eps > 0.0f) || !std::isfinite(ln_eps))
    return fail(DSA_ERR_INVALID_ARG, "%s: ln_eps must be finite and > 0", fn);
  if (dtype != DSA_F32 && dtype != DSA_BF16)
    return fail(DSA_ERR_INVALID_ARG, "%s: bad dtype %d", fn, dtype);
  if (dtype != DSA_BF16) return fail(DSA_ERR_UNSUPPORTED, "%s: bf16 only", fn);
  if (idx_dim != 64 && idx_dim != 128)
    return fail(DSA_ERR_UNSUPPORTED, "%s: idx_dim must be 64 or 128 (got %d)", fn, idx_dim);
  if (q_lora_rank % 32 != 0 || hidden_dim % 32 != 0)
    return fail(DSA_ERR_UNSUPPORTED, "%s: q_lora_rank and hidden_dim must be multiples of 32",
                fn);
  if ((long long)B * S > 0x7FFFFFFF / 128 || (long long)n_idx_heads * idx_dim > 0x7FFFFFFF / 128)
    return fail(DSA_ERR_UNSUPPORTED, "%s: sizes too large", fn);
  if (n_idx_heads > kMaxIndexHeads)
    return fail(DSA_ERR_UNSUPPORTED, "%s: more than %d index heads", fn, kMaxIndexHeads);
  if (!keys_ok(T)) return fail(DSA_ERR_UNSUPPORTED, "%s: more than %d keys", fn, kMaxKeys);
  int st = check_ws(fn, workspace, workspace_bytes,
                    dsa_indexer_prologue_workspace_size(B, S, idx_dim));
  if (st) return st;
  return hip_status(dsa::launch_indexer_prologue(q_lora, hidden, wq_b, wk, k_norm_weight,
                                                 k_norm_bias, weights_proj, rope_cos, rope_sin,
                                                 q_idx, k_idx_cache, w, B, S, T, past_len,
                                                 q_lora_rank, hidden_dim, n_idx_heads, idx_dim,
                                                 rope_dim, ln_eps, workspace, stream),
                    fn);
}

size_t dsa_mla_prologue_workspace_size(int B, int S, int kv_lora_rank) {
  if (B < 1 || S < 1 || kv_lora_rank < 32 || kv_lora_rank % 32 != 0 || !rows_ok(B, S)) return 0;
  return (size_t)B * S * kv_lora_rank * 2;  // the latent (bf16)
}

int dsa_mla_prologue(const void* q_resid, const void* q_compressed, const void* hidden,
                     const void* wq_gate, const void* wkv_a, const void* wkv_b,
                     const float* rope_cos, const float* rope_sin, void* q, void* gate,
                     void* k_cache, void* v_cache, int B, int S, int T, int past_len,
                     int q_resid_dim, int q_comp_dim, int hidden_dim, int kv_lora_rank, int H,
                     int qk_nope_dim, int qk_rope_dim, int v_dim, int dtype, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  const char* fn = "dsa_mla_prologue";
  g_err.clear();
  if (!q_resid || !q_compressed || !hidden || !wq_gate || !wkv_a || !wkv_b || !q || !gate ||
      !k_cache || !v_cache)
    return fail(DSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (qk_rope_dim > 0 && (!rope_cos || !rope_sin))
    return fail(DSA_ERR_INVALID_ARG, "%s: rope tables are NULL with qk_rope_dim %d", fn,
                qk_rope_dim);
  if (B < 1 || S < 1 || T < 1 || past_len < 0 || q_resid_dim < 1 || q_comp_dim < 1 ||
      hidden_dim < 1 || kv_lora_rank < 1 || H < 1 || qk_nope_dim < 0 || qk_rope_dim < 0 ||
      v_dim < 1 || qk_nope_dim + (long long)qk_rope_dim < 1)
    return fail(DSA_ERR_INVALID_ARG, "%s: sizes must be >= 1 (nope, rope >= 0) and past_len >= 0",
                fn);
  if ((long long)past_len + S > T)
    return fail(DSA_ERR_INVALID_ARG, "%s: T (%d) < past_len + S (%d + %d)", fn, T, past_len, S);
  if (dtype != DSA_F32 && dtype != DSA_BF16)
    return fail(DSA_ERR_INVALID_ARG, "%s: bad dtype %d", fn, dtype);
  if (dtype != DSA_BF16) return fail(DSA_ERR_UNSUPPORTED, "%s: bf16 only", fn);
  if (q_resid_dim % 32 || q_comp_dim % 32 || hidden_dim % 32 || kv_lora_rank % 32)
    return fail(DSA_ERR_UNSUPPORTED,
                "%s: q_resid_dim, q_comp_dim, hidden_dim and kv_lora_rank must be multiples of 32",
                fn);
  if (qk_nope_dim % 16 || qk_rope_dim % 16 || v_dim % 16 ||
      qk_nope_dim + qk_rope_dim > DSA_MAX_HEAD_DIM || v_dim > DSA_MAX_HEAD_DIM)
    return fail(DSA_ERR_UNSUPPORTED,
                "%s: head dims must be multiples of 16 with nope + rope and v at most %d", fn,
                DSA_MAX_HEAD_DIM);
  if (!rows_ok(B, S)) return fail(DSA_ERR_UNSUPPORTED, "%s: B*S above %lld", fn, kMaxRows);
  if (!keys_ok(T)) return fail(DSA_ERR_UNSUPPORTED, "%s: more than %d keys", fn, kMaxKeys);
  if (H > kMaxHeads) return fail(DSA_ERR_UNSUPPORTED, "%s: more than %d heads", fn, kMaxHeads);
  if ((long long)q_resid_dim + q_comp_dim > 0x7FFFFFFF / 256 || hidden_dim > 0x7FFFFFFF / 256 ||
      kv_lora_rank > 0x7FFFFFFF / 256)
    return fail(DSA_ERR_UNSUPPORTED, "%s: input widths too large", fn);
  int st = check_ws(fn, workspace, workspace_bytes,
                    dsa_mla_prologue_workspace_size(B, S, kv_lora_rank));
  if (st) return st;
  return hip_status(dsa::launch_mla_prologue(q_resid, q_compressed, hidden, wq_gate, wkv_a, wkv_b,
                                             rope_cos, rope_sin, q, gate, k_cache, v_cache, B, S,
                                             T, past_len, q_resid_dim, q_comp_dim, hidden_dim,
                                             kv_lora_rank, H, qk_nope_dim, qk_rope_dim, v_dim,
                                             workspace, stream),
                    fn);
}

size_t dsa_topk_workspace_size(int B, int S, int T, int topk) {
  // (sizes the call itself rejects need no workspace)
  if (B < 1 || S < 1 || T < 1 || topk < 1 || topk > T || topk > DSA_MAX_TOPK || !rows_ok(B, S) ||
      !keys_ok(T))
    return 0;
  return dsa::topk_workspace_bytes(B, S, T, topk);
}

static int topk_impl(const char* fn, const float* scores, int32_t* indices, int B, int S, int T,
                     int topk, void* workspace, size_t workspace_bytes, hipStream_t stream,
                     int order) {
  g_err.clear();
  if (!scores || !indices) return fail(DSA_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (B < 1 || S < 1 || T < 1) return fail(DSA_ERR_INVALID_ARG, "%s: sizes must be >= 1", fn);
  if (topk < 1 || topk > T)
    return fail(DSA_ERR_INVALID_ARG, "%s: topk must be in [1, T] (topk %d, T %d)", fn, topk, T);
  if (topk > DSA_MAX_TOPK)
    return fail(DSA_ERR_UNSUPPORTED, "%s: topk %d > %d", fn, topk, DSA_MAX_TOPK);
  if (!rows_ok(B, S)) return fail(DSA_ERR_UNSUPPORTED, "%s: B*S above %lld", fn, kMaxRows);
  if (!keys_ok(T)) return fail(DSA_ERR_UNSUPPORTED, "%s: more than %d keys", fn, kMaxKeys);
  int st = check_ws(fn, workspace, workspace_bytes, dsa::topk_workspace_bytes(B, S, T, topk));
  if (st) return st;
  return hip_status(dsa::launch_topk(scores, indices, B, S, T, topk, workspace, stream, order),
                    fn);
}

int dsa_topk(const float* scores, int32_t* indices, int B, int S, int T, int topk,
             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return topk_impl("dsa_topk", scores, indices, B, S, T, topk, workspace, workspace_bytes, stream,
                   0);
}

int dsa_topk_unsorted(const float* scores, int32_t* indices, int B, int S, int T, int topk,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return topk_impl("dsa_topk_unsorted", scores, indices, B, S, T, topk, workspace,
                   workspace_bytes, stream, 1);
}

size_t dsa_sparse_attn_prefill_workspace_size(int B, int S, int T, int H, int qk_dim, int v_dim,
                                              int topk, int dtype) {
  return dsa_sparse_attn_prefill_pas_workspace_size(B, S, T, H, qk_dim, v_dim, topk, 0, dtype);
}

size_t dsa_sparse_attn_prefill_pas_workspace_size(int B, int S, int T, int H, int qk_dim,
                                                  int v_dim, int topk, int n_sink, int dtype) {
  if (!attn_sizes_ok(B, S, H, qk_dim, v_dim, n_sink, dtype) || T < S || !keys_ok(T) ||
      topk < 1 || topk > T || topk > DSA_MAX_TOPK)
    return 0;
  return prefill_ws(B, S, T, H, qk_dim, v_dim, topk, dtype, n_sink);
}

int dsa_sparse_attn_prefill(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* indices, const void* gate, void* out, int B, int S,
                            int T, int past_len, int H, int qk_nope_dim, int qk_rope_dim,
                            int v_dim, int topk, float sm_scale, int gate_dim, int dtype,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return prefill_impl("dsa_sparse_attn_prefill", q, k_cache, v_cache, nullptr, nullptr, 0, indices,
                      gate, out, B, S, T, past_len, H, qk_nope_dim, qk_rope_dim, v_dim, topk,
                      sm_scale, gate_dim, dtype, workspace, workspace_bytes, stream);
}

int dsa_sparse_attn_prefill_pas(const void* q, const void* k_cache, const void* v_cache,
                                const void* sink_k, const void* sink_v, int n_sink,
                                const int32_t* indices, const void* gate, void* out, int B, int S,
                                int T, int past_len, int H, int qk_nope_dim, int qk_rope_dim,
                                int v_dim, int topk, float sm_scale, int gate_dim, int dtype,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return prefill_impl("dsa_sparse_attn_prefill_pas", q, k_cache, v_cache, sink_k, sink_v, n_sink,
                      indices, gate, out, B, S, T, past_len, H, qk_nope_dim, qk_rope_dim, v_dim,
                      topk, sm_scale, gate_dim, dtype, workspace, workspace_bytes, stream);
}

int dsa_prefill_work_plan(int B, int S, int T, int past_len, int H, int kv_offset, int window,
                          int* n_tiles, int* n_items, int* max_blocks, int* item_start, int cap) {
  const char* fn = "dsa_prefill_work_plan";
  g_err.clear();
  if (!n_tiles || !n_items || !max_blocks) return fail(DSA_ERR_INVALID_ARG, "%s: null output", fn);
  if (B < 1 || S < 1 || T < 1 || H < 1 || past_len < 0 || kv_offset < 0 ||
      (long long)past_len + S - kv_offset > T || (long long)past_len + S > 0x7FFFFFFF)
    return fail(DSA_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (!rows_ok(B, S)) return fail(DSA_ERR_UNSUPPORTED, "%s: B*S above %lld", fn, kMaxRows);
  if (!keys_ok(T) || !keys_ok((long long)past_len + S))
    return fail(DSA_ERR_UNSUPPORTED, "%s: more than %d keys", fn, kMaxKeys);
  dsa::prefill_work_plan(B, S, T, past_len, H, kv_offset, window, n_tiles, n_items, max_blocks,
                         item_start, cap);
  return DSA_OK;
}

size_t dsa_sparse_attn_decode_workspace_size(int B, int H, int v_dim, int topk) {
  return dsa_sparse_attn_decode_pas_workspace_size(B, H, v_dim, topk, 0);
}

size_t dsa_sparse_attn_decode_pas_workspace_size(int B, int H, int v_dim, int topk, int n_sink) {
  if (!attn_sizes_ok(B, 1, H, 16, v_dim, n_sink, DSA_BF16) || topk < 1 || topk > DSA_MAX_TOPK)
    return 0;
  return dsa::gather_workspace_bytes(B, H, v_dim, (int64_t)topk + n_sink);
}

int dsa_sparse_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* indices, const void* gate, void* out, int B, int T,
                           int H, int qk_nope_dim, int qk_rope_dim, int v_dim, int topk,
                           float sm_scale, int gate_dim, int dtype, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  return decode_impl("dsa_sparse_attn_decode", q, k_cache, v_cache, nullptr, nullptr, 0, indices,
                     gate, out, B, T, H, qk_nope_dim, qk_rope_dim, v_dim, topk, sm_scale,
                     gate_dim, dtype, workspace, workspace_bytes, stream);
}

int dsa_sparse_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* indices, const void* gate, void* out, int B,
                                   int T, int H, int qk_nope_dim, int qk_rope_dim, int v_dim,
                                   int topk, float sm_scale, int gate_dim, int dtype,
                                   hipStream_t stream) {
  const char* fn = "dsa_sparse_attn_decode_noalloc";
  g_err.clear();
  int st = check_attn(fn, q, k_cache, v_cache, gate, out, B, 1, T, H, qk_nope_dim, qk_rope_dim,
                      v_dim, sm_scale, gate_dim, dtype);
  if (st) return st;
  if (!indices) return fail(DSA_ERR_INVALID_ARG, "%s: indices is NULL", fn);
  if (topk < 1 || topk > T)
    return fail(DSA_ERR_INVALID_ARG, "%s: topk must be in [1, T] (topk %d, T %d)", fn, topk, T);
  if (topk > DSA_MAX_TOPK)
    return fail(DSA_ERR_UNSUPPORTED, "%s: topk %d > %d", fn, topk, DSA_MAX_TOPK);
  const size_t need = dsa::gather_workspace_bytes(B, H, v_dim, topk);
  if (need > DSA_STATIC_SCRATCH_BYTES)
    return fail(DSA_ERR_UNSUPPORTED,
                "%s: this call's partial states need %zu bytes; the static scratch holds %zu "
                "(use dsa_sparse_attn_decode with a workspace)",
                fn, need, (size_t)DSA_STATIC_SCRATCH_BYTES);
  void* ws = nullptr;
  hipError_t e = dsa::static_scratch(&ws);
  if (e != hipSuccess) return hip_status(e, fn);
  return hip_status(dsa::launch_gather(q, k_cache, v_cache, nullptr, nullptr, 0, indices, gate, out,
                                       B, 1, T, T - 1, 0, H, H, qk_nope_dim + qk_rope_dim, v_dim,
                                       topk, 0, sm_scale, gate_dim, dtype, ws, stream),
                    fn);
}

int dsa_sparse_attn_decode_pas(const void* q, const void* k_cache, const void* v_cache,
                               const void* sink_k, const void* sink_v, int n_sink,
                               const int32_t* indices, const void* gate, void* out, int B, int T,
                               int H, int qk_nope_dim, int qk_rope_dim, int v_dim, int topk,
                               float sm_scale, int gate_dim, int dtype, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  return decode_impl("dsa_sparse_attn_decode_pas", q, k_cache, v_cache, sink_k, sink_v, n_sink,
                     indices, gate, out, B, T, H, qk_nope_dim, qk_rope_dim, v_dim, topk, sm_scale,
                     gate_dim, dtype, workspace, workspace_bytes, stream);
}

size_t swa_attn_workspace_size(int B, int S, int H, int qk_dim, int v_dim, int window,
                               int dtype) {
  return swa_attn_pas_workspace_size(B, S, H, qk_dim, v_dim, window, 0, dtype);
}

size_t swa_attn_pas_workspace_size(int B, int S, int H, int qk_dim, int v_dim, int window,
                                   int n_sink, int dtype) {
  if (!attn_sizes_ok(B, S, H, qk_dim, v_dim, n_sink, dtype) || window < 1) return 0;
  return swa_ws(B, S, H, qk_dim, v_dim, window, dtype, n_sink);
}

int swa_attn(const void* q, const void* k_buf, const void* v_buf, const void* gate, void* out,
             int B, int S, int T_buf, int past_len, int kv_offset, int H, int qk_nope_dim,
             int qk_rope_dim, int v_dim, int window, float sm_scale, int gate_dim, int dtype,
             void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return swa_impl("swa_attn", q, k_buf, v_buf, nullptr, nullptr, 0, gate, out, B, S, T_buf,
                  past_len, kv_offset, H, H, qk_nope_dim, qk_rope_dim, v_dim, window, sm_scale,
                  gate_dim, dtype, workspace, workspace_bytes, stream);
}

int swa_attn_pas(const void* q, const void* k_buf, const void* v_buf, const void* sink_k,
                 const void* sink_v, int n_sink, const void* gate, void* out, int B, int S,
                 int T_buf, int past_len, int kv_offset, int H, int qk_nope_dim, int qk_rope_dim,
                 int v_dim, int window, float sm_scale, int gate_dim, int dtype, void* workspace,
                 size_t workspace_bytes, hipStream_t stream) {
  return swa_impl("swa_attn_pas", q, k_buf, v_buf, sink_k, sink_v, n_sink, gate, out, B, S, T_buf,
                  past_len, kv_offset, H, H, qk_nope_dim, qk_rope_dim, v_dim, window, sm_scale,
                  gate_dim, dtype, workspace, workspace_bytes, stream);
}

size_t swa_attn_gqa_workspace_size(int B, int S, int H, int qk_dim, int v_dim, int window,
                                   int dtype) {
  return swa_attn_pas_workspace_size(B, S, H, qk_dim, v_dim, window, 0, dtype);
}

int swa_attn_gqa(const void* q, const void* k_buf, const void* v_buf, const void* gate, void* out,
                 int B, int S, int T_buf, int past_len, int kv_offset, int H, int H_kv,
                 int qk_nope_dim, int qk_rope_dim, int v_dim, int window, float sm_scale,
                 int gate_dim, int dtype, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
  return swa_impl("swa_attn_gqa", q, k_buf, v_buf, nullptr, nullptr, 0, gate, out, B, S, T_buf,
                  past_len, kv_offset, H, H_kv, qk_nope_dim, qk_rope_dim, v_dim, window, sm_scale,
                  gate_dim, dtype, workspace, workspace_bytes, stream);
}

}  // extern "C"
