// C ABI of the verification-attention library: argument validation, workspace
// sizing and kernel launches.  Validation touches no HIP API, so every error
// path can be exercised on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "sv.h"
#include "sv_internal.h"

namespace {

thread_local char g_err[512] = "";
thread_local void* g_ev_start = nullptr;
thread_local void* g_ev_stop = nullptr;

sv_status fail(sv_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

sv_status ok() {
  g_err[0] = '\0';
  return SV_OK;
}

sv_status check_heads(int Hq, int Hkv, int D) {
  if (Hq <= 0 || Hkv <= 0) return fail(SV_E_INVALID, "Hq (%d) and Hkv (%d) must be positive", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(SV_E_INVALID, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (D != 64 && D != 128) return fail(SV_E_UNSUPPORTED, "head dim %d not supported (64 or 128)", D);
  return SV_OK;
}

sv_status check_kv(const sv_kv_cache* kv, int B) {
  if (!kv) return fail(SV_E_INVALID, "kv is NULL");
  if (!kv->k || !kv->v) return fail(SV_E_INVALID, "kv.k / kv.v is NULL");
  if (kv->num_slots <= 0) return fail(SV_E_INVALID, "kv.num_slots must be positive");
  if (kv->page_table) {
    if (kv->page_size <= 0) return fail(SV_E_INVALID, "kv.page_size must be >= 1 for a paged cache");
    if (kv->max_pages <= 0) return fail(SV_E_INVALID, "kv.max_pages must be >= 1 for a paged cache");
  } else {
    if (kv->seq_stride < 0) return fail(SV_E_INVALID, "kv.seq_stride must be >= 0");
    if (B > 1 && kv->seq_stride == 0) return fail(SV_E_INVALID, "kv.seq_stride is 0 with B > 1");
  }
  return SV_OK;
}

sv_status check_dtype(sv_dtype dt) {
  if (dt != SV_F32 && dt != SV_BF16) return fail(SV_E_UNSUPPORTED, "dtype %d not supported", (int)dt);
  return SV_OK;
}

float resolve_scale(float s, int D) { return s > 0.f ? s : 1.0f / sqrtf((float)D); }

sv::KvArgs kv_args(const sv_kv_cache* kv) {
  return sv::KvArgs{kv->k, kv->v, kv->page_table, kv->page_size, kv->max_pages,
                    (long long)kv->seq_stride, (long long)kv->num_slots};
}

sv_status hip_status(int e, const char* what) {
  if (e != 0) return fail(SV_E_HIP, "%s: %s", what, hipGetErrorString((hipError_t)e));
  return ok();
}

}  // namespace

namespace sv {
sv_status set_error(sv_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}
}  // namespace sv

extern "C" {

int sv_abi_version(void) { return SV_ABI_VERSION; }

const char* sv_last_error(void) { return g_err; }

sv_status sv_set_verify_timing_events(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(SV_E_INVALID, "timing events must be both set or both NULL");
  g_ev_start = start_event;
  g_ev_stop = stop_event;
  return ok();
}

size_t sv_verify_workspace_size(int B, int N, int Hq, int Hkv, int D, int P_max, sv_dtype dtype,
                                int is_tree, int n_score_rows, int page_size) {
  if (B <= 0 || N <= 0 || N > sv::kMaxNodes || Hq <= 0 || Hkv <= 0 || Hq % Hkv || (D != 64 && D != 128) ||
      P_max < 0 || n_score_rows < 0 || page_size < 0)
    return 0;
  return sv::plan_verify(B, N, Hq, Hkv, D, P_max, (int)dtype, is_tree != 0, n_score_rows, page_size).bytes;
}

}  // extern "C"

namespace {

sv_status verify_common(const void* q, sv_dtype dtype, int B, int N, int Hq, int Hkv, int D, const sv_kv_cache* kv,
                        const int32_t* prefix_len, int P_max, const int32_t* parent, const int32_t* score_rows_host,
                        int n_score_rows, float softmax_scale, void* out, float* scores, void* workspace,
                        size_t workspace_bytes, sv_stream stream, int head_scores,
                        const sv::SelectArgs* sel = nullptr) {
  sv_status st;
  if ((st = check_dtype(dtype))) return st;
  if (B < 0) return fail(SV_E_INVALID, "B must be >= 0");
  if (N <= 0) return fail(SV_E_INVALID, "N must be >= 1");
  if (N > sv::kMaxNodes) return fail(SV_E_UNSUPPORTED, "N = %d verify nodes exceeds %d", N, sv::kMaxNodes);
  if ((st = check_heads(Hq, Hkv, D))) return st;
  if (P_max < 0) return fail(SV_E_INVALID, "P_max must be >= 0");
  if (!(softmax_scale >= 0.f) || isinf(softmax_scale)) return fail(SV_E_INVALID, "softmax_scale must be finite and >= 0");
  if (n_score_rows < 0 || n_score_rows > N) return fail(SV_E_INVALID, "n_score_rows = %d not in [0, N]", n_score_rows);
  if (n_score_rows > 0) {
    if (!score_rows_host) return fail(SV_E_INVALID, "score_rows_host is NULL");
    if (!scores) return fail(SV_E_INVALID, "scores is NULL but n_score_rows > 0");
    unsigned char seen[sv::kMaxNodes] = {0};
    for (int i = 0; i < n_score_rows; ++i) {
      const int t = score_rows_host[i];
      if (t < 0 || t >= N) return fail(SV_E_INVALID, "score row %d = %d not in [0, N)", i, t);
      if (seen[t]) return fail(SV_E_INVALID, "score row %d listed twice", t);
      seen[t] = 1;
    }
  }
  if (B == 0) return ok();
  if (!q || !out || !prefix_len) return fail(SV_E_INVALID, "q, out and prefix_len must be non-NULL");
  if ((st = check_kv(kv, B))) return st;
  const sv::VerifyPlan p = sv::plan_verify(B, N, Hq, Hkv, D, P_max, (int)dtype, parent != nullptr, n_score_rows,
                                           kv->page_table ? kv->page_size : 0);
  const size_t need = sel ? sv::align_up(p.bytes) + sv::select_workspace_bytes(B) : p.bytes;
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(SV_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, need);
  sv::SelectArgs sa{};
  if (sel) {
    sa = *sel;
    sa.ws = reinterpret_cast<char*>(workspace) + sv::align_up(p.bytes);
  }
  const int e = sv::launch_verify(p, q, kv_args(kv), prefix_len, parent, score_rows_host, n_score_rows,
                                  resolve_scale(softmax_scale, D), out, scores, workspace, stream, g_ev_start,
                                  g_ev_stop, 0, head_scores, sel ? &sa : nullptr);
  return hip_status(e, sel ? "sv_verify_select launch" : "sv_verify_attn launch");
}

}  // namespace

extern "C" {

sv_status sv_verify_attn(const void* q, sv_dtype dtype, int B, int N, int Hq, int Hkv, int D,
                         const sv_kv_cache* kv, const int32_t* prefix_len, int P_max,
                         const int32_t* parent, const int32_t* score_rows_host, int n_score_rows,
                         float softmax_scale, void* out, float* scores, void* workspace,
                         size_t workspace_bytes, sv_stream stream) {
  return verify_common(q, dtype, B, N, Hq, Hkv, D, kv, prefix_len, P_max, parent, score_rows_host, n_score_rows,
                       softmax_scale, out, scores, workspace, workspace_bytes, stream, 0);
}

sv_status sv_verify_attn_per_head(const void* q, sv_dtype dtype, int B, int N, int Hq, int Hkv, int D,
                                  const sv_kv_cache* kv, const int32_t* prefix_len, int P_max,
                                  const int32_t* parent, const int32_t* score_rows_host, int n_score_rows,
                                  float softmax_scale, void* out, float* head_scores, void* workspace,
                                  size_t workspace_bytes, sv_stream stream) {
  return verify_common(q, dtype, B, N, Hq, Hkv, D, kv, prefix_len, P_max, parent, score_rows_host, n_score_rows,
                       softmax_scale, out, head_scores, workspace, workspace_bytes, stream, 1);
}

size_t sv_verify_select_workspace_size(int B, int N, int Hq, int Hkv, int D, int P_max, sv_dtype dtype, int is_tree,
                                       int n_score_rows, int page_size) {
  const size_t v = sv_verify_workspace_size(B, N, Hq, Hkv, D, P_max, dtype, is_tree, n_score_rows, page_size);
  if (v == 0 || n_score_rows <= 0 || P_max > sv::kSelectMaxP) return 0;
  return sv::align_up(v) + sv::select_workspace_bytes(B);
}

sv_status sv_verify_select(const void* q, sv_dtype dtype, int B, int N, int Hq, int Hkv, int D,
                           const sv_kv_cache* kv, const int32_t* prefix_len, int P_max, const int32_t* parent,
                           const int32_t* score_rows_host, int n_score_rows, float softmax_scale, const int32_t* k,
                           int k_max, void* out, float* scores, int32_t* idx, int32_t* count, void* workspace,
                           size_t workspace_bytes, sv_stream stream) {
  if (n_score_rows <= 0) return fail(SV_E_INVALID, "sv_verify_select needs score rows (n_score_rows >= 1)");
  if (k_max < 0) return fail(SV_E_INVALID, "k_max must be >= 0");
  if (P_max > sv::kSelectMaxP)
    return fail(SV_E_UNSUPPORTED, "sv_verify_select takes prefixes up to %d (P_max = %d): use sv_verify_attn and "
                "sv_topk_select", sv::kSelectMaxP, P_max);
  if (B > 0 && (!k || (!idx && k_max > 0))) return fail(SV_E_INVALID, "k and idx must be non-NULL");
  const sv::SelectArgs sel{k, k_max, idx, count, nullptr};
  return verify_common(q, dtype, B, N, Hq, Hkv, D, kv, prefix_len, P_max, parent, score_rows_host, n_score_rows,
                       softmax_scale, out, scores, workspace, workspace_bytes, stream, 0, &sel);
}

size_t sv_topk_workspace_size(int B, int P_max) {
  if (B <= 0 || P_max < 0 || !sv::topk_supported(P_max)) return 0;
  return sv::topk_workspace_bytes(B, P_max);
}

sv_status sv_topk_select(const float* scores, int B, int P_max, const int32_t* prefix_len, const int32_t* k,
                         int k_max, int32_t* idx, int32_t* count, void* workspace, size_t workspace_bytes,
                         sv_stream stream) {
  if (B < 0 || P_max < 0 || k_max < 0) return fail(SV_E_INVALID, "B, P_max and k_max must be >= 0");
  if (B == 0) return ok();
  if (!scores || !prefix_len || !k || (!idx && k_max > 0))
    return fail(SV_E_INVALID, "scores, prefix_len, k and idx must be non-NULL");
  const size_t need = sv::topk_workspace_bytes(B, P_max);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(SV_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, need);
  return hip_status(sv::launch_topk(scores, B, P_max, prefix_len, k, k_max, idx, count, workspace, stream),
                    "sv_topk_select launch");
}

size_t sv_sparse_workspace_size(int B, int Hq, int Hkv, int D, int max_idx) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || (D != 64 && D != 128) || max_idx < 0) return 0;
  return sv::plan_sparse(B, Hq, Hkv, D, max_idx).bytes;
}

}  // extern "C"

namespace {

sv_status sparse_common(const void* q, sv_dtype dtype, int B, int Hq, int Hkv, int D, const sv_kv_cache* kv,
                        const int32_t* idx, int idx_stride, const int32_t* n_idx, int max_idx, float softmax_scale,
                        void* out, void* workspace, size_t workspace_bytes, sv_stream stream, int per_head) {
  sv_status st;
  if ((st = check_dtype(dtype))) return st;
  if (B < 0) return fail(SV_E_INVALID, "B must be >= 0");
  if ((st = check_heads(Hq, Hkv, D))) return st;
  if (Hq / Hkv > 16) return fail(SV_E_UNSUPPORTED, "more than 16 query heads per KV head");
  if (max_idx < 0 || idx_stride < max_idx) return fail(SV_E_INVALID, "need 0 <= max_idx <= idx_stride");
  if (!(softmax_scale >= 0.f) || isinf(softmax_scale)) return fail(SV_E_INVALID, "softmax_scale must be finite and >= 0");
  if (B == 0) return ok();
  if (!q || !out || !n_idx || (!idx && max_idx > 0)) return fail(SV_E_INVALID, "q, out, idx and n_idx must be non-NULL");
  if ((st = check_kv(kv, B))) return st;
  const sv::SparsePlan p = sv::plan_sparse(B, Hq, Hkv, D, max_idx);
  if (p.bytes > 0 && (!workspace || workspace_bytes < p.bytes))
    return fail(SV_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, p.bytes);
  return hip_status(sv::launch_sparse(p, (int)dtype, q, kv_args(kv), idx, idx_stride, n_idx,
                                      resolve_scale(softmax_scale, D), out, workspace, stream, per_head),
                    "sv_sparse_draft_attn launch");
}

}  // namespace

extern "C" {

sv_status sv_sparse_draft_attn(const void* q, sv_dtype dtype, int B, int Hq, int Hkv, int D,
                               const sv_kv_cache* kv, const int32_t* idx, int idx_stride, const int32_t* n_idx,
                               int max_idx, float softmax_scale, void* out, void* workspace,
                               size_t workspace_bytes, sv_stream stream) {
  return sparse_common(q, dtype, B, Hq, Hkv, D, kv, idx, idx_stride, n_idx, max_idx, softmax_scale, out, workspace,
                       workspace_bytes, stream, 0);
}

sv_status sv_sparse_draft_attn_per_head(const void* q, sv_dtype dtype, int B, int Hq, int Hkv, int D,
                                        const sv_kv_cache* kv, const int32_t* idx, int idx_stride,
                                        const int32_t* n_idx, int max_idx, float softmax_scale, void* out,
                                        void* workspace, size_t workspace_bytes, sv_stream stream) {
  return sparse_common(q, dtype, B, Hq, Hkv, D, kv, idx, idx_stride, n_idx, max_idx, softmax_scale, out, workspace,
                       workspace_bytes, stream, 1);
}

sv_status sv_select_sink_window(int B, int P_max, const int32_t* prefix_len, int sink, int window, int k_max,
                                int32_t* idx, int32_t* count, sv_stream stream) {
  if (B < 0 || P_max < 0) return fail(SV_E_INVALID, "B and P_max must be >= 0");
  if (sink < 0 || window < 0) return fail(SV_E_INVALID, "sink and window must be >= 0");
  if (k_max < sink + window) return fail(SV_E_INVALID, "k_max = %d is smaller than sink + window = %d", k_max,
                                         sink + window);
  if (B == 0) return ok();
  if (!prefix_len || (!idx && k_max > 0)) return fail(SV_E_INVALID, "prefix_len and idx must be non-NULL");
  return hip_status(sv::launch_sink_window(B, P_max, prefix_len, sink, window, k_max, idx, count, stream),
                    "sv_select_sink_window launch");
}

sv_status sv_compact_kv(sv_dtype dtype, int B, int Hkv, int D, const sv_kv_cache* kv, const int32_t* idx,
                        int idx_stride, const int32_t* n_idx, int max_idx, void* ck, void* cv, int cap,
                        sv_stream stream) {
  sv_status st;
  if ((st = check_dtype(dtype))) return st;
  if (B < 0) return fail(SV_E_INVALID, "B must be >= 0");
  if ((st = check_heads(Hkv, Hkv, D))) return st;
  if (max_idx < 0 || idx_stride < max_idx) return fail(SV_E_INVALID, "need 0 <= max_idx <= idx_stride");
  if (cap < 1) return fail(SV_E_INVALID, "cap must be >= 1");
  if (B == 0) return ok();
  if (!n_idx || !ck || !cv || (!idx && max_idx > 0)) return fail(SV_E_INVALID, "idx, n_idx, ck and cv must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(ck) | reinterpret_cast<uintptr_t>(cv)) & 15)
    return fail(SV_E_INVALID, "ck and cv must be 16-byte aligned");
  if ((st = check_kv(kv, B))) return st;
  return hip_status(sv::launch_compact((int)dtype, B, Hkv, D, kv_args(kv), idx, idx_stride, n_idx, max_idx, ck, cv,
                                       cap, stream),
                    "sv_compact_kv launch");
}

size_t sv_dense_draft_workspace_size(int B, int Hq, int Hkv, int D, int cap, sv_dtype dtype) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || (D != 64 && D != 128) || cap < 1 ||
      (dtype != SV_F32 && dtype != SV_BF16))
    return 0;
  return sv::plan_verify(B, 1, Hq, Hkv, D, cap - 1, (int)dtype, false, 0, 0).bytes;
}

sv_status sv_dense_draft_attn(const void* q, sv_dtype dtype, int B, int Hq, int Hkv, int D, const void* ck,
                              const void* cv, int cap, const int32_t* n_rows, float softmax_scale, void* out,
                              void* workspace, size_t workspace_bytes, sv_stream stream) {
  sv_status st;
  if ((st = check_dtype(dtype))) return st;
  if (B < 0) return fail(SV_E_INVALID, "B must be >= 0");
  if ((st = check_heads(Hq, Hkv, D))) return st;
  if (cap < 1) return fail(SV_E_INVALID, "cap must be >= 1");
  if (!(softmax_scale >= 0.f) || isinf(softmax_scale)) return fail(SV_E_INVALID, "softmax_scale must be finite and >= 0");
  if (B == 0) return ok();
  if (!q || !out || !ck || !cv || !n_rows) return fail(SV_E_INVALID, "q, out, ck, cv and n_rows must be non-NULL");
  // the dense buffers are a contiguous cache with cap slots per sequence; the
  // decode is verification of N = 1 query whose prefix is its first n - 1 rows
  const sv::VerifyPlan p = sv::plan_verify(B, 1, Hq, Hkv, D, cap - 1, (int)dtype, false, 0, 0);
  if (p.bytes > 0 && (!workspace || workspace_bytes < p.bytes))
    return fail(SV_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required", workspace_bytes, p.bytes);
  const sv::KvArgs kv{ck, cv, nullptr, 1, 0, (long long)cap, (long long)B * cap};
  const int e = sv::launch_verify(p, q, kv, n_rows, nullptr, nullptr, 0, resolve_scale(softmax_scale, D), out,
                                  nullptr, workspace, stream, nullptr, nullptr, -1);
  return hip_status(e, "sv_dense_draft_attn launch");
}

sv_status sv_accept_commit(sv_dtype dtype, int B, int N, int Hkv, int D, const sv_kv_cache* kv,
                           const int32_t* prefix_len, int P_max, const int32_t* parent, const int32_t* draft_tokens,
                           const int32_t* target_tokens, int32_t* path, int32_t* n_accepted, int32_t* bonus,
                           int32_t* new_prefix_len, sv_stream stream) {
  sv_status st;
  if (B < 0) return fail(SV_E_INVALID, "B must be >= 0");
  if (N <= 0) return fail(SV_E_INVALID, "N must be >= 1");
  if (N > sv::kMaxNodes) return fail(SV_E_UNSUPPORTED, "N = %d draft nodes exceeds %d", N, sv::kMaxNodes);
  if (P_max < 0) return fail(SV_E_INVALID, "P_max must be >= 0");
  if (kv) {
    if ((st = check_dtype(dtype))) return st;
    if ((st = check_heads(Hkv, Hkv, D))) return st;
  }
  if (B == 0) return ok();
  if (!draft_tokens || !target_tokens || !path || !n_accepted)
    return fail(SV_E_INVALID, "draft_tokens, target_tokens, path and n_accepted must be non-NULL");
  if ((kv || new_prefix_len) && !prefix_len) return fail(SV_E_INVALID, "prefix_len is NULL");
  sv::KvArgs ka{};
  if (kv) {
    if ((st = check_kv(kv, B))) return st;
    ka = kv_args(kv);
  }
  return hip_status(sv::launch_accept((int)dtype, B, N, Hkv, D, kv ? &ka : nullptr, prefix_len, P_max, parent,
                                      draft_tokens, target_tokens, path, n_accepted, bonus, new_prefix_len, stream),
                    "sv_accept_commit launch");
}

sv_status sv_build_tree(int B, int n_nodes, int max_depth, int n_cand, const double* logprobs, int32_t* parent,
                        int32_t* depth, int32_t* rank, sv_stream stream) {
  if (B < 0) return fail(SV_E_INVALID, "B must be >= 0");
  if (n_nodes < 1) return fail(SV_E_INVALID, "n_nodes must be >= 1");
  if (n_nodes > sv::kMaxNodes) return fail(SV_E_UNSUPPORTED, "n_nodes = %d exceeds %d", n_nodes, sv::kMaxNodes);
  if (n_cand < 1 || n_cand > 256) return fail(SV_E_UNSUPPORTED, "n_cand = %d not in [1, 256]", n_cand);
  if (max_depth < 0) return fail(SV_E_INVALID, "max_depth must be >= 0");
  // nodes reachable within the depth limit (saturating): the budget must fit
  long long reach = 1, level = 1;
  for (int d = 1; d <= max_depth && reach < n_nodes; ++d) {
    level = level * n_cand > (1LL << 20) ? (1LL << 20) : level * n_cand;
    reach += level;
  }
  if (reach < n_nodes)
    return fail(SV_E_INVALID, "only %lld nodes are reachable with n_cand = %d and max_depth = %d", reach, n_cand,
                max_depth);
  if (B == 0) return ok();
  if (!logprobs || !parent) return fail(SV_E_INVALID, "logprobs and parent must be non-NULL");
  return hip_status(sv::launch_build_tree(B, n_nodes, max_depth, n_cand, logprobs, parent, depth, rank, stream),
                    "sv_build_tree launch");
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Contract checks of device arrays (debugging aids; asynchronous, allocate nothing).

namespace {
sv_status check_err_ptr(const int32_t* err) {
  if (!err) return fail(SV_E_INVALID, "err must be a device int32[4]");
  if (reinterpret_cast<uintptr_t>(err) & 3) return fail(SV_E_INVALID, "err must be 4-byte aligned");
  return SV_OK;
}
}  // namespace

extern "C" sv_status sv_validate_kv(int B, int N, const sv_kv_cache* kv, const int32_t* prefix_len, int P_max,
                                    int32_t* err, sv_stream stream) {
  sv_status st;
  if ((st = check_err_ptr(err))) return st;
  if (B < 0 || N < 0 || P_max < 0) return fail(SV_E_INVALID, "B, N and P_max must be >= 0");
  if (B > 65535) return fail(SV_E_UNSUPPORTED, "B > 65535");
  if (B > 0 && !prefix_len) return fail(SV_E_INVALID, "prefix_len is NULL");
  if ((st = check_kv(kv, B))) return st;
  return hip_status(sv::launch_validate_kv(B, N, kv_args(kv), prefix_len, P_max, err, stream), "sv_validate_kv launch");
}

extern "C" sv_status sv_validate_tree(int B, int N, const int32_t* parent, int32_t* err, sv_stream stream) {
  sv_status st;
  if ((st = check_err_ptr(err))) return st;
  if (B < 0 || N < 0) return fail(SV_E_INVALID, "B and N must be >= 0");
  if (B > 65535) return fail(SV_E_UNSUPPORTED, "B > 65535");
  if (B > 0 && N > 0 && !parent) return fail(SV_E_INVALID, "parent is NULL");
  return hip_status(sv::launch_validate_tree(B, N, parent, err, stream), "sv_validate_tree launch");
}

extern "C" sv_status sv_validate_index(int B, int lists_per_seq, const sv_kv_cache* kv, const int32_t* idx,
                                       int idx_stride, const int32_t* n_idx, int max_idx, int32_t* err,
                                       sv_stream stream) {
  sv_status st;
  if ((st = check_err_ptr(err))) return st;
  if (B < 0 || lists_per_seq < 1) return fail(SV_E_INVALID, "need B >= 0 and lists_per_seq >= 1");
  if (max_idx < 0 || idx_stride < max_idx) return fail(SV_E_INVALID, "need 0 <= max_idx <= idx_stride");
  const long long lists = (long long)B * lists_per_seq;
  if (lists > 65535) return fail(SV_E_UNSUPPORTED, "more than 65535 index lists");
  if (lists > 0 && (!n_idx || (!idx && max_idx > 0))) return fail(SV_E_INVALID, "idx and n_idx must be non-NULL");
  if ((st = check_kv(kv, B))) return st;
  return hip_status(sv::launch_validate_index((int)lists, lists_per_seq, kv_args(kv), idx, idx_stride, n_idx, max_idx,
                                              err, stream),
                    "sv_validate_index launch");
}
