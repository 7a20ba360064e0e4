/*
 * sv.h -- C ABI of the verification-attention hot path for MI355X (gfx950).
 *
 * One speculative-decoding iteration on one attention layer:
 *
 *   sv_verify_attn        full (dense) attention of the N verify queries of each
 *                         sequence -- a linear draft chain or a draft tree whose
 *                         nodes see only the prefix, their ancestors and
 *                         themselves -- over the KV cache, plus one fp32
 *                         criticality score per prefix entry: the pre-softmax
 *                         logits summed over the chosen scoring rows and over
 *                         all query heads.
 *   sv_topk_select        the k highest-scoring prefix entries of each sequence.
 *   sv_sparse_draft_attn  the next draft step's decode attention restricted to
 *                         a gathered index set.
 *   sv_compact_kv, sv_dense_draft_attn   the same draft steps over the set
 *                         gathered once into dense buffers, plus a tail of
 *                         drafted tokens' rows.
 *   sv_verify_attn_per_head, sv_sparse_draft_attn_per_head, sv_select_sink_window
 *                         selection variants: one key set per KV head, and a
 *                         sink + recent-window baseline.
 *   sv_build_tree         best-first draft tree (parent array) from per-depth
 *                         draft log-probabilities.
 *   sv_validate_kv, sv_validate_tree, sv_validate_index   checks of the
 *                         device-array contract (debugging aids).
 *   sv_accept_commit      greedy acceptance of the verified drafts and the
 *                         accepted branch's K/V moved behind the prefix.
 *
 * Sources (technical-summary pages on gist.science/pt/paper/...):
 *   Vegas (2602.07223): §2 "Mecanismo Central" steps 1-3 (verify with full
 *     attention, select critical KV entries as a by-product, draft with sparse
 *     attention over them); §2.A selection equation; §2.B Collect-2-Query;
 *     §3 kernel instrumentation (pre-softmax logits) and sparse execution
 *     (paged attention with one-token pages, token indices as page indices).
 *   JETFLOW (2606.18394): §2 tree causal attention mask; §3 item 3 (paged
 *     attention with a tree-mask stage).
 *
 * Conventions for every entry point:
 *   - Pointers without a _host suffix are DEVICE pointers, owned by the caller.
 *     The library never allocates, frees or retains them, and keeps no state
 *     between calls (except the optional timing events, see below).
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and performs no host synchronisation.  Host arrays (_host) are
 *     read before the call returns.
 *   - Results are deterministic: no floating-point atomics; re-running a call
 *     on the same inputs gives bit-identical outputs.
 *   - Host-visible arguments are validated before any launch; on error nothing
 *     is launched, the status is returned and sv_last_error() describes it.
 *     Contents of device arrays (prefix lengths, parents, page tables, index
 *     lists) are a caller contract.  Kernels never access K/V outside the
 *     storage described by sv_kv_cache.num_slots: a position whose slot falls
 *     outside [0, num_slots) is read from slot 0 instead, and results that
 *     depend on it are unspecified.
 */
#ifndef SV_H
#define SV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_ABI_VERSION 1

typedef enum {
  SV_OK = 0,
  SV_E_INVALID = 1,      /* bad shape, null pointer, inconsistent sizes        */
  SV_E_UNSUPPORTED = 2,  /* valid but not implemented: D not in {64,128}, N>256 */
  SV_E_WORKSPACE = 3,    /* workspace missing or smaller than *_workspace_size */
  SV_E_HIP = 4           /* a HIP runtime call or kernel launch failed          */
} sv_status;

typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

typedef void* sv_stream; /* hipStream_t */

/* KV cache of one attention layer.
 * K and V are token-major rows [slot][Hkv][D] of the call's dtype, D contiguous.
 * Logical position i of sequence b lives in
 *   contiguous (page_table == NULL): slot = b * seq_stride + i
 *   paged:                            slot = page_table[b * max_pages + i / page_size] * page_size
 *                                            + i % page_size
 * For verification, the N verify tokens of sequence b have their K/V at
 * logical positions [P_b, P_b + N) (they attend to themselves). */
typedef struct {
  const void* k;
  const void* v;
  const int32_t* page_table; /* device [B][max_pages], or NULL for contiguous */
  int32_t page_size;         /* tokens per page (paged only), >= 1             */
  int32_t max_pages;         /* row stride of page_table (paged only)          */
  int64_t seq_stride;        /* slots per sequence (contiguous only)           */
  int64_t num_slots;         /* number of [Hkv][D] rows in k and in v          */
} sv_kv_cache;

int sv_abi_version(void);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* sv_last_error(void);

/* ------------------------------------------------------------------------ */
/* Verification attention + criticality scores.
 *
 * Vegas §2 step 1 and §5: every verify query attends with exact softmax
 * attention to the whole prefix; JETFLOW §2: a tree node additionally sees its
 * ancestors and itself among the verify tokens (never siblings or
 * descendants).  Vegas §2.A / §3: the score of prefix entry i is
 *     s[b][i] = sum_{t in score_rows} sum_{h < Hq} scale * q[b][t][h] . k[b][i][h / (Hq/Hkv)]
 * i.e. pre-softmax logits summed over the scoring rows (all drafts, or the
 * Collect-2-Query pair of Vegas §2.B) and over all query heads; rejected
 * drafts count as well (the scores come from this pass alone).
 *
 *   q            [B][N][Hq][D] dtype; row t = verify node t (node 0 = root).
 *   dtype        SV_F32 or SV_BF16 (q, K, V and out share it).
 *   B, N, Hq, Hkv, D   batch, verify nodes (1..256), query heads, KV heads
 *                (Hq % Hkv == 0; query head h reads KV head h / (Hq/Hkv)),
 *                head dim (64 or 128).
 *   kv           KV cache (see sv_kv_cache).
 *   prefix_len   device int32[B]: P_b, committed prefix length (0 <= P_b <= P_max).
 *   P_max        host scalar, >= every P_b; row stride of `scores`.
 *   parent       device int32[B][N] draft-tree parents (parent[b][0] = -1,
 *                0 <= parent[b][i] < i), or NULL for a linear chain (node i's
 *                parent is i - 1, which is ordinary causal attention).
 *   score_rows_host  host int32[n_score_rows], distinct nodes in [0, N) whose
 *                logits are summed; n_score_rows = 0 means no scores.
 *   softmax_scale    > 0, or 0 for 1/sqrt(D).
 *   out          [B][N][Hq][D] dtype (round-to-nearest-even from fp32).
 *   scores       fp32 [B][P_max]; entries i < P_b are written, the rest are
 *                left untouched.  May be NULL iff n_score_rows == 0.
 *   workspace    device scratch of at least sv_verify_workspace_size(...)
 *                bytes (same B, N, Hq, Hkv, D, P_max, dtype, parent != NULL,
 *                n_score_rows and kv->page_size, or 0 for a contiguous cache);
 *                contents on entry are ignored.
 */
size_t sv_verify_workspace_size(int B, int N, int Hq, int Hkv, int D, int P_max,
                                sv_dtype dtype, int is_tree, int n_score_rows, int page_size);
sv_status sv_verify_attn(const void* q, sv_dtype dtype, int B, int N, int Hq, int Hkv, int D,
                         const sv_kv_cache* kv, const int32_t* prefix_len, int P_max,
                         const int32_t* parent, const int32_t* score_rows_host, int n_score_rows,
                         float softmax_scale, void* out, float* scores,
                         void* workspace, size_t workspace_bytes, sv_stream stream);

/* ------------------------------------------------------------------------ */
/* Top-k selection (Vegas §2 step 2 and §2.A: the k-subset of the prefix with
 * the largest summed score is the set of the k largest scores).
 *
 *   scores       fp32 [B][P_max] (only entries i < P_b are read).
 *   prefix_len   device int32[B] (clamped to [0, P_max]).
 *   k            device int32[B]: requested k_b; k'_b = min(k_b, P_b, k_max), >= 0.
 *   k_max        host scalar: row stride of idx.
 *   idx          device int32[B][k_max]: the k'_b selected indices in increasing
 *                order, then -1 up to k_max.  Ties are broken toward the lower
 *                index; -0.0 and +0.0 are equal.  Scores must be finite; NaN
 *                entries are never selected (unless k'_b = P_b), so a row with
 *                fewer than k'_b others gets fewer indices.
 *   count        device int32[B] (may be NULL): the number of indices written
 *                (k'_b for finite scores).
 *   workspace    sv_topk_workspace_size(B, P_max) bytes of device scratch;
 *                contents on entry are ignored.
 */
size_t sv_topk_workspace_size(int B, int P_max);
sv_status sv_topk_select(const float* scores, int B, int P_max, const int32_t* prefix_len,
                         const int32_t* k, int k_max, int32_t* idx, int32_t* count,
                         void* workspace, size_t workspace_bytes, sv_stream stream);

/* ------------------------------------------------------------------------ */
/* Verification with the selection fused in (Vegas §2 steps 1-2: the critical
 * entries are selected as a by-product of the verification pass).  Exactly
 * sv_verify_attn followed by sv_topk_select on its scores (same outputs,
 * bit for bit), with the selection's first pass run on the scores as they are
 * summed and its second pass on the last workgroup of each sequence to finish,
 * inside the verification's final kernel, so no launch and no trip through
 * memory is spent between the two.
 *
 *   Arguments as sv_verify_attn, plus (as sv_topk_select):
 *   k            device int32[B]: requested k_b; k'_b = min(k_b, P_b, k_max).
 *   k_max        host scalar: row stride of idx.
 *   idx          device int32[B][k_max]: selected prefix indices, increasing,
 *                then -1.
 *   count        device int32[B] (may be NULL): the number of indices written.
 *   n_score_rows must be >= 1 and P_max <= 131072 (SV_E_UNSUPPORTED above:
 *   use the two calls).
 *   workspace    sv_verify_select_workspace_size(...) bytes (same arguments
 *                as sv_verify_workspace_size); contents on entry are ignored.
 */
size_t sv_verify_select_workspace_size(int B, int N, int Hq, int Hkv, int D, int P_max, sv_dtype dtype,
                                       int is_tree, int n_score_rows, int page_size);
sv_status sv_verify_select(const void* q, sv_dtype dtype, int B, int N, int Hq, int Hkv, int D,
                           const sv_kv_cache* kv, const int32_t* prefix_len, int P_max, const int32_t* parent,
                           const int32_t* score_rows_host, int n_score_rows, float softmax_scale,
                           const int32_t* k, int k_max, void* out, float* scores, int32_t* idx, int32_t* count,
                           void* workspace, size_t workspace_bytes, sv_stream stream);

/* ------------------------------------------------------------------------ */
/* Sparse draft attention (Vegas §2 step 3 and §3: decode attention of one
 * draft query per sequence over exactly the listed token positions, as a
 * paged kernel whose pages hold one token and whose page indices are the
 * token indices).
 *
 *   q            [B][Hq][D] dtype, one query per sequence.
 *   kv           KV cache; idx entries are LOGICAL positions mapped through it
 *                (so positions past the prefix -- accepted or drafted tokens --
 *                may be listed too).
 *   idx          device int32[B][idx_stride] logical positions.
 *   n_idx        device int32[B]: entries of idx[b] to use (clamped to [0, max_idx]);
 *                0 gives a zero output.  sv_topk_select's `count` fits here.
 *   max_idx      host scalar >= every n_idx[b], <= idx_stride.
 *   out          [B][Hq][D] dtype.
 *   workspace    sv_sparse_workspace_size(B, Hq, Hkv, D, max_idx) bytes.
 */
size_t sv_sparse_workspace_size(int B, int Hq, int Hkv, int D, int max_idx);
sv_status sv_sparse_draft_attn(const void* q, sv_dtype dtype, int B, int Hq, int Hkv, int D,
                               const sv_kv_cache* kv, const int32_t* idx, int idx_stride,
                               const int32_t* n_idx, int max_idx, float softmax_scale, void* out,
                               void* workspace, size_t workspace_bytes, sv_stream stream);

/* ------------------------------------------------------------------------ */
/* Selection variants.
 *
 * Per-KV-head selection: the score of Vegas §2.A kept per KV head g (summed
 * over the scoring rows and the query heads of group g only), so each KV head
 * can keep its own k entries; the draft step then reads one list per KV head.
 *
 * sv_verify_attn_per_head: exactly sv_verify_attn, except that head_scores
 *   is fp32 [B][Hkv][P_max]: head_scores[b][g][i] = sum_{t in score_rows}
 *   sum_{h in group g} scale * q[b][t][h] . k[b][i][g], entries i < P_b
 *   written; summed over g it is sv_verify_attn's score.  Selection per head is
 *   sv_topk_select over the B * Hkv rows (prefix_len and k given per row).
 * sv_sparse_draft_attn_per_head: exactly sv_sparse_draft_attn, except that
 *   idx is [B][Hkv][idx_stride] and n_idx [B][Hkv]: the query heads of group g
 *   attend to the list of KV head g.
 *
 * sv_select_sink_window: the query-agnostic baseline the Vegas results
 * compare against (attention sinks plus a recent window): idx[b] = the first
 * `sink` and the last `window` prefix positions, increasing, then -1 up to
 * k_max; count[b] (may be NULL) their number.  Needs k_max >= sink + window.
 */
sv_status sv_verify_attn_per_head(const void* q, sv_dtype dtype, int B, int N, int Hq, int Hkv, int D,
                                  const sv_kv_cache* kv, const int32_t* prefix_len, int P_max,
                                  const int32_t* parent, const int32_t* score_rows_host, int n_score_rows,
                                  float softmax_scale, void* out, float* head_scores,
                                  void* workspace, size_t workspace_bytes, sv_stream stream);
sv_status sv_sparse_draft_attn_per_head(const void* q, sv_dtype dtype, int B, int Hq, int Hkv, int D,
                                        const sv_kv_cache* kv, const int32_t* idx, int idx_stride,
                                        const int32_t* n_idx, int max_idx, float softmax_scale, void* out,
                                        void* workspace, size_t workspace_bytes, sv_stream stream);
sv_status sv_select_sink_window(int B, int P_max, const int32_t* prefix_len, int sink, int window, int k_max,
                                int32_t* idx, int32_t* count, sv_stream stream);

/* ------------------------------------------------------------------------ */
/* Draft loop over a compacted KV.  The draft model's attention is called once
 * per draft token over the same selected set (Vegas §2 step 3; §3, the sparse
 * kernel invoked several times per speculative step), so the set is gathered
 * once into dense buffers and each drafted token's own K/V row is appended
 * behind it (its tail) before the token's decode reads all rows so far.
 *
 * sv_compact_kv: for j < n_b = min(n_idx[b], max_idx, cap), copy the K and V
 * rows (all Hkv heads) of logical position idx[b][j] into row j of sequence b:
 *   ck, cv       device [B][cap][Hkv][D] dtype, 16-byte aligned, caller-owned;
 *                rows j >= n_b are left untouched (the caller appends tail
 *                rows there with plain copies).
 *   kv, idx, idx_stride, n_idx, max_idx   as for sv_sparse_draft_attn.
 * Bytes are copied unchanged (results are bit-identical to the cache rows).
 */
sv_status sv_compact_kv(sv_dtype dtype, int B, int Hkv, int D, const sv_kv_cache* kv,
                        const int32_t* idx, int idx_stride, const int32_t* n_idx, int max_idx,
                        void* ck, void* cv, int cap, sv_stream stream);

/* sv_dense_draft_attn: decode attention of one query per sequence over rows
 * [0, n_rows[b]) of dense buffers (the compacted set, then the tail, the last
 * row being the drafted token's own).
 *   q            [B][Hq][D] dtype.
 *   ck, cv       device [B][cap][Hkv][D] dtype.
 *   n_rows       device int32[B], 0 <= n_rows[b] <= cap (larger values are
 *                clamped to cap); 0 gives a zero output.
 *   out          [B][Hq][D] dtype (round-to-nearest-even from fp32).
 *   workspace    sv_dense_draft_workspace_size(B, Hq, Hkv, D, cap, dtype) bytes;
 *                contents on entry are ignored.
 * Same result (up to rounding order) as sv_sparse_draft_attn over the listed
 * positions of the rows.
 */
size_t sv_dense_draft_workspace_size(int B, int Hq, int Hkv, int D, int cap, sv_dtype dtype);
sv_status sv_dense_draft_attn(const void* q, sv_dtype dtype, int B, int Hq, int Hkv, int D,
                              const void* ck, const void* cv, int cap, const int32_t* n_rows,
                              float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                              sv_stream stream);

/* ------------------------------------------------------------------------ */
/* Best-first draft tree construction (JETFLOW §2, tree construction: the
 * draft head gives log-probabilities for every depth at once, a branch is
 * scored by its cumulative draft log-probability, and best-first expansion
 * grows the tree up to a node budget), on the device so the parent array feeds
 * sv_verify_attn without a host round trip.
 *
 * Node 0 is the root.  A candidate (parent node v, rank r) sits at depth
 * depth(v) + 1 with score score(v) + logprobs[b][depth][r] (fp64, the root
 * scoring 0).  Repeatedly the best candidate -- highest score, then lower
 * parent id, then lower rank -- becomes the next node; a new node offers its
 * rank-0 child (within max_depth) and a taken candidate offers its parent's
 * next rank.  Nodes are numbered in that order, so parents precede children.
 *
 *   logprobs   device fp64 [B][max_depth + 1][n_cand]; row d holds depth d's
 *              candidate log-probabilities in decreasing order (row 0 unused).
 *   n_nodes    node budget including the root, 1..256; it must not exceed
 *              the nodes reachable with n_cand ranks per depth (checked).
 *   n_cand     1..256.
 *   parent     device int32[B][n_nodes] out (parent[b][0] = -1).
 *   depth, rank   device int32[B][n_nodes] out, or NULL.
 */
sv_status sv_build_tree(int B, int n_nodes, int max_depth, int n_cand, const double* logprobs,
                        int32_t* parent, int32_t* depth, int32_t* rank, sv_stream stream);

/* ------------------------------------------------------------------------ */
/* Acceptance after verification and the accepted path's KV (Vegas §2: draft,
 * verify, accept; JETFLOW §2: a drafted node is conditioned on its own branch,
 * so what is accepted is one root-to-node branch of the tree).
 *
 * Greedy acceptance: target_tokens[b][t] is the target model's token after
 * node t (its argmax at verify row t).  From the root, the path moves to the
 * child whose drafted token equals the target token at the current node (the
 * lowest-index child if several do) and stops when no child does.  Then, when
 * kv is non-NULL, the K/V rows of the path are moved IN PLACE to consecutive
 * positions: position P_b + d receives the row of position P_b + path[d]
 * (d >= 1; the root stays at P_b), all KV heads, bytes unchanged.  The
 * committed prefix then ends at P_b + path length; the bonus token (the target
 * token at the path's last node) is the next token to decode.
 *
 *   dtype, Hkv, D    row format of the cache (ignored when kv is NULL).
 *   kv               the cache to update, or NULL for acceptance only.  This
 *                    call WRITES kv->k and kv->v (the rows P_b + 1 .. P_b + d).
 *   prefix_len       device int32[B] P_b (clamped to [0, P_max]); may be NULL
 *                    only when kv and new_prefix_len are NULL.
 *   parent           device int32[B][N] tree parents, or NULL for a chain.
 *   draft_tokens     device int32[B][N]: the drafted token of each node (the
 *                    root's entry is not read).
 *   target_tokens    device int32[B][N].
 *   path             device int32[B][N] out: path node ids by depth, root
 *                    first, then -1.
 *   n_accepted       device int32[B] out: accepted drafted nodes (path length - 1).
 *   bonus            device int32[B] out, or NULL.
 *   new_prefix_len   device int32[B] out, or NULL: P_b + path length.
 */
sv_status sv_accept_commit(sv_dtype dtype, int B, int N, int Hkv, int D, const sv_kv_cache* kv,
                           const int32_t* prefix_len, int P_max, const int32_t* parent,
                           const int32_t* draft_tokens, const int32_t* target_tokens, int32_t* path,
                           int32_t* n_accepted, int32_t* bonus, int32_t* new_prefix_len, sv_stream stream);

/* ------------------------------------------------------------------------ */
/* Contract checks of device arrays (debugging aids, not steps of the method).
 *
 * The calls above trust the contents of their device arrays; a violation
 * gives unspecified results, never an access outside the caller's buffers.
 * These calls check those contents on `stream` (asynchronously, allocating
 * nothing) and write an error record to `err`, a device int32[4]
 * {code, b, i, value}: all zeros when every check passes, otherwise ONE of
 * the violations found (which one is unspecified when there are several).
 * Read `err` after the stream has reached the call.  Codes:
 *   1  prefix_len[b] = value lies outside [0, P_max];
 *   2  logical position i of sequence b (i < P_b + N) maps to no slot in
 *      [0, num_slots) (value: its page-table entry, or -1);
 *   3  parent[b][i] = value: the root's is not -1, or another's is not in [0, i);
 *   4  n_idx of list b = value lies outside [0, max_idx];
 *   5  entry i of list b is position value, negative or mapped to no slot.
 *
 * sv_validate_kv:    prefix lengths and the mapping of positions [0, P_b + N)
 *                    (the ranges sv_verify_attn reads; N = 0 for the prefix).
 * sv_validate_tree:  the parent arrays of sv_verify_attn / sv_accept_commit.
 * sv_validate_index: index lists of the sparse draft step: B * lists_per_seq
 *                    lists ([B][lists_per_seq][idx_stride], 1 list per
 *                    sequence or Hkv for the per-head variant) and their counts.
 * Errors: SV_E_INVALID for a NULL or misaligned err, NULL arrays or bad sizes;
 * SV_E_UNSUPPORTED for more than 65535 sequences or lists. */
sv_status sv_validate_kv(int B, int N, const sv_kv_cache* kv, const int32_t* prefix_len, int P_max,
                         int32_t* err, sv_stream stream);
sv_status sv_validate_tree(int B, int N, const int32_t* parent, int32_t* err, sv_stream stream);
sv_status sv_validate_index(int B, int lists_per_seq, const sv_kv_cache* kv, const int32_t* idx, int idx_stride,
                            const int32_t* n_idx, int max_idx, int32_t* err, sv_stream stream);

/* ------------------------------------------------------------------------ */
/* Verification attention that allocates nothing, for callers that cannot
 * allocate device memory (code under graph capture, serving loops and
 * harnesses that forbid hipMalloc).
 *
 * Same arguments and results as sv_verify_attn, without the workspace: the
 * scratch it needs (chunk partials, score partials, ancestor sets) is a
 * static device array of SV_NOALLOC_SCRATCH_BYTES owned by the library, one
 * per GPU, held until the process ends.  A call whose scratch need
 * (sv_verify_workspace_size of the same arguments) exceeds it returns
 * SV_E_WORKSPACE and launches nothing.  The array's contents are not needed
 * on entry.  All calls on one GPU share its array: calls that may overlap on
 * one GPU (different streams, threads or processes sharing the library
 * instance) race and give unspecified results; calls ordered on one stream
 * are safe.  The first call on a device looks up the array's device address
 * (hipGetSymbolAddress); no call allocates or frees memory. */
#define SV_NOALLOC_SCRATCH_BYTES (64u << 20)
sv_status sv_verify_attn_noalloc(const void* q, sv_dtype dtype, int B, int N, int Hq, int Hkv, int D,
                                 const sv_kv_cache* kv, const int32_t* prefix_len, int P_max,
                                 const int32_t* parent, const int32_t* score_rows_host, int n_score_rows,
                                 float softmax_scale, void* out, float* scores, sv_stream stream);

/* ------------------------------------------------------------------------ */
/* Optional timing hook for profiling: while set (non-NULL), every
 * sv_verify_attn call on this thread records `start_event` on its stream right
 * before its main attention kernel and `stop_event` right after it (both are
 * hipEvent_t created by the caller).  Pass NULL, NULL to clear. */
sv_status sv_set_verify_timing_events(void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* SV_H */
