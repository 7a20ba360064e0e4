// Host-side plans shared by the C ABI layer and the kernel launchers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "sv.h"

namespace sv {

constexpr int kMaxNodes = 256;       // verify nodes per sequence
constexpr int kAncWords = 8;         // ancestor bitset words per node (256 bits)
constexpr int kInlineQbarRows = 64;  // scoring (row, head) pairs summed inside the main kernel
constexpr int kQbarPairs = 64;       // pairs per partial sum when a prep kernel forms qbar
constexpr size_t kAlign = 256;

// Records the thread's error message (sv_last_error) and returns st.
sv_status set_error(sv_status st, const char* fmt, ...);

inline size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// How one sv_verify_attn call is split into workgroups and workspace regions.
struct VerifyPlan {
  int B, N, Hq, Hkv, G, D, P_max, dtype;
  int R;            // query rows per KV head = N * G (row = node * G + head-in-group)
  int RT, WR, WK;   // row tiles per wave, waves along rows, waves along keys (WR*WK = 4)
  int rows_per_block, RB, Rpad;
  int TK;           // keys per LDS tile
  int qsplit;       // qbar partial sums per (sequence, KV head) (prep_qbar only)
  int chunk;        // keys per split of the KV range
  int n_chunks;     // splits covering the longest sequence (P_max + N)
  int n_wg;         // workgroups of the main kernel (multiple of 8)
  bool tree, scores, prep_qbar, prep;
  bool stream;      // bf16 with R <= 64: the key-split streaming kernel (verify_stream)
  bool treek;       // bf16 with R > 64: the eight-wave row-split tree kernel (verify_tree)
  size_t off_o, off_ml, off_s, off_qbar, off_anc, bytes;
};

// page_size: tokens per page of a paged cache, 0 for a contiguous cache.
VerifyPlan plan_verify(int B, int N, int Hq, int Hkv, int D, int P_max, int dtype, bool tree,
                       int n_score_rows, int page_size);

struct SparsePlan {
  int B, Hq, Hkv, G, D, max_idx, KCH, n_chunks;
  size_t off_o, off_ml, bytes;
};
SparsePlan plan_sparse(int B, int Hq, int Hkv, int D, int max_idx);

struct KvArgs {
  const void* k;
  const void* v;
  const int32_t* page_table;
  int page_size, max_pages;
  long long seq_stride, num_slots;
};

// Selection fused into verification (sv_verify_select): the top-k of the
// scores, with its own workspace of select_workspace_bytes(B).
struct SelectArgs {
  const int32_t* k;  // device [B]
  int k_max;
  int32_t* idx;      // device [B][k_max]
  int32_t* count;    // device [B] or null
  void* ws;
};
size_t select_workspace_bytes(int B);
constexpr int kSelectMaxP = 32 * 4096;  // longest prefix the fused selection takes

// Launchers (return a hipError_t as int; 0 = success).
// len_bias: 0 for verification; -1 turns prefix_len into row counts of a dense
// decode (N = 1: the query sees rows [0, prefix_len[b]), none when it is 0).
int launch_verify(const VerifyPlan& p, const void* q, const KvArgs& kv, const int32_t* prefix_len,
                  const int32_t* parent, const int32_t* score_rows, int n_score_rows, float scale,
                  void* out, float* scores, void* ws, void* stream, void* ev_start, void* ev_stop,
                  int len_bias = 0, int head_scores = 0, const SelectArgs* sel = nullptr);
// Best-first draft trees from per-depth log-probabilities (one wave per sequence).
int launch_build_tree(int B, int n, int max_depth, int n_cand, const double* lp, int32_t* parent, int32_t* depth,
                      int32_t* rank, void* stream);
// Greedy acceptance on draft trees and the accepted path's K/V move (kv may be null).
int launch_accept(int dtype, int B, int N, int Hkv, int D, const KvArgs* kv, const int32_t* prefix_len, int P_max,
                  const int32_t* parent, const int32_t* draft, const int32_t* target, int32_t* path,
                  int32_t* n_accepted, int32_t* bonus, int32_t* new_prefix, void* stream);
// Gather the listed rows (all KV heads) into dense [B][cap][Hkv][D] buffers.
int launch_compact(int dtype, int B, int Hkv, int D, const KvArgs& kv, const int32_t* idx, int idx_stride,
                   const int32_t* n_idx, int max_idx, void* ck, void* cv, int cap, void* stream);
int launch_topk(const float* scores, int B, int P_max, const int32_t* prefix_len, const int32_t* k,
                int k_max, int32_t* idx, int32_t* count, void* ws, void* stream);
size_t topk_workspace_bytes(int B, int P_max);
bool topk_supported(int P_max);
// per_head: idx is [B][Hkv][idx_stride] and n_idx [B][Hkv], one list per KV head.
int launch_sparse(const SparsePlan& p, int dtype, const void* q, const KvArgs& kv, const int32_t* idx,
                  int idx_stride, const int32_t* n_idx, float scale, void* out, void* ws, void* stream,
                  int per_head = 0);
// The first `sink` and the last `window` prefix positions of each sequence.
int launch_sink_window(int B, int P_max, const int32_t* prefix_len, int sink, int window, int k_max, int32_t* idx,
                       int32_t* count, void* stream);

// Contract checks of device arrays (error record {code, b, i, value}; codes below).
constexpr int kErrPrefixLen = 1;  // prefix_len[b] = value outside [0, P_max]
constexpr int kErrUnmapped = 2;   // position i of sequence b maps to no slot (value: its page entry, or -1)
constexpr int kErrParent = 3;     // parent[b][i] = value is not -1 for the root / not in [0, i)
constexpr int kErrCount = 4;      // n_idx[list b] = value outside [0, max_idx]
constexpr int kErrIndex = 5;      // entry i of list b is position value, negative or mapped to no slot
int launch_validate_kv(int B, int N, const KvArgs& kv, const int32_t* prefix_len, int P_max, int32_t* err,
                       void* stream);
int launch_validate_tree(int B, int N, const int32_t* parent, int32_t* err, void* stream);
int launch_validate_index(int n_lists, int lists_per_seq, const KvArgs& kv, const int32_t* idx, int idx_stride,
                          const int32_t* n_idx, int max_idx, int32_t* err, void* stream);

}  // namespace sv
