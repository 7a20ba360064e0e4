// Greedy acceptance after verification, and the accepted path's K/V moved to
// consecutive positions (Vegas §2: draft, verify, accept; JETFLOW §2: a node's
// token is conditioned on its own branch, so what is accepted is one
// root-to-node branch of the draft tree).
//
// One wave per sequence.  The tree (parents, drafted tokens, target tokens)
// sits in LDS; the walk from the root takes at each node the lowest-index child
// whose drafted token equals the target's token at that node (a wave minimum
// over the candidate children, which have higher indices than their parent),
// so a path of length d costs d wave reductions and no barrier.  The K/V rows
// of path depth d are then copied from position P_b + path[d] to P_b + d, in
// depth order: a row's source lies past every earlier destination (path[d] >=
// d), and each lane copies the same 16-byte pieces of every row, so the
// in-place moves need no synchronisation.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

struct AcceptArgs {
  KvView kv;  // rows are written in place
  const int32_t* prefix_len;
  const int32_t* parent;  // [B][N], or null for a chain
  const int32_t* draft;   // [B][N]
  const int32_t* target;  // [B][N]
  int32_t* path;          // [B][N]: node ids by depth (root first), then -1
  int32_t* n_accepted;    // [B]: accepted drafted nodes (path length - 1)
  int32_t* bonus;         // [B] or null: target token at the last path node
  int32_t* new_prefix;    // [B] or null: P_b + path length
  int N, P_max;
  int row_pieces;         // 16-byte pieces of one K (or V) row; 0 = no K/V move
};

__global__ void __launch_bounds__(64) accept_commit(const AcceptArgs a) {
  __shared__ int par[kMaxNodes], dr[kMaxNodes], tg[kMaxNodes], pth[kMaxNodes];
  const int b = blockIdx.x, lane = threadIdx.x, N = a.N;
  const long long row0 = (long long)b * N;
  for (int t = lane; t < N; t += 64) {
    par[t] = a.parent ? a.parent[row0 + t] : t - 1;
    dr[t] = a.draft[row0 + t];
    tg[t] = a.target[row0 + t];
  }
  if (lane == 0) pth[0] = 0;
  __syncthreads();
  int cur = 0, len = 1;
  for (;;) {  // cur strictly increases, so at most N - 1 steps
    const int want = tg[cur];
    uint32_t best = 0x7fffffffu;
    for (int t = cur + 1 + lane; t < N; t += 64)
      if (par[t] == cur && dr[t] == want) best = min(best, (uint32_t)t);
    best = wave_min_u32(best);
    if (best == 0x7fffffffu) break;
    cur = (int)best;
    if (lane == 0) pth[len] = cur;
    ++len;
  }
  __syncthreads();
  for (int t = lane; t < N; t += 64) a.path[row0 + t] = t < len ? pth[t] : -1;
  int Pb = a.prefix_len ? a.prefix_len[b] : 0;
  Pb = Pb < 0 ? 0 : (Pb > a.P_max ? a.P_max : Pb);
  if (lane == 0) {
    a.n_accepted[b] = len - 1;
    if (a.bonus) a.bonus[b] = tg[cur];
    if (a.new_prefix) a.new_prefix[b] = Pb + len;
  }
  if (a.row_pieces <= 0) return;
  const long long row_bytes = (long long)a.row_pieces * 16;
  char* kb = reinterpret_cast<char*>(const_cast<void*>(a.kv.k));
  char* vb = reinterpret_cast<char*>(const_cast<void*>(a.kv.v));
  for (int d = 1; d < len; ++d) {
    const int v = pth[d];
    if (v == d) continue;  // already in place (a chain's path never moves)
    const long long src = a.kv.slot(b, Pb + v), dst = a.kv.slot(b, Pb + d);
    if (src < 0 || dst < 0) continue;  // unmapped positions: caller contract, nothing is moved
    for (int c = lane; c < a.row_pieces; c += 64) {
      const uint4 kx = *reinterpret_cast<const uint4*>(kb + src * row_bytes + c * 16);
      const uint4 vx = *reinterpret_cast<const uint4*>(vb + src * row_bytes + c * 16);
      *reinterpret_cast<uint4*>(kb + dst * row_bytes + c * 16) = kx;
      *reinterpret_cast<uint4*>(vb + dst * row_bytes + c * 16) = vx;
    }
  }
}

int launch_accept(int dtype, int B, int N, int Hkv, int D, const KvArgs* kv, const int32_t* prefix_len, int P_max,
                  const int32_t* parent, const int32_t* draft, const int32_t* target, int32_t* path,
                  int32_t* n_accepted, int32_t* bonus, int32_t* new_prefix, void* stream) {
  AcceptArgs a{};
  if (kv) {
    a.kv = KvView{kv->k, kv->v, kv->page_table, kv->page_size, kv->max_pages, kv->seq_stride, kv->num_slots};
    a.row_pieces = Hkv * D * (dtype == SV_BF16 ? 2 : 4) / 16;
  }
  a.prefix_len = prefix_len;
  a.parent = parent;
  a.draft = draft;
  a.target = target;
  a.path = path;
  a.n_accepted = n_accepted;
  a.bonus = bonus;
  a.new_prefix = new_prefix;
  a.N = N;
  a.P_max = P_max;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (B == 0) return 0;
  hipLaunchKernelGGL(accept_commit, dim3(B), dim3(64), 0, st, a);
  return (int)hipGetLastError();
}

}  // namespace sv
