// Best-first draft tree construction on the device (JETFLOW §2, tree
// construction: per-depth draft log-probabilities, branches scored by their
// cumulative log-probability, the best candidate expanded first until the
// node budget is reached), so the parent array the verify pass needs never
// makes a host round trip.
//
// One wave per sequence.  The live candidates sit in LDS: each expansion
// takes one (its slot is reused by the new node's rank-0 child) and adds at
// most one (the parent's next rank), so at most n_nodes slots are ever used.
// The best candidate -- highest fp64 score, then lower parent id, then lower
// rank -- is found with each lane scanning its slots and a DPP wave reduction
// over (score, key), the key packing parent, rank and slot (lower wins).
// Scores are the same fp64 sums, in the same order, as a sequential
// implementation, so the tree is identical bit for bit.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

struct BuildArgs {
  const double* lp;  // [B][max_depth + 1][n_cand]
  int32_t* parent;   // [B][n]
  int32_t* depth;    // [B][n] or null
  int32_t* rank;     // [B][n] or null
  int n, max_depth, n_cand;
};

__device__ __forceinline__ bool cand_better(double s1, uint32_t k1, double s2, uint32_t k2) {
  return s1 > s2 || (s1 == s2 && k1 < k2);
}

template <int CTRL, int ROWS>
__device__ __forceinline__ void cand_dpp(double& s, uint32_t& k) {
  const unsigned long long bits = (unsigned long long)__double_as_longlong(s);
  // lanes without a source keep the identity (-inf, 0xffffffff)
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)bits, CTRL, ROWS, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)0xfff00000u, (int)(uint32_t)(bits >> 32), CTRL, ROWS,
                                                            0xf, false);
  const uint32_t ko = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)k, CTRL, ROWS, 0xf, false);
  const double so = __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
  if (cand_better(so, ko, s, k)) {
    s = so;
    k = ko;
  }
}

__global__ void __launch_bounds__(64) build_tree(const BuildArgs a) {
  __shared__ double cs[kMaxNodes];     // candidate score, -inf = free slot
  __shared__ uint32_t ck[kMaxNodes];   // parent << 16 | rank << 8 | slot
  __shared__ int cd[kMaxNodes];        // candidate depth
  __shared__ double cum[kMaxNodes];    // node scores
  const int b = blockIdx.x, lane = threadIdx.x, n = a.n, nc = a.n_cand;
  const double* lp = a.lp + (long long)b * (a.max_depth + 1) * nc;
  const long long o = (long long)b * n;
  const double ninf = -__builtin_inf();
  int nslots = 0;
  if (lane == 0) {
    a.parent[o] = -1;
    if (a.depth) a.depth[o] = 0;
    if (a.rank) a.rank[o] = 0;
    cum[0] = 0.0;
    if (n > 1 && a.max_depth >= 1) {
      cs[0] = 0.0 + lp[1 * nc + 0];
      ck[0] = 0u;
      cd[0] = 1;
    }
  }
  if (n > 1 && a.max_depth >= 1) nslots = 1;
  __syncthreads();
  for (int i = 1; i < n; ++i) {
    double bs = ninf;
    uint32_t bk = 0xffffffffu;
    for (int j = lane; j < nslots; j += 64) {
      const double s = cs[j];
      const uint32_t k = ck[j];
      if (cand_better(s, k, bs, bk)) {
        bs = s;
        bk = k;
      }
    }
    cand_dpp<0x111, 0xf>(bs, bk);  // row_shr:1
    cand_dpp<0x112, 0xf>(bs, bk);  // row_shr:2
    cand_dpp<0x114, 0xf>(bs, bk);  // row_shr:4
    cand_dpp<0x118, 0xf>(bs, bk);  // row_shr:8
    cand_dpp<0x142, 0xa>(bs, bk);  // row_bcast:15
    cand_dpp<0x143, 0xc>(bs, bk);  // row_bcast:31
    const unsigned long long bb = (unsigned long long)__double_as_longlong(bs);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)bb, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(bb >> 32), 63);
    const uint32_t key = (uint32_t)__builtin_amdgcn_readlane((int)bk, 63);
    const double sc = __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
    // the host checked that n nodes are reachable, so a live candidate exists
    const int slot = (int)(key & 0xffu), r = (int)((key >> 8) & 0xffu), p = (int)(key >> 16);
    const int d = cd[slot];
    const bool sib = r + 1 < nc;
    if (lane == 0) {
      a.parent[o + i] = p;
      if (a.depth) a.depth[o + i] = d;
      if (a.rank) a.rank[o + i] = r;
      cum[i] = sc;
      if (d < a.max_depth) {  // the new node's rank-0 child takes the slot
        cs[slot] = sc + lp[(d + 1) * nc + 0];
        ck[slot] = ((uint32_t)i << 16) | (uint32_t)slot;
        cd[slot] = d + 1;
      } else {
        cs[slot] = ninf;
        ck[slot] = 0xffffffffu;
      }
      if (sib) {  // the parent's next rank
        cs[nslots] = cum[p] + lp[d * nc + r + 1];
        ck[nslots] = ((uint32_t)p << 16) | ((uint32_t)(r + 1) << 8) | (uint32_t)nslots;
        cd[nslots] = d;
      }
    }
    nslots += sib ? 1 : 0;
    __syncthreads();
  }
}

int launch_build_tree(int B, int n, int max_depth, int n_cand, const double* lp, int32_t* parent, int32_t* depth,
                      int32_t* rank, void* stream) {
  BuildArgs a{lp, parent, depth, rank, n, max_depth, n_cand};
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (B == 0) return 0;
  hipLaunchKernelGGL(build_tree, dim3(B), dim3(64), 0, st, a);
  return (int)hipGetLastError();
}

}  // namespace sv
