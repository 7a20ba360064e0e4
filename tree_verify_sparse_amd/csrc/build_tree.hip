// Best-first draft tree construction on the device (JETFLOW §2, tree
// construction: per-depth draft log-probabilities, branches scored by their
// cumulative log-probability, the best candidate expanded first until the
// node budget is reached), so the parent array the verify pass needs never
// makes a host round trip.
//
// One wave per sequence.  The live candidates sit in registers, slot j in
// lane j % 64: each expansion takes one (its slot is reused by the new node's
// rank-0 child) and adds at most one (the parent's next rank), so at most
// n_nodes slots are ever used.  The best candidate -- highest fp64 score,
// then lower parent id, then lower rank -- is found with each lane comparing
// its slots and a DPP wave reduction over (score, key), the key packing
// parent, rank, slot and depth (lower wins; slots are unique).
// Scores are the same fp64 sums, in the same order, as a sequential
// implementation, so the tree is identical bit for bit.  The log-probabilities
// and the growing tree stay in LDS; global memory is touched once before and
// once after the expansions.
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

constexpr int kLpLds = 4096;  // log-probabilities kept in LDS when they fit (32 KB)

template <bool IN_LDS>
__global__ void __launch_bounds__(64) build_tree(const BuildArgs a) {
  __shared__ double lps[kLpLds];     // the sequence's log-probabilities (when they fit)
  __shared__ double cum[kMaxNodes];  // node scores
  __shared__ int np_[kMaxNodes], nd_[kMaxNodes], nr_[kMaxNodes];  // node parent, depth, rank
  constexpr int SPL = kMaxNodes / 64;  // candidate slots per lane: slot j lives in lane j % 64, entry j / 64
  const int b = blockIdx.x, lane = threadIdx.x, n = a.n, nc = a.n_cand;
  const int nlp = (a.max_depth + 1) * nc;
  const double* lpg = a.lp + (long long)b * nlp;
  // every expansion reads two log-probabilities: from LDS when they fit (a
  // separate instantiation, so the reads are plain LDS reads, not flat ones)
  if constexpr (IN_LDS)
    for (int j = lane; j < nlp; j += 64) lps[j] = lpg[j];
  const double* lp = IN_LDS ? lps : lpg;
  const long long o = (long long)b * n;
  const double ninf = -__builtin_inf();
  // candidate (score, key) in registers; key = parent << 24 | rank << 16 | slot << 8 | depth
  // (lower wins among equal scores: parent, then rank; slots are unique)
  double cs[SPL];
  uint32_t ck[SPL];
#pragma unroll
  for (int u = 0; u < SPL; ++u) {
    cs[u] = ninf;
    ck[u] = 0xffffffffu;
  }
  int nslots = 0;
  if (n > 1 && a.max_depth >= 1) {
    if (lane == 0) {
      cs[0] = 0.0 + lpg[1 * nc + 0];
      ck[0] = 1u;  // parent 0, rank 0, slot 0, depth 1
    }
    nslots = 1;
  }
  if (lane == 0) {
    np_[0] = -1;
    nd_[0] = 0;
    nr_[0] = 0;
    cum[0] = 0.0;
  }
  __syncthreads();
  for (int i = 1; i < n; ++i) {
    double bs = cs[0];
    uint32_t bk = ck[0];
#pragma unroll
    for (int u = 1; u < SPL; ++u)
      if (cand_better(cs[u], ck[u], bs, bk)) {
        bs = cs[u];
        bk = ck[u];
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
    const int p = (int)(key >> 24), r = (int)((key >> 16) & 0xffu), slot = (int)((key >> 8) & 0xffu),
              d = (int)(key & 0xffu);
    const bool child = d < a.max_depth, sib = r + 1 < nc;
    // the three reads the new candidates need, issued together (indices kept in range)
    const double lp_child = lp[(child ? d + 1 : d) * nc + 0];
    const double lp_sib = lp[d * nc + (sib ? r + 1 : r)];
    const double cum_p = cum[p];
    const double s_child = child ? sc + lp_child : ninf;
    const uint32_t k_child = child ? (((uint32_t)i << 24) | ((uint32_t)slot << 8) | (uint32_t)(d + 1)) : 0xffffffffu;
    const double s_sib = cum_p + lp_sib;
    const uint32_t k_sib = ((uint32_t)p << 24) | ((uint32_t)(r + 1) << 16) | ((uint32_t)nslots << 8) | (uint32_t)d;
    // the new node's rank-0 child takes the slot; the parent's next rank a new one
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      if (slot == u * 64 + lane) {
        cs[u] = s_child;
        ck[u] = k_child;
      }
      if (sib && nslots == u * 64 + lane) {
        cs[u] = s_sib;
        ck[u] = k_sib;
      }
    }
    if (lane == 0) {
      np_[i] = p;
      nd_[i] = d;
      nr_[i] = r;
      cum[i] = sc;
    }
    nslots += sib ? 1 : 0;
    // one wave: its LDS accesses complete in order, so the next expansion sees
    // these writes without a barrier (a barrier would also wait on memory)
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  for (int t = lane; t < n; t += 64) {
    a.parent[o + t] = np_[t];
    if (a.depth) a.depth[o + t] = nd_[t];
    if (a.rank) a.rank[o + t] = nr_[t];
  }
}

int launch_build_tree(int B, int n, int max_depth, int n_cand, const double* lp, int32_t* parent, int32_t* depth,
                      int32_t* rank, void* stream) {
  BuildArgs a{lp, parent, depth, rank, n, max_depth, n_cand};
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (B == 0) return 0;
  if ((max_depth + 1) * n_cand <= kLpLds)
    hipLaunchKernelGGL(build_tree<true>, dim3(B), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL(build_tree<false>, dim3(B), dim3(64), 0, st, a);
  return (int)hipGetLastError();
}

}  // namespace sv
