// Best-first draft tree construction on the device (JETFLOW §2, tree
// construction: per-depth draft log-probabilities, branches scored by their
// cumulative log-probability, the best candidate expanded first until the
// node budget is reached), so the parent array the verify pass needs never
// makes a host round trip.
//
// A node is a rank sequence (r_1 .. r_d) with score S = sum_j lp[j][r_j]
// (fp64, accumulated from the root in depth order, as the sequential
// expansion adds a candidate's log-probability to its parent's score).  Log-
// probabilities are at most 0 and each depth's list is sorted, so a node's
// parent and its lower-rank siblings score at least as high as the node, and
// the sequential expansion takes nodes in the order
//     higher score first; equal scores: the parent taken earlier first, then
//     the lower rank
// (an order in which every candidate comes after the node that offered it, so
// always taking the best offered candidate follows it exactly).  The tree is
// therefore the first n - 1 sequences of that order, and it is built without
// the sequential loop:
//   1. a threshold tau with n - 1 <= |{S >= tau}| <= kBtCap is found by
//      counting, in each of the 16 waves, the sequences at or above one trial
//      value (level by level: a node at depth d - 1 with score s has exactly
//      the children r with s + lp[d][r] >= tau, a prefix of the sorted list);
//      the first round tries 16 values from 0.4 to 1.67 times the spread of
//      the depth-1 list below the best depth-1 score (10% apart), later rounds
//      16 evenly spaced values inside the bracket found so far, or values
//      spaced ever wider below the lowest one tried;
//   2. the wave that counted the chosen value holds C = {S >= tau}, which
//      contains the tree; every node of C gets its place in the order from a
//      histogram of the scores (the nodes of earlier bins, which all score
//      higher) plus the nodes of its own bin before it (equal scores compare
//      parents, walking up), and the first n - 1 places are numbered
//      1 .. n - 1.
// A wave stops expanding once a wave with a higher trial value has isolated
// the tree (the first value reaching n - 1 is then known to be at or below
// that one), so a round lasts as long as its winner, not its slowest wave.
// If no trial value isolates at most kBtCap sequences (many exactly equal
// scores at the threshold), wave 0 runs the sequential expansion instead.
// The only atomics are LDS integer ones whose order decides nothing (an early-
// stop flag, a node's slot inside its score bin): the result is the same bits
// on every run, and the same tree as the sequential expansion.
#include "select_dev.h"
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

constexpr int kLpLds = 4096;   // log-probabilities kept in LDS when they fit (32 KB)
constexpr int kBtWaves = 16;   // trial thresholds counted at once (one per wave)
constexpr int kBtCap = 512;    // sequences a wave holds for one trial value
constexpr int kBtRounds = 8;   // bracketing rounds before the sequential expansion
constexpr int kBtBins = kBtWaves * 64;  // score bins of the placement (one per thread)
constexpr uint32_t kBtRoot = 0xffffu;

struct BtShared {
  double lp[kLpLds];
  double S[kBtWaves][kBtCap];            // scores
  uint32_t meta[kBtWaves][kBtCap];       // parent's index in the same list << 16 | rank << 8 | depth
  int pos[kBtCap];                       // place in the expansion order
  int wsum[kBtWaves];                    // per-wave totals of the placement's scan
  int8_t mark[kBtWaves][kBtCap + 64];    // child placement marks (lane numbers)
  int cnt[kBtWaves];
  int done_min;  // the lowest wave whose count already isolates the tree (kBtWaves: none yet)
  double tau[kBtWaves];
  // sequential expansion
  double cum[kMaxNodes];
  int np_[kMaxNodes], nd_[kMaxNodes], nr_[kMaxNodes];
};

// The next double above a finite x.
__device__ __forceinline__ double next_up(double x) {
  if (x == 0.0) return __longlong_as_double(1LL);
  const long long u = __double_as_longlong(x);
  return __longlong_as_double(x > 0.0 ? u + 1 : u - 1);
}

// The first step of the search over a depth's sorted list: span and the
// eight probes (the same for every parent of the level, so loaded once).  The
// steps of spans 64, 8 and 1 reach rank 583, past the 256 ranks a depth may
// hold (sv_build_tree rejects more), so every count is exact.
struct BtProbe {
  int span;
  double p[8];
};
__device__ __forceinline__ BtProbe bt_probe(const double* row, int nc) {
  BtProbe q;
  q.span = nc > 64 ? 64 : (nc > 8 ? 8 : 1);
#pragma unroll
  for (int k = 0; k < 8; ++k) q.p[k] = row[min(q.span * (k + 1) - 1, nc - 1)];
  return q;
}

// Number of ranks r < nc with sv + row[r] >= tau (a prefix of the sorted
// list): an 8-way search, the first step from the level's probes, each later
// step's eight probes loaded together at clamped places and tested after (a
// branch around each load made every probe its own trip to LDS).
__device__ __forceinline__ int bt_count(const double* row, int nc, double sv, double tau, const BtProbe& q) {
  int m = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) m += int((q.span * (k + 1) - 1 < nc) & (sv + q.p[k] >= tau));
  int c = q.span * m;
  for (int span = q.span >> 3; span >= 1; span >>= 3) {
    double x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = row[min(c + span * (k + 1) - 1, nc - 1)];
    m = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) m += int((c + span * (k + 1) - 1 < nc) & (sv + x[k] >= tau));
    c += span * m;
  }
  return c;
}

// Inclusive max over lanes 0 .. lane (DPP, no LDS).
__device__ __forceinline__ int wave_incl_max(int x) {
  x = max(x, (int)__builtin_amdgcn_update_dpp(-1, x, 0x111, 0xf, 0xf, false));
  x = max(x, (int)__builtin_amdgcn_update_dpp(-1, x, 0x112, 0xf, 0xf, false));
  x = max(x, (int)__builtin_amdgcn_update_dpp(-1, x, 0x114, 0xf, 0xf, false));
  x = max(x, (int)__builtin_amdgcn_update_dpp(-1, x, 0x118, 0xf, 0xf, false));
  x = max(x, (int)__builtin_amdgcn_update_dpp(-1, x, 0x142, 0xa, 0xf, false));
  x = max(x, (int)__builtin_amdgcn_update_dpp(-1, x, 0x143, 0xc, 0xf, false));
  return x;
}

// The sequences with score >= tau, level by level, into one wave's lists;
// their number, or kBtCap + 1 as soon as there would be more than kBtCap, or
// as soon as a wave below this one (a higher trial value) has isolated the
// tree (*done_min < wave: this wave's count can no longer be the first to
// reach n - 1).  mark: the wave's kBtCap + 64 LDS bytes for placing children.
__device__ int bt_expand(const double* lp, int nc, int max_depth, double tau, double* S, uint32_t* meta,
                         int8_t* mark, const int* done_min, int wave, int lane) {
  int cnt = 0;
  int p0 = -1, np = 1;  // the previous level: first index and size (the root alone at first)
  for (int d = 1; d <= max_depth; ++d) {
    const double* row = lp + (long long)d * nc;
    // the level's constants, loaded once: the search's first probes and the
    // first four log-probabilities (the children of a parent with few)
    const BtProbe q = bt_probe(row, nc);
    double r4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) r4[j] = row[min(j, nc - 1)];
    int level = 0;
    for (int base = 0; base < np; base += 64) {
      const int i = base + lane;
      const bool act = i < np;
      const int v = p0 < 0 ? -1 : p0 + i;
      const double s = S[(act && v >= 0) ? v : 0];  // loaded with the flag below
      const int dm = *done_min;
      if (dm < wave) return kBtCap + 1;  // wave-uniform
      const double sv = (act && v >= 0) ? s : 0.0;
      const int c = act ? bt_count(row, nc, sv, tau, q) : 0;
      const int incl = (int)sel_wave_scan((uint32_t)c);
      const int tot = __builtin_amdgcn_readlane(incl, 63);
      if (cnt + level + tot > kBtCap) return kBtCap + 1;
      const int o = cnt + level + incl - c;  // this lane's first child's place
      const uint32_t pm = (uint32_t)(v < 0 ? kBtRoot : (uint32_t)v) << 16;
      if (wave_max_u32((uint32_t)c) <= 4) {
        // few children per parent: each lane writes its own
        double ch[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) ch[j] = sv + r4[j];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (j < c) {
            S[o + j] = ch[j];
            meta[o + j] = pm | (uint32_t)j << 8 | (uint32_t)d;
          }
      } else {
        // children in lane order: lane l's occupy [incl_l - c_l, incl_l) of
        // this batch.  Each parent marks its first child's place; an
        // inclusive max over the marks gives every place its parent lane.
        for (int t = lane; t < tot; t += 64) mark[t] = (int8_t)-1;
        __builtin_amdgcn_wave_barrier();
        if (c > 0) mark[incl - c] = (int8_t)lane;
        __builtin_amdgcn_wave_barrier();
        int carry = -1;
        for (int t0 = 0; t0 < tot; t0 += 64) {
          const int t = t0 + lane;
          int pl = wave_incl_max(t < tot ? (int)mark[t] : -1);
          pl = max(pl, carry);  // every place below tot has a parent; lanes past it read lane 0
          carry = __builtin_amdgcn_readlane(pl, 63);
          pl = max(pl, 0);
          // the parent lane's score, index and first place
          const double psv = __shfl(sv, pl);
          const int pv = __shfl(v, pl);
          const int pfirst = __shfl(incl - c, pl);
          if (t < tot) {
            const int r = t - pfirst;
            const int w = cnt + level + t;
            S[w] = psv + row[r];
            meta[w] = (uint32_t)(pv < 0 ? kBtRoot : (uint32_t)pv) << 16 | (uint32_t)r << 8 | (uint32_t)d;
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
      level += tot;
    }
    // one wave: its LDS accesses complete in order, so the next level reads
    // these writes without a barrier
    __builtin_amdgcn_wave_barrier();
    if (level == 0) break;
    p0 = cnt;
    np = level;
    cnt += level;
  }
  return cnt;
}

// u before v (u != v) in the expansion order: higher score; equal scores, the
// parent taken earlier (the same comparison one level up), then the lower rank.
__device__ __forceinline__ bool bt_before(const double* S, const uint32_t* meta, int u, int v) {
  for (;;) {
    const double su = S[u], sv = S[v];
    if (su != sv) return su > sv;
    const uint32_t mu = meta[u], mv = meta[v];
    const uint32_t pu = mu >> 16, pv = mv >> 16;
    if (pu == pv) return ((mu >> 8) & 0xffu) < ((mv >> 8) & 0xffu);
    if (pu == kBtRoot) return true;
    if (pv == kBtRoot) return false;
    u = (int)pu;
    v = (int)pv;
  }
}

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

// The sequential expansion by one wave, for thresholds no trial value
// isolates.  The live candidates sit in registers, slot j in lane j % 64: each
// expansion takes one (its slot is reused by the new node's rank-0 child) and
// adds at most one (the parent's next rank), so at most n slots are ever used.
// The best candidate is found with each lane comparing its slots and a DPP
// wave reduction over (score, key), the key packing parent, rank, slot and
// depth (lower wins; slots are unique).
__device__ void bt_sequential(const double* lp, const double* lpg, int n, int max_depth, int nc, BtShared& L,
                              int lane) {
  constexpr int SPL = kMaxNodes / 64;
  const double ninf = -__builtin_inf();
  double cs[SPL];
  uint32_t ck[SPL];
#pragma unroll
  for (int u = 0; u < SPL; ++u) {
    cs[u] = ninf;
    ck[u] = 0xffffffffu;
  }
  int nslots = 0;
  if (n > 1 && max_depth >= 1) {
    if (lane == 0) {
      cs[0] = 0.0 + lpg[1 * nc + 0];
      ck[0] = 1u;  // parent 0, rank 0, slot 0, depth 1
    }
    nslots = 1;
  }
  if (lane == 0) {
    L.np_[0] = -1;
    L.nd_[0] = 0;
    L.nr_[0] = 0;
    L.cum[0] = 0.0;
  }
  __builtin_amdgcn_wave_barrier();
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
    const bool child = d < max_depth, sib = r + 1 < nc;
    const double lp_child = lp[(child ? d + 1 : d) * nc + 0];
    const double lp_sib = lp[d * nc + (sib ? r + 1 : r)];
    const double cum_p = L.cum[p];
    const double s_child = child ? sc + lp_child : ninf;
    const uint32_t k_child = child ? (((uint32_t)i << 24) | ((uint32_t)slot << 8) | (uint32_t)(d + 1)) : 0xffffffffu;
    const double s_sib = cum_p + lp_sib;
    const uint32_t k_sib = ((uint32_t)p << 24) | ((uint32_t)(r + 1) << 16) | ((uint32_t)nslots << 8) | (uint32_t)d;
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
      L.np_[i] = p;
      L.nd_[i] = d;
      L.nr_[i] = r;
      L.cum[i] = sc;
    }
    nslots += sib ? 1 : 0;
    __builtin_amdgcn_wave_barrier();
  }
}

template <bool IN_LDS>
__global__ void __launch_bounds__(kBtWaves * 64) build_tree(const BuildArgs a) {
  __shared__ BtShared L;
  const int b = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = a.n, nc = a.n_cand;
  const int nlp = (a.max_depth + 1) * nc;
  const double* lpg = a.lp + (long long)b * nlp;
  if constexpr (IN_LDS)
    for (int j = tid; j < nlp; j += kBtWaves * 64) L.lp[j] = lpg[j];
  const double* lp = IN_LDS ? L.lp : lpg;
  const long long o = (long long)b * n;
  if (tid == 0) {
    a.parent[o] = -1;
    if (a.depth) a.depth[o] = 0;
    if (a.rank) a.rank[o] = 0;
  }
  if (n <= 1) return;  // the root alone (a uniform exit: no barrier follows)
  if (tid == 0) L.done_min = kBtWaves;
  __syncthreads();

  // 1. bracket the threshold
  const double hi = lp[1 * nc + 0];  // the best depth-1 score: no sequence scores higher
  double lo_ok = -__builtin_inf();   // a value at which more than kBtCap sequences score at least as high
  double hi_bad = next_up(hi);       // fewer than n - 1 at or above it (none above hi)
  double geo = 0.125;
  int win = -1;
  // scale of the first round: the spread of the depth-1 list over its first
  // min(n_cand, n) ranks (the answer's distance below hi is of that order)
  const double spread = hi - lp[1 * nc + min(nc, n) - 1];
  const bool scaled = spread > 0.0 && spread < 1e300;
  for (int rnd = 0; rnd < kBtRounds && win < 0; ++rnd) {
    double tau;
    if (rnd == 0 && scaled) {
      double o = 0.4 * spread;  // 0.4 .. 1.67 spreads below hi, 10% apart
      for (int w = 0; w < wave; ++w) o *= 1.1;
      tau = hi - o;
    } else if (rnd == 0) {
      double g = geo;
      for (int w = 1; w < wave; ++w) g *= 1.6;
      tau = wave == 0 ? hi : hi - g;
    } else if (lo_ok == -__builtin_inf()) {
      double g = geo;
      for (int w = 0; w < wave; ++w) g *= 1.6;
      tau = hi_bad - g;  // below every value known to isolate fewer than n - 1
    } else {
      tau = hi_bad - (hi_bad - lo_ok) * (double)(wave + 1) / (double)(kBtWaves + 1);
    }
    const int c = bt_expand(lp, nc, a.max_depth, tau, L.S[wave], L.meta[wave], L.mark[wave],
                            &L.done_min, wave, lane);
    if (lane == 0) {
      L.cnt[wave] = c;
      L.tau[wave] = tau;
      // the waves above this one test lower values: once this count isolates the
      // tree, theirs are not needed (the first wave reaching n - 1 is at most this one)
      if (c >= n - 1 && c <= kBtCap) atomicMin(&L.done_min, wave);
    }
    __syncthreads();
    if (tid == 0) L.done_min = kBtWaves;  // for the next round, which starts after a barrier
    // the first trial value reaching n - 1 (every count loaded at once)
    int cj[kBtWaves];
#pragma unroll
    for (int j = 0; j < kBtWaves; ++j) cj[j] = L.cnt[j];
    int w = -1;
#pragma unroll
    for (int j = kBtWaves - 1; j >= 0; --j) w = cj[j] >= n - 1 ? j : w;
    if (w >= 0) {
      if (L.cnt[w] <= kBtCap) {
        win = w;
      } else {
        lo_ok = L.tau[w];
        if (w > 0) hi_bad = L.tau[w - 1];
      }
    } else {
      hi_bad = L.tau[kBtWaves - 1];  // every value tested isolates fewer than n - 1
      if (lo_ok == -__builtin_inf() && !(rnd == 0 && scaled))
        for (int j = 0; j < kBtWaves; ++j) geo *= 1.6;
    }
    if (win < 0) __syncthreads();  // the lists are rewritten by the next round
  }

  if (win >= 0) {
    // 2. places in the expansion order; the first n - 1 become nodes 1 .. n - 1.
    // The scores are binned (1024 bins over [tau, hi], one per thread; an
    // earlier bin means a strictly higher score), a scan of the bin counts
    // gives every bin its first place, and a node's place is that plus the
    // nodes of its own bin that come before it.
    const int M = L.cnt[win];  // <= kBtCap < one node per thread
    const double* S = L.S[win];
    const uint32_t* meta = L.meta[win];
    // the other waves' score lists are free now
    static_assert(kBtCap * sizeof(double) >= kBtBins * sizeof(int), "a list holds a histogram");
    int* hist = reinterpret_cast<int*>(L.S[(win + 1) % kBtWaves]);
    int* start = reinterpret_cast<int*>(L.S[(win + 2) % kBtWaves]);
    int* bucket = reinterpret_cast<int*>(L.S[(win + 3) % kBtWaves]);
    const double span = hi - L.tau[win];
    const double inv = span > 0.0 ? (double)kBtBins / span : 0.0;  // 0: a single bin
    hist[tid] = 0;
    __syncthreads();
    int bv = 0, slot = 0;
    if (tid < M) {
      const double x = (hi - S[tid]) * inv;  // >= 0: every score is at most hi
      bv = x >= (double)(kBtBins - 1) ? kBtBins - 1 : (x > 0.0 ? (int)x : 0);
      slot = atomicAdd(&hist[bv], 1);  // a place inside the bin (any order: only membership is used)
    }
    __syncthreads();
    {
      const int h = hist[tid];
      const int incl = (int)sel_wave_scan((uint32_t)h);
      if (lane == 63) L.wsum[wave] = incl;
      __syncthreads();
      int before = 0;
#pragma unroll
      for (int w = 0; w < kBtWaves; ++w) before += w < wave ? L.wsum[w] : 0;
      start[tid] = before + incl - h;
    }
    __syncthreads();
    if (tid < M) bucket[start[bv] + slot] = tid;
    __syncthreads();
    if (tid < M) {
      const int b0 = start[bv], nb = hist[bv];
      int pos = b0;
      for (int j = 0; j < nb; ++j) {
        const int u = bucket[b0 + j];
        pos += (u != tid && bt_before(S, meta, u, tid)) ? 1 : 0;
      }
      L.pos[tid] = pos;
    }
    __syncthreads();
    for (int v = tid; v < M; v += kBtWaves * 64) {
      const int p = L.pos[v];
      if (p < n - 1) {
        const uint32_t m = meta[v];
        const uint32_t pv = m >> 16;
        a.parent[o + p + 1] = pv == kBtRoot ? 0 : L.pos[pv] + 1;
        if (a.depth) a.depth[o + p + 1] = (int)(m & 0xffu);
        if (a.rank) a.rank[o + p + 1] = (int)((m >> 8) & 0xffu);
      }
    }
  } else {
    if (wave == 0) bt_sequential(lp, lpg, n, a.max_depth, nc, L, lane);
    __syncthreads();
    for (int t = tid + 1; t < n; t += kBtWaves * 64) {
      a.parent[o + t] = L.np_[t];
      if (a.depth) a.depth[o + t] = L.nd_[t];
      if (a.rank) a.rank[o + t] = L.nr_[t];
    }
  }
}

int launch_build_tree(int B, int n, int max_depth, int n_cand, const double* lp, int32_t* parent, int32_t* depth,
                      int32_t* rank, void* stream) {
  BuildArgs a{lp, parent, depth, rank, n, max_depth, n_cand};
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (B == 0) return 0;
  if ((long long)(max_depth + 1) * n_cand <= kLpLds)
    hipLaunchKernelGGL(build_tree<true>, dim3(B), dim3(kBtWaves * 64), 0, st, a);
  else
    hipLaunchKernelGGL(build_tree<false>, dim3(B), dim3(kBtWaves * 64), 0, st, a);
  return (int)hipGetLastError();
}

}  // namespace sv
