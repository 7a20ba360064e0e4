// Top-k selection of prefix entries by score, one 512-thread workgroup per
// sequence (Vegas §2 step 2 and §2.A: the k-subset with the largest summed
// score is the set of the k largest scores; ties go to the lower index).
//
// The result is the set {i : s_i > tau, or s_i == tau and i <= i_tie}: tau is
// the k-th largest score and i_tie the index of the last kept entry equal to
// it.  Rows of up to 32768 entries stay in registers between passes (loaded
// as coalesced 16-byte chunks), longer rows are re-read from memory each pass.
//
// Fast path:
//   1. load the row, find its minimum and maximum;
//   2. histogram over 2048 bins linear in the score value between them
//      (bin = trunc((s - lo) * 2048 / (hi - lo)), a non-decreasing function of
//      s: every entry of a higher bin beats every entry of a lower one), then
//      the bin beta holding the k-th largest entry and the entries above it;
//   3. collect the entries of bin beta (usually a few dozen) into LDS and rank
//      them by (score descending, index ascending): the last kept one gives
//      (tau, i_tie);
//   4. emit: the kept entries as a bitmap in index order (LDS), each thread
//      then owning a contiguous run of it: popcount, one workgroup scan, and
//      the thread's kept indices written from its offset.
// Linear bins spread typical score distributions over many bins, so the LDS
// histogram atomics see little contention, unlike digits of the float bit
// pattern, which pile most scores into a handful of exponent bins.
//
// Fallback (width of the range not finite, all-equal rows, a threshold bin
// with more than kCand entries): tau by a radix select over order-preserving
// integer keys of the whole row, 11 bits per pass from the top of the
// occupied key range, and i_tie by counting equal entries in index order.
// Histograms use integer atomics only, so the selection never depends on
// thread timing.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

constexpr int kTopkThreads = 512;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kRegRound = kTopkThreads * 64;  // rows up to this length stay in registers
constexpr int kBins = 2048;
constexpr int kCand = 2048;                    // threshold-bin entries held in LDS
constexpr int kRankMax = 256;                  // bins up to this size are ranked pairwise
constexpr int kCandCap = 8192;                 // compacted candidate entries held in LDS
constexpr int kCandWave = kCandCap / kTopkWaves;  // each wave's region of them
constexpr int kMaskWords = 4096;               // selection bitmap of the candidate path (rows <= 131072)

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0) u = 0;  // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {  // inverse of order_key (zero -> +0.0)
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Inclusive scan over the 64 lanes of a wave (DPP row shifts, then row broadcasts).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// Exclusive scan of one value per thread over the workgroup; `sh` holds >= 16 words.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* sh, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const uint32_t inc = wave_incl_scan(x);
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
  for (int v = 0; v < nw; ++v) {
    const uint32_t c = sh[v];
    before += v < w ? c : 0u;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return before + inc - x;
}

// Exclusive scan of one value per thread over the workgroup with a single
// barrier; `slots` (>= kTopkWaves words) must not be reused before the next
// barrier of the caller.
__device__ __forceinline__ uint32_t block_excl_scan1(uint32_t x, uint32_t* slots, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan(x);
  if (lane == 63) slots[w] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int v = 0; v < kTopkWaves; ++v) {
    const uint32_t c = slots[v];
    before += v < w ? c : 0u;
    tot += c;
  }
  *total = tot;
  return before + inc - x;
}

struct TopkShared {
  int32_t stage[kRegRound / 32];  // one round's selection bitmap, in index order
  uint32_t hist[kBins];
  uint32_t cand_key[kCand];
  int32_t cand_idx[kCand];
  float cval[kCandCap + kTopkThreads];  // candidate path: compacted (value, index), per-wave
  int32_t cidx[kCandCap + kTopkThreads];  // regions, then one discard slot per thread
  uint32_t mask[kMaskWords];      // candidate path: selection bitmap over the row
  uint32_t sh[64];
  float fsh[2 * kTopkWaves + 8];
};

// Wave-level suffix search over hist[0, NB) (NB a multiple of 64, the whole
// wave active): the bin holding the kk-th largest entry.  Returns it, with the
// entries in higher bins in *above and those in it in *inbin; -1 when the
// histogram holds fewer than kk entries.  Lane l reads bins NB-1-BPL*l down to
// NB-BPL*(l+1); a lane-order scan of their sums is a count from the top.
template <int NB>
__device__ __forceinline__ int wave_threshold_bin(const uint32_t* hist, uint32_t kk, uint32_t* above,
                                                  uint32_t* inbin) {
  constexpr int BPL = NB / 64;
  const int lane = threadIdx.x & 63;
  uint32_t c[BPL], sum = 0;
#pragma unroll
  for (int q = 0; q < BPL; ++q) {
    c[q] = hist[NB - 1 - BPL * lane - q];
    sum += c[q];
  }
  const uint32_t inc = wave_incl_scan(sum);
  const uint64_t m = __ballot(inc >= kk);
  if (m == 0) return -1;
  const int l0 = __builtin_ctzll(m);
  int bin = -1;
  uint32_t ab = 0, ib = 0;
  if (lane == l0) {
    uint32_t a = inc - sum;
#pragma unroll
    for (int q = 0; q < BPL; ++q) {
      if (bin < 0 && a + c[q] >= kk) {
        bin = NB - 1 - BPL * lane - q;
        ab = a;
        ib = c[q];
      }
      a += c[q];
    }
  }
  *above = (uint32_t)__builtin_amdgcn_readlane((int)ab, l0);
  *inbin = (uint32_t)__builtin_amdgcn_readlane((int)ib, l0);
  return __builtin_amdgcn_readlane(bin, l0);
}

// Suffix search over hist[0, kBins): the bin holding the kk-th largest entry
// (kk >= 1); sets sh[18] = bin, sh[19] = entries in higher bins, sh[20] =
// entries in it, visible after the call.  Thread t owns bins
// kBins-1-BPT*t down to kBins-BPT*(t+1).
__device__ __forceinline__ void find_threshold_bin(TopkShared& S, uint32_t kk) {
  constexpr int BPT = kBins / kTopkThreads;
  const int tid = threadIdx.x;
  uint32_t c[BPT], sum = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    c[q] = S.hist[kBins - 1 - BPT * tid - q];
    sum += c[q];
  }
  uint32_t tot;
  uint32_t above = block_excl_scan(sum, S.sh, &tot);
  if (above < kk && kk <= above + sum) {
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      if (above < kk && kk <= above + c[q]) {
        S.sh[18] = (uint32_t)(kBins - 1 - BPT * tid - q);
        S.sh[19] = above;
        S.sh[20] = c[q];
      }
      above += c[q];
    }
  }
  __syncthreads();
}

// Radix select of the kk-th largest of the keys that for_each_key(add) feeds
// to add(key) (all in [kmin, kmax]), 11 bits per pass from the top of the
// range.  Returns that key; *need gets how many entries equal to it are among
// the kk largest.
template <typename F>
__device__ __forceinline__ uint32_t radix_select(TopkShared& S, uint32_t kmin, uint32_t kmax, uint32_t kk,
                                                 F&& for_each_key, uint32_t* need) {
  const int tid = threadIdx.x;
  const uint32_t range = kmax - kmin;
  const int nbits = range == 0 ? 0 : 32 - __builtin_clz(range);
  uint32_t prefix = 0, pmask = 0;
  for (int hi = nbits; hi > 0;) {
    const int lo = hi > 11 ? hi - 11 : 0;
    const uint32_t dmask = (1u << (hi - lo)) - 1u;
    for (int i = tid; i < kBins; i += kTopkThreads) S.hist[i] = 0;
    __syncthreads();
    for_each_key([&](uint32_t key) {
      const uint32_t d = key - kmin;
      if ((d & pmask) == prefix) atomicAdd(&S.hist[(d >> lo) & dmask], 1u);
    });
    __syncthreads();
    find_threshold_bin(S, kk);
    prefix |= S.sh[18] << lo;
    kk -= S.sh[19];
    pmask |= dmask << lo;
    __syncthreads();
    hi = lo;
  }
  *need = kk;
  return prefix + kmin;
}

// Rank cut among the C entries of S.cand_key / S.cand_idx (C <= kRankMax): the
// entry beaten by exactly krem - 1 others (a larger key, or an equal key at a
// lower index) is the last kept one.  Returns its key; *i_tie gets its index.
__device__ __forceinline__ uint32_t rank_cut(TopkShared& S, uint32_t C, uint32_t krem, int* i_tie) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kRankMax; i += kTopkThreads) S.hist[i] = 0;
  __syncthreads();
  constexpr int PARTS = kTopkThreads / kRankMax, SPANR = kRankMax / PARTS;
  const int j = tid % kRankMax, part = tid / kRankMax;
  if (j < (int)C) {
    const uint32_t kj = S.cand_key[j];
    const int ij = S.cand_idx[j];
    uint32_t rank = 0;
    const int i1 = min((int)C, part * SPANR + SPANR);
    int i = part * SPANR;
    for (; i + 8 <= i1; i += 8) {
      uint32_t ki[8];
      int ii[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        ki[u] = S.cand_key[i + u];
        ii[u] = S.cand_idx[i + u];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) rank += (ki[u] > kj || (ki[u] == kj && ii[u] < ij)) ? 1u : 0u;
    }
    for (; i < i1; ++i) {
      const uint32_t ki = S.cand_key[i];
      rank += (ki > kj || (ki == kj && S.cand_idx[i] < ij)) ? 1u : 0u;
    }
    atomicAdd(&S.hist[j], rank);
  }
  __syncthreads();
  if (tid < (int)C && S.hist[tid] == krem - 1) {
    S.sh[22] = S.cand_key[tid];
    S.sh[23] = (uint32_t)S.cand_idx[tid];
  }
  __syncthreads();
  *i_tie = (int)S.sh[23];
  return S.sh[22];
}

// Radix cut over the (order key, index) pairs that for_each(f) passes to
// f(key, idx): the kk-th largest key (kk >= 1, at most the number of pairs),
// and in *i_tie the index of the last kept pair equal to it (the need-th
// smallest index among the pairs with that key).
template <typename F>
__device__ __forceinline__ uint32_t radix_cut(TopkShared& S, uint32_t kk, F&& for_each, int* i_tie) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for_each([&](uint32_t key, int) {
    kmin = min(kmin, key);
    kmax = max(kmax, key);
  });
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0) {
    S.fsh[wave] = __uint_as_float(kmin);
    S.fsh[kTopkWaves + wave] = __uint_as_float(kmax);
  }
  __syncthreads();
  kmin = __float_as_uint(S.fsh[0]);
  kmax = __float_as_uint(S.fsh[kTopkWaves]);
  for (int w = 1; w < kTopkWaves; ++w) {
    kmin = min(kmin, __float_as_uint(S.fsh[w]));
    kmax = max(kmax, __float_as_uint(S.fsh[kTopkWaves + w]));
  }
  __syncthreads();
  uint32_t need;
  const uint32_t tau = radix_select(S, kmin, kmax, kk, [&](auto&& add) {
    for_each([&](uint32_t key, int) { add(key); });
  }, &need);
  // indices are distinct: the need-th smallest index is the need-th largest ~index
  uint32_t unused;
  const uint32_t nidx = radix_select(S, 0u, 0xffffffffu, need, [&](auto&& add) {
    for_each([&](uint32_t key, int idx) {
      if (key == tau) add(~(uint32_t)idx);
    });
  }, &unused);
  *i_tie = (int)~nidx;
  return tau;
}

// NR > 0: the row (at most NR rounds) is held in registers across passes;
// NR == 0: every pass streams the row from memory.  A round is
// kTopkThreads * PL consecutive entries; wave w loads the span
// [w * 64 * PL, (w + 1) * 64 * PL) of it as 16-byte chunks, chunk q * 64 + lane
// of the span going to lane `lane` (coalesced loads), so register x[4 q + e]
// holds entry  w * 64 * PL + 4 * (q * 64 + lane) + e  of the round.
template <int NR, int PL>
__device__ __forceinline__ void topk_row(TopkShared& S, const float* __restrict__ s, int P, int k,
                                         int32_t* __restrict__ out) {
  constexpr int kRound = kTopkThreads * PL;
  constexpr int kSpan = 64 * PL;
  constexpr int NQ = PL / 4;
  constexpr int WPT = PL / 32;  // bitmap words per thread in the ordered emit
  constexpr int NRR = NR > 0 ? NR : 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nrounds = (P + kRound - 1) / kRound;
  const bool vec = (reinterpret_cast<uintptr_t>(s) & 15) == 0;
  float xr[NRR][PL];
  auto entry = [&](int r, int q, int e) { return r * kRound + wave * kSpan + 4 * (q * 64 + lane) + e; };
  auto load = [&](int r, float (&x)[PL]) {  // past the row end: NaN (scores are finite)
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int i = entry(r, q, 0);
      if (vec && i + 4 <= P) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(s + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * q + e] = v[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * q + e] = i + e < P ? s[i + e] : __builtin_nanf("");
      }
    }
  };
  auto rounds = [&](auto&& f) {  // f(r, x) over every round, values from registers or memory
    if constexpr (NR > 0) {
#pragma unroll
      for (int r = 0; r < NR; ++r)
        if (r < nrounds) f(r, xr[r]);
    } else {  // two buffers: round r + 1 is in flight while round r is processed
      float xb[PL];
      if (nrounds > 0) load(0, xr[0]);
#pragma unroll 1
      for (int r = 0; r < nrounds; r += 2) {
        if (r + 1 < nrounds) load(r + 1, xb);
        f(r, xr[0]);
        if (r + 1 < nrounds) {
          if (r + 2 < nrounds) load(r + 2, xr[0]);
          f(r + 1, xb);
        }
      }
    }
  };
  // Bitmap of pred over round r in index order (S.stage reused as kRound / 32
  // words), then thread t's contiguous entries [t * PL, t * PL + PL) of the
  // round as WPT words.  Ends with every thread holding its words.
  uint32_t* bits = reinterpret_cast<uint32_t*>(S.stage);
  auto owned_bits = [&](int r, const float(&x)[PL], auto&& pred, uint32_t (&wv)[WPT]) {
    for (int j = tid; j < kRound / 32; j += kTopkThreads) bits[j] = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      uint32_t nib = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) nib |= pred(x[4 * q + e], entry(r, q, e)) ? (1u << e) : 0u;
      const int c = wave * kSpan + 4 * (q * 64 + lane);  // round-relative first entry of the chunk
      if (nib) atomicOr(&bits[c >> 5], nib << (c & 31));
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < WPT; ++j) wv[j] = bits[tid * WPT + j];
  };

  // ---- candidate path (k <= kCandCap / 2, rows up to kMaskWords * 32).
  // A strided sample places a band [t_lo, t_hi] that should hold the k-th
  // largest entry (a little more than k entries of the row above t_lo, a
  // little less than k above t_hi).  Rows longer than kCandCap keep only their
  // entries >= t_lo (compacted into LDS); shorter rows keep every entry.  The
  // cut then bins the kept entries inside the band (entries above t_hi are
  // only counted), ranks the threshold bin, and the emit sets the kept
  // entries' bits in a bitmap over the row.  Whenever an estimate misses (too
  // few or too many kept entries, the cut outside the band, a crowded bin) a
  // slower exact step takes over: a radix cut over the kept entries, or the
  // full-row path below.  The compaction predicate is monotone in the value,
  // so once at least k entries are kept, the k largest and every entry tied
  // with the k-th are among them.  Single waves take the small sequential
  // steps (band bins, threshold bin, ranking) so the workgroup meets few
  // barriers.
  const bool cand = k <= kCandCap / 2 && P <= kMaskWords * 32;
  const bool compact = cand && P > kCandCap;
  constexpr int SPT = NR > 0 ? 2 : 8;           // sampled entries per thread (more for longer rows)
  constexpr int kSample = SPT * kTopkThreads;
  float smp[SPT];
  if (cand) {  // issued before the row, so they return first
#pragma unroll
    for (int u = 0; u < SPT; ++u) smp[u] = s[(int)((long long)(SPT * tid + u) * P / kSample)];
  }
  if constexpr (NR > 0) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
      if (r < nrounds) load(r, xr[r]);
  }
  if (cand) {
    const int nwords = (P + 31) >> 5;
    for (int i = tid; i < kBins; i += kTopkThreads) S.hist[i] = 0;
    for (int j = tid; j < nwords; j += kTopkThreads) S.mask[j] = 0;
    if (tid == 0) S.sh[24] = 0;
    // sample band: the sample's range, 256 value bins over it, then wave 0
    // finds the bins of the sample ranks r + 4 sqrt(r) + 4 (t_lo = that bin's
    // lower edge) and r - 4 sqrt(r) (t_hi = that bin's upper edge), where
    // r = k kSample / P is where the k-th largest entry is expected among the
    // samples (about Poisson-distributed, so 4 sqrt(r) is four deviations)
    uint32_t* sb = S.cand_key;  // 256 bins
    if (tid < 256) sb[tid] = 0;
    float a0 = __builtin_inff(), a1 = -__builtin_inff();
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
      a0 = fminf(a0, smp[u]);  // NaN skipped
      a1 = fmaxf(a1, smp[u]);
    }
    a0 = wave_min(a0);
    a1 = wave_max(a1);
    if (lane == 0) {
      S.fsh[wave] = a0;
      S.fsh[kTopkWaves + wave] = a1;
    }
    __syncthreads();
    float smin = S.fsh[0], smax = S.fsh[kTopkWaves];
#pragma unroll
    for (int w = 1; w < kTopkWaves; ++w) {
      smin = fminf(smin, S.fsh[w]);
      smax = fmaxf(smax, S.fsh[kTopkWaves + w]);
    }
    const float sw = smax - smin;
    const float sbs = 256.f / sw;
    const bool sok = sw > 0.f && sw < __builtin_inff() && sbs < __builtin_inff();
    if (sok) {
#pragma unroll
      for (int u = 0; u < SPT; ++u) {
        const float b = (smp[u] - smin) * sbs;
        if (smp[u] == smp[u]) atomicAdd(&sb[b < 255.f ? (int)b : 255], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) {
      float tl = smin, th = smax;
      if (sok) {
        const float rk = (float)k * (float)kSample / (float)P;  // expected sample rank of the cut
        const float dev = 4.f * __builtin_sqrtf(rk);
        const uint32_t want_lo = (uint32_t)fminf(rk + dev + 4.f, (float)kSample);
        const uint32_t want_hi = (uint32_t)fmaxf(rk - dev, 1.f);
        uint32_t ab, ib;
        const int bh = wave_threshold_bin<256>(sb, want_hi, &ab, &ib);
        const int bl = wave_threshold_bin<256>(sb, want_lo, &ab, &ib);
        tl = smin + sw * ((float)(bl > 0 ? bl : 0) * (1.f / 256.f));
        th = bh >= 0 ? fminf(smin + sw * ((float)(bh + 1) * (1.f / 256.f)), smax) : smax;
      }
      if (lane == 0) {
        S.fsh[2 * kTopkWaves] = tl;
        S.fsh[2 * kTopkWaves + 1] = th;
      }
    }
    __syncthreads();
    const float t_lo = S.fsh[2 * kTopkWaves], t_hi = S.fsh[2 * kTopkWaves + 1];

    // compaction without branches.  Long rows: wave w appends its entries
    // >= t_lo to its region [w * kCandWave, (w + 1) * kCandWave) at ballot
    // positions.  Short rows: every entry sits at its own index, so region w
    // holds entries [w * kCandWave, (w + 1) * kCandWave).  Lanes with nothing
    // to keep write their discard slot.
    uint32_t wbase = 0;  // wave-uniform
    const int discard = kCandCap + tid;
    if (compact) {
      rounds([&](int r, const float(&x)[PL]) {
#pragma unroll
        for (int e = 0; e < PL; ++e) {
          const bool pr = x[e] >= t_lo;  // NaN padding: no
          const uint64_t m = __ballot(pr);
          const uint32_t pos =
              wbase + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          const int slot = (pr && pos < (uint32_t)kCandWave) ? wave * kCandWave + (int)pos : discard;
          S.cval[slot] = x[e];
          S.cidx[slot] = entry(r, e >> 2, e & 3);
          wbase += (uint32_t)__builtin_popcountll(m);
        }
      });
    } else {
      rounds([&](int r, const float(&x)[PL]) {
#pragma unroll
        for (int e = 0; e < PL; ++e) {
          const int i = entry(r, e >> 2, e & 3);
          const int slot = i < P ? i : discard;
          S.cval[slot] = x[e];
          S.cidx[slot] = i;
        }
      });
    }
    if (lane == 0) S.sh[wave] = wbase;
    __syncthreads();
    uint32_t c_total = 0, nw[kTopkWaves];
    bool fits = true;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) {
      nw[w] = compact ? S.sh[w] : (uint32_t)min(max(P - w * kCandWave, 0), kCandWave);
      c_total += nw[w];
      fits = fits && nw[w] <= (uint32_t)kCandWave;
    }

    if (fits && c_total >= (uint32_t)k) {
      // thread t holds the kept entries of slots t + kTopkThreads * u (u < CPT)
      constexpr int CPT = kCandCap / kTopkThreads;
      static_assert(kCandWave == 2 * kTopkThreads, "two slots of each region per thread");
      bool own[CPT];
      float cv[CPT];
      int ci[CPT];
#pragma unroll
      for (int u = 0; u < CPT; ++u) {  // slot u: region u / 2, offset tid + kTopkThreads * (u % 2)
        const int j = tid + kTopkThreads * u;
        own[u] = (uint32_t)(tid + kTopkThreads * (u & 1)) < nw[u >> 1];
        cv[u] = S.cval[j];
        ci[u] = S.cidx[j];
      }
      // band histogram: kept entries inside [t_lo, t_hi] binned, those above t_hi counted
      constexpr int kBand = 512;  // value bins over the band
      const float bw = t_hi - t_lo;
      const float bbs = (float)kBand / bw;
      const bool band = bw > 0.f && bw < __builtin_inff() && bbs < __builtin_inff();
      auto in_band = [&](float v) { return band && v >= t_lo && v <= t_hi; };  // NaN: no
      auto bbin = [&](float v) {
        const float t = (v - t_lo) * bbs;
        return t < (float)(kBand - 1) ? (int)t : kBand - 1;
      };
      uint32_t above = 0;
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        above += (own[u] && cv[u] > t_hi) ? 1u : 0u;
        if (own[u] && in_band(cv[u])) atomicAdd(&S.hist[bbin(cv[u])], 1u);
      }
      above = wave_sum_u32(above);
      if (lane == 0) S.sh[8 + wave] = above;
      __syncthreads();
      if (wave == 0) {
        uint32_t A = 0;
#pragma unroll
        for (int w = 0; w < kTopkWaves; ++w) A += S.sh[8 + w];
        uint32_t ab = 0, ib = 0;
        const int beta = (band && A < (uint32_t)k) ? wave_threshold_bin<kBand>(S.hist, (uint32_t)k - A, &ab, &ib) : -1;
        if (lane == 0) {
          S.sh[18] = (uint32_t)beta;
          S.sh[19] = A + ab;
          S.sh[20] = ib;
        }
      }
      __syncthreads();
      const int beta = (int)S.sh[18];
      const uint32_t C = S.sh[20];
      const uint32_t krem = (uint32_t)k - S.sh[19];
      uint32_t tau_c = 0;
      int tie_c = -1;
      if (beta >= 0 && C <= (uint32_t)kRankMax) {
        // the threshold bin's entries, ranked by (key descending, index ascending)
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
          if (own[u] && in_band(cv[u]) && bbin(cv[u]) == beta) {
            const uint32_t at = atomicAdd(&S.sh[24], 1u);
            S.cand_key[at] = order_key(cv[u]);
            S.cand_idx[at] = ci[u];
          }
        }
        __syncthreads();
        if (C <= 64u) {
          if (wave == 0) {  // lane j ranks entry j against all C (register broadcasts)
            const bool act = lane < (int)C;
            const uint32_t kj = act ? S.cand_key[lane] : 0u;
            const int ij = act ? S.cand_idx[lane] : 0;
            uint32_t rank = 0;
            for (int i = 0; i < (int)C; ++i) {
              const uint32_t ki = (uint32_t)__builtin_amdgcn_readlane((int)kj, i);
              const int ii = __builtin_amdgcn_readlane(ij, i);
              rank += (ki > kj || (ki == kj && ii < ij)) ? 1u : 0u;
            }
            if (act && rank == krem - 1) {
              S.sh[22] = kj;
              S.sh[23] = (uint32_t)ij;
            }
          }
          __syncthreads();
          tau_c = S.sh[22];
          tie_c = (int)S.sh[23];
        } else {
          tau_c = rank_cut(S, C, krem, &tie_c);
        }
      } else {
        tau_c = radix_cut(S, (uint32_t)k, [&](auto&& f) {
#pragma unroll
          for (int u = 0; u < CPT; ++u)
            if (own[u]) f(order_key(cv[u]), ci[u]);
        }, &tie_c);
      }

      // emit: kept entries as a bitmap over the row (zeroed above), then
      // each thread's contiguous words -> popcount, one scan, indices in order
      const float tf = key_value(tau_c);
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const bool keep = own[u] && (cv[u] > tf || (cv[u] == tf && ci[u] <= tie_c));
        if (keep) atomicOr(&S.mask[ci[u] >> 5], 1u << (ci[u] & 31));
      }
      __syncthreads();
      const int wpt = (nwords + kTopkThreads - 1) / kTopkThreads;  // at most kMaskWords / kTopkThreads
      uint32_t mw[kMaskWords / kTopkThreads];
      uint32_t cnt = 0;
#pragma unroll
      for (int j = 0; j < kMaskWords / kTopkThreads; ++j) {
        const int wi = tid * wpt + j;
        mw[j] = (j < wpt && wi < nwords) ? S.mask[wi] : 0u;
        cnt += (uint32_t)__builtin_popcount(mw[j]);
      }
      uint32_t tot;
      uint32_t pos = block_excl_scan1(cnt, S.sh + 48, &tot);
#pragma unroll
      for (int j = 0; j < kMaskWords / kTopkThreads; ++j) {
        uint32_t m = mw[j];
        while (m) {
          const int bpos = __builtin_ctz(m);
          m &= m - 1;
          if (pos < (uint32_t)k) out[pos] = (tid * wpt + j) * 32 + bpos;
          ++pos;
        }
      }
      return;
    }
    __syncthreads();  // the full-row path below rewrites LDS the candidate path read
  }

  // ---- pass 1: range
  float vmin = __builtin_inff(), vmax = -__builtin_inff();
  rounds([&](int, const float(&x)[PL]) {
#pragma unroll
    for (int e = 0; e < PL; ++e) {  // fminf / fmaxf skip the NaN padding
      vmin = fminf(vmin, x[e]);
      vmax = fmaxf(vmax, x[e]);
    }
  });
  vmin = wave_min(vmin);
  vmax = wave_max(vmax);
  if (lane == 0) {
    S.fsh[wave] = vmin;
    S.fsh[kTopkWaves + wave] = vmax;
  }
  for (int i = tid; i < kBins; i += kTopkThreads) S.hist[i] = 0;
  if (tid == 0) S.sh[24] = 0;
  __syncthreads();
  vmin = S.fsh[0];
  vmax = S.fsh[kTopkWaves];
#pragma unroll
  for (int w = 1; w < kTopkWaves; ++w) {
    vmin = fminf(vmin, S.fsh[w]);
    vmax = fmaxf(vmax, S.fsh[kTopkWaves + w]);
  }
  const float width = vmax - vmin;
  bool fast = width > 0.f && width < __builtin_inff();
  const float bscale = fast ? (float)kBins / width : 0.f;
  fast = fast && bscale < __builtin_inff();
  auto bin_of = [&](float x) -> int {  // x >= vmin: non-negative and non-decreasing in x
    const float t = (x - vmin) * bscale;
    return t < (float)(kBins - 1) ? (int)t : kBins - 1;
  };

  uint32_t tau_key = 0;  // order key of the k-th largest entry
  int i_tie = -1;        // index of the last kept entry equal to it
  bool have_cut = false;

  if (fast) {
    // ---- pass 2: value histogram, threshold bin
    rounds([&](int, const float(&x)[PL]) {
#pragma unroll
      for (int e = 0; e < PL; ++e)
        if (x[e] == x[e]) atomicAdd(&S.hist[bin_of(x[e])], 1u);
    });
    __syncthreads();
    find_threshold_bin(S, (uint32_t)k);
    const int beta = (int)S.sh[18];
    const uint32_t above = S.sh[19], C = S.sh[20];
    const uint32_t krem = (uint32_t)k - above;  // 1 <= krem <= C
    __syncthreads();
    if (C <= (uint32_t)kCand) {
      // ---- pass 3: collect bin beta (any order: candidates carry their index)
      rounds([&](int r, const float(&x)[PL]) {
        uint64_t mask = 0;
#pragma unroll
        for (int e = 0; e < PL; ++e) mask |= (x[e] == x[e] && bin_of(x[e]) == beta ? 1ull : 0ull) << e;
        while (mask) {
          const int b = __builtin_ctzll(mask);
          mask &= mask - 1;
          float xe = 0.f;
#pragma unroll
          for (int q = 0; q < PL; ++q) xe = q == b ? x[q] : xe;
          const uint32_t pos = atomicAdd(&S.sh[24], 1u);
          S.cand_key[pos] = order_key(xe);
          S.cand_idx[pos] = entry(r, b >> 2, b & 3);
        }
      });
      __syncthreads();
      if (C <= (uint32_t)kRankMax) {
        tau_key = rank_cut(S, C, krem, &i_tie);
      } else {
        // the krem-th largest key among the candidates, then the index of the
        // last kept candidate equal to it
        tau_key = radix_cut(S, krem, [&](auto&& f) {
          for (uint32_t j = tid; j < C; j += kTopkThreads) f(S.cand_key[j], S.cand_idx[j]);
        }, &i_tie);
      }
      have_cut = true;
    }
  }

  if (!have_cut) {
    // ---- fallback: tau over the order keys of the whole row, then i_tie = the
    // need-th entry equal to tau in index order
    uint32_t need;
    tau_key = radix_select(S, order_key(vmin), order_key(vmax), (uint32_t)k, [&](auto&& add) {
      rounds([&](int, const float(&x)[PL]) {
#pragma unroll
        for (int e = 0; e < PL; ++e)
          if (x[e] == x[e]) add(order_key(x[e]));
      });
    }, &need);
    const float tf = key_value(tau_key);
    uint32_t seen = 0;
    if (tid == 0) S.sh[23] = 0;
    rounds([&](int r, const float(&x)[PL]) {
      uint32_t wv[WPT];
      owned_bits(r, x, [&](float v, int) { return v == tf; }, wv);
      uint32_t c = 0;
#pragma unroll
      for (int j = 0; j < WPT; ++j) c += (uint32_t)__builtin_popcount(wv[j]);
      uint32_t tot;
      uint32_t before = seen + block_excl_scan(c, S.sh, &tot);
      if (before < need && need <= before + c) {
#pragma unroll
        for (int j = 0; j < WPT; ++j) {
          uint32_t m = wv[j];
          while (m) {
            const int bpos = __builtin_ctz(m);
            m &= m - 1;
            if (++before == need) S.sh[23] = (uint32_t)(r * kRound + tid * PL + 32 * j + bpos);
          }
        }
      }
      seen += tot;
    });
    __syncthreads();
    i_tie = (int)S.sh[23];
  }

  // ---- emit in increasing index order
  const float tf = key_value(tau_key);
  uint32_t carry = 0;
  rounds([&](int r, const float(&x)[PL]) {
    uint32_t wv[WPT];
    owned_bits(r, x, [&](float v, int i) { return v > tf || (v == tf && i <= i_tie); }, wv);  // NaN: false
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < WPT; ++j) c += (uint32_t)__builtin_popcount(wv[j]);
    uint32_t tot;
    uint32_t pos = carry + block_excl_scan(c, S.sh, &tot);
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      uint32_t m = wv[j];
      while (m) {
        const int bpos = __builtin_ctz(m);
        m &= m - 1;
        if (pos < (uint32_t)k) out[pos] = r * kRound + tid * PL + 32 * j + bpos;
        ++pos;
      }
    }
    carry += tot;
  });
}

// NR and PL as in topk_row; the host picks them from P_max (every row is at most P_max long)
template <int NR, int PL>
__global__ void __launch_bounds__(kTopkThreads) topk_kernel(const float* __restrict__ scores, int P_max,
                                                           const int32_t* __restrict__ prefix_len,
                                                           const int32_t* __restrict__ kreq, int k_max,
                                                           int32_t* __restrict__ idx, int32_t* __restrict__ count) {
  __shared__ TopkShared S;
  const int b = blockIdx.x, tid = threadIdx.x;
  int P = prefix_len[b];
  P = P < 0 ? 0 : (P > P_max ? P_max : P);
  int k = kreq[b];
  k = k < 0 ? 0 : k;
  k = k > P ? P : k;
  k = k > k_max ? k_max : k;
  const float* s = scores + (long long)b * P_max;
  int32_t* out = idx + (long long)b * k_max;
  if (tid == 0 && count) count[b] = k;
  if (k == 0 || k == P) {
    for (int i = tid; i < k_max; i += kTopkThreads) out[i] = i < k ? i : -1;
    return;
  }
  topk_row<NR, PL>(S, s, P, k, out);
  for (int i = k + tid; i < k_max; i += kTopkThreads) out[i] = -1;
}

int launch_topk(const float* scores, int B, int P_max, const int32_t* prefix_len, const int32_t* k,
                int k_max, int32_t* idx, int32_t* count, void* ws, void* stream) {
  (void)ws;
  (void)hipGetLastError();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (B > 0 && P_max <= kRegRound)
    hipLaunchKernelGGL((topk_kernel<1, 64>), dim3(B), dim3(kTopkThreads), 0, st, scores, P_max, prefix_len, k,
                       k_max, idx, count);
  else if (B > 0)
    hipLaunchKernelGGL((topk_kernel<0, 32>), dim3(B), dim3(kTopkThreads), 0, st, scores, P_max, prefix_len, k,
                       k_max, idx, count);
  return (int)hipGetLastError();
}

size_t topk_workspace_bytes(int B, int P_max) {
  (void)B;
  (void)P_max;
  return 0;
}

bool topk_supported(int P_max) { return P_max >= 0; }

}  // namespace sv
