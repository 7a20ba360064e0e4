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

struct TopkShared {
  int32_t stage[kRegRound / 32];  // one round's selection bitmap, in index order
  uint32_t hist[kBins];
  uint32_t cand_key[kCand];
  int32_t cand_idx[kCand];
  uint32_t sh[32];
  float fsh[2 * kTopkWaves];
};

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
    } else {
#pragma unroll 1
      for (int r = 0; r < nrounds; ++r) {
        load(r, xr[0]);
        f(r, xr[0]);
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

  // ---- pass 1: range
  if constexpr (NR > 0) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
      if (r < nrounds) load(r, xr[r]);
  }
  float vmin = __builtin_inff(), vmax = -__builtin_inff();
  rounds([&](int, const float(&x)[PL]) {
#pragma unroll
    for (int e = 0; e < PL; ++e) {  // fminf / fmaxf skip the NaN padding
      vmin = fminf(vmin, x[e]);
      vmax = fmaxf(vmax, x[e]);
    }
  });
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    vmin = fminf(vmin, __shfl_xor(vmin, o));
    vmax = fmaxf(vmax, __shfl_xor(vmax, o));
  }
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
        // rank of candidate j = number of candidates beating it (larger key, or equal key at a lower index)
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
        tau_key = S.sh[22];
        i_tie = (int)S.sh[23];
      } else {
        // radix select of the krem-th largest key among the candidates, then
        // the need-th smallest index among the candidates equal to it
        uint32_t cmin = 0xffffffffu, cmax = 0u;
        for (uint32_t j = tid; j < C; j += kTopkThreads) {
          cmin = min(cmin, S.cand_key[j]);
          cmax = max(cmax, S.cand_key[j]);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          cmin = min(cmin, (uint32_t)__shfl_xor((int)cmin, o));
          cmax = max(cmax, (uint32_t)__shfl_xor((int)cmax, o));
        }
        if (lane == 0) {
          S.fsh[wave] = __uint_as_float(cmin);
          S.fsh[kTopkWaves + wave] = __uint_as_float(cmax);
        }
        __syncthreads();
        cmin = __float_as_uint(S.fsh[0]);
        cmax = __float_as_uint(S.fsh[kTopkWaves]);
        for (int w = 1; w < kTopkWaves; ++w) {
          cmin = min(cmin, __float_as_uint(S.fsh[w]));
          cmax = max(cmax, __float_as_uint(S.fsh[kTopkWaves + w]));
        }
        __syncthreads();
        uint32_t need;
        tau_key = radix_select(S, cmin, cmax, krem, [&](auto&& add) {
          for (uint32_t j = tid; j < C; j += kTopkThreads) add(S.cand_key[j]);
        }, &need);
        // indices are distinct: the need-th smallest index is the need-th largest ~index
        const uint32_t tk = tau_key;
        uint32_t unused;
        const uint32_t nidx = radix_select(S, 0u, 0xffffffffu, need, [&](auto&& add) {
          for (uint32_t j = tid; j < C; j += kTopkThreads)
            if (S.cand_key[j] == tk) add(~(uint32_t)S.cand_idx[j]);
        }, &unused);
        i_tie = (int)~nidx;
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
