// Top-k selection over many workgroups (Vegas §2 step 2 and §2.A: the
// k-subset with the largest summed score is the set of the k largest scores;
// ties go to the lower index).  Device pieces shared by the selection kernels
// and by the verify merge kernel, which runs the first pass on the scores it
// has just summed.
//
// A row of P scores is cut into blocks of 2048 entries, 4096 for rows longer
// than 65536 (a row has at most 32 blocks), and 1024 when k is more than an
// eighth of a row of up to 32768 (a block's share must fit its slots).
//   Pass A, one workgroup per block: every workgroup of a row computes the
//     same band [t_lo, t_hi] from the same sample of the row (the k-th largest
//     entry is expected inside it), and writes its block's entries at or
//     above t_lo, in index order, to the block's kSelCap fixed slots in the
//     workspace, with the number of them and the number above t_hi.
//   Pass B, one workgroup per row: one trip to memory for every block's
//     counts and slots (at fixed places, so no load waits for a count); the
//     k-th largest entry tau and the index i_tie of the last kept entry equal
//     to it (ties to lower indices) among the band entries; then each block's
//     kept slots (s > tau, or s == tau and i <= i_tie), in order, at the
//     block's offset (the kept entries of the blocks before it).
// When the band misses (fewer than k entries at or above t_lo, at least k
// above t_hi, a block with more entries than its slots, or a crowded
// threshold bin), and for short rows, pass B runs an exact radix selection
// over the whole row instead.  Only integer atomics on LDS are used, and every
// cross-workgroup result is written once and read after a kernel boundary, so
// no result depends on the order in which workgroups run.
#pragma once

#include "sv_device.h"

namespace sv {

constexpr int kSelThreads = 256;       // pass A
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelThreadsB = 1024;     // pass B (four waves per SIMD hide its latency chains)
constexpr int kSelCap = 512;           // slots per block (its entries >= t_lo)
constexpr int kSelMinP = 4096;         // rows up to this length take the radix path
constexpr int kSelSampleBins = 512;    // value bins over the sample's range (and over the band)
constexpr int kSelMaxBlocks = 32;      // blocks per row
constexpr int kSelMaxP = 32 * 4096;    // rows up to this length take the two-pass path
constexpr int kSelRankMax = 64;        // threshold-bin entries ranked by one wave

// Per-row result of pass A: the band (every block computes the same one).
struct SelBand {
  float t_lo, t_hi;
  int32_t pad[2];
};

// Workspace of the two passes for B rows.
struct SelWs {
  SelBand* band;    // [B]
  int32_t* above;   // [B][kSelMaxBlocks]: entries above t_hi
  int32_t* nge;     // [B][kSelMaxBlocks]: entries >= t_lo (more than kSelCap: overflow)
  float* cv;        // [B][kSelMaxBlocks][kSelCap]: their values, in index order ...
  int32_t* ci;      // [B][kSelMaxBlocks][kSelCap]: ... and indices
};

__host__ __device__ inline size_t sel_align(size_t x) { return (x + 255) / 256 * 256; }
// Workspace bytes of B rows, and the layout at `base`.
__host__ __device__ inline size_t sel_ws_bytes(int B) {
  size_t off = sel_align((size_t)B * sizeof(SelBand));
  off = sel_align(off + (size_t)B * kSelMaxBlocks * 4);
  off = sel_align(off + (size_t)B * kSelMaxBlocks * 4);
  off = sel_align(off + (size_t)B * kSelMaxBlocks * kSelCap * 4);
  off = sel_align(off + (size_t)B * kSelMaxBlocks * kSelCap * 4);
  return off;
}
__host__ __device__ inline SelWs sel_ws_at(void* base, int B) {
  SelWs w{};
  char* p = reinterpret_cast<char*>(base);
  size_t off = 0;
  w.band = reinterpret_cast<SelBand*>(p + off);
  off = sel_align(off + (size_t)B * sizeof(SelBand));
  w.above = reinterpret_cast<int32_t*>(p + off);
  off = sel_align(off + (size_t)B * kSelMaxBlocks * 4);
  w.nge = reinterpret_cast<int32_t*>(p + off);
  off = sel_align(off + (size_t)B * kSelMaxBlocks * 4);
  w.cv = reinterpret_cast<float*>(p + off);
  off = sel_align(off + (size_t)B * kSelMaxBlocks * kSelCap * 4);
  w.ci = reinterpret_cast<int32_t*>(p + off);
  return w;
}

// block length of a row: 2048 entries up to 65536, 4096 above (at most 32
// blocks); 1024 for rows up to 32768 whose k is more than an eighth of the row,
// so that a block's share of the kept entries and the band stays within its
// 512 slots (with 2048-entry blocks the 8192-entry row at k = 2048 overflowed
// them and fell back to the radix path; smaller blocks everywhere cost the
// 32768-entry row 1.6 us)
__host__ __device__ inline int sel_blk(int P, int k) {
  return P > 65536 ? 4096 : ((P <= 32768 && 8LL * k > P) ? 1024 : 2048);
}
// sample of 2048 entries (4096 for rows above 65536): 256 segments of 8 (16)
// consecutive entries on 256 threads, nseg segments of sel_seg(P) * 256 / nseg
__host__ __device__ inline int sel_seg(int P) { return P > 65536 ? 16 : 8; }
// first entry of segment t of nseg (segments of seg entries spread over the
// row, all inside it; a multiple of 4 when seg is)
__device__ __forceinline__ int sel_seg_start(int t, int P, int seg, int nseg) {
  return (int)((long long)t * (P - seg) / (nseg - 1)) & (seg % 4 == 0 ? ~3 : ~1);
}

// k' = min(k, P, k_max) of a row, with P clamped to [0, P_max] and k to >= 0
__device__ __forceinline__ void sel_row_sizes(const int32_t* prefix_len, const int32_t* kreq, int b, int P_max,
                                              int k_max, int* P, int* k) {
  int p = prefix_len[b];
  int kk = kreq[b];  // both loads in flight before either is used
  p = p < 0 ? 0 : (p > P_max ? P_max : p);
  kk = kk < 0 ? 0 : kk;
  kk = kk > p ? p : kk;
  kk = kk > k_max ? k_max : kk;
  *P = p;
  *k = kk;
}

// Does the row take the two-pass path?  (Otherwise pass B does the whole row
// by radix selection: short rows, k = 0 and k = P.)
__device__ __forceinline__ bool sel_multi(int P, int k) { return P > kSelMinP && P <= kSelMaxP && k > 0 && k < P; }

// Order-preserving integer key of a float (-0.0 == +0.0) and its inverse.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// hist[bin] += 1 for every lane of the wave with `hit`.  When all of them hold
// the same bin (rows of equal scores), one lane adds their number: a whole
// wave's atomics on one LDS address are serialized, and the fallback that rows
// of equal scores take would otherwise spend most of its time there.
__device__ __forceinline__ void sel_hist_add(uint32_t* hist, uint32_t bin, bool hit) {
  const unsigned long long hm = __ballot(hit);
  if (hm == 0ull) return;
  const int first = __builtin_ctzll(hm);
  const uint32_t b0 = (uint32_t)__builtin_amdgcn_readlane((int)bin, first);
  if (__ballot(hit && bin == b0) == hm) {
    if ((int)(threadIdx.x & 63) == first) atomicAdd(&hist[b0], (uint32_t)__builtin_popcountll(hm));
  } else if (hit) {
    atomicAdd(&hist[bin], 1u);
  }
}

// Inclusive scan over the 64 lanes of a wave (DPP row shifts, then row broadcasts).
__device__ __forceinline__ uint32_t sel_wave_scan(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);
  return x;
}

// Suffix search over hist[0, NB) by one whole wave: the bin holding the kk-th
// largest entry; *above gets the entries in higher bins, *inbin those in it.
// -1 when the histogram holds fewer than kk entries.
template <int NB>
__device__ __forceinline__ int sel_wave_bin(const uint32_t* hist, uint32_t kk, uint32_t* above, uint32_t* inbin) {
  constexpr int BPL = NB / 64;
  const int lane = threadIdx.x & 63;
  uint32_t c[BPL], sum = 0;
#pragma unroll
  for (int q = 0; q < BPL; ++q) {
    c[q] = hist[NB - 1 - BPL * lane - q];
    sum += c[q];
  }
  const uint32_t inc = sel_wave_scan(sum);  // lane order = descending bins
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

// LDS of both passes and of the radix path (up to 16 waves)
struct SelShared {
  uint32_t hist[kSelSampleBins];
  uint32_t cand_key[kSelRankMax];
  int32_t cand_idx[kSelRankMax];
  uint32_t bsel[kSelMaxBlocks];  // kept entries per block, then their offsets
  uint32_t sh[64];   // per-wave partials: [0, 16), [16, 32), [48, 64); scans: [32, 48)
  float mm[32];
  float band[2];
  uint32_t ctr;      // threshold-bin entries gathered so far
  uint32_t tau_key;  // the cut: order key of tau ...
  int32_t tau_idx;   // ... and i_tie
  uint32_t rq, rab;  // radix path: the digit, the entries above it
  uint32_t total;    // kept entries of the row
};

// Exclusive scan of one value per thread over a workgroup of NT threads (one
// barrier; L.sh[32..32 + NT / 64) must not be reused before the caller's next
// barrier).
template <int NT>
__device__ __forceinline__ uint32_t sel_block_scan(SelShared& L, uint32_t x, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t inc = sel_wave_scan(x);
  if (lane == 63) L.sh[32 + w] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int v = 0; v < NT / 64; ++v) {
    const uint32_t c = L.sh[32 + v];
    before += v < w ? c : 0u;
    tot += c;
  }
  *total = tot;
  return before + inc - x;
}

// The band of a row from its sample (SPT values per thread, NaN where no
// sample): t_lo = the lower edge of the value bin holding sample rank
// r + 4 sqrt(r) + 4, t_hi = the upper edge of the bin of rank r - 4 sqrt(r),
// with r = k S / P the rank where the k-th largest entry is expected among the
// S samples (about Poisson-distributed, so 4 sqrt(r) is four deviations).
// Ends with a barrier; every thread of the NT gets the same (t_lo, t_hi).
template <int NT, int SPT>
__device__ __forceinline__ void sel_band(SelShared& L, const float (&smp)[SPT], int S, int P, int k, float* t_lo,
                                         float* t_hi) {
  constexpr int NW = NT / 64;
  static_assert(NW <= 16, "wave partials fit L.mm");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kSelSampleBins; i += NT) L.hist[i] = 0;
  float a0 = __builtin_inff(), a1 = -__builtin_inff();
#pragma unroll
  for (int u = 0; u < SPT; ++u) {  // fminf / fmaxf skip NaN
    a0 = fminf(a0, smp[u]);
    a1 = fmaxf(a1, smp[u]);
  }
  a0 = wave_min(a0);
  a1 = wave_max(a1);
  if (lane == 0) {
    L.mm[wave] = a0;
    L.mm[16 + wave] = a1;
  }
  __syncthreads();
  float smin = L.mm[0], smax = L.mm[16];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    smin = fminf(smin, L.mm[w]);
    smax = fmaxf(smax, L.mm[16 + w]);
  }
  const float sw = smax - smin;
  const float sbs = (float)kSelSampleBins / sw;
  const bool sok = sw > 0.f && sw < __builtin_inff() && sbs < __builtin_inff();
  if (sok) {
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
      const float x = (smp[u] - smin) * sbs;
      if (smp[u] == smp[u]) atomicAdd(&L.hist[x < (float)(kSelSampleBins - 1) ? (int)x : kSelSampleBins - 1], 1u);
    }
  }
  __syncthreads();
  if (wave == 0) {
    float tl = smin, th = smax;
    if (sok) {
      const float rk = (float)k * (float)S / (float)P;
      const float dev = 4.f * __builtin_sqrtf(rk);
      const uint32_t want_lo = (uint32_t)fminf(rk + dev + 4.f, (float)S);
      const uint32_t want_hi = (uint32_t)fmaxf(rk - dev, 1.f);
      uint32_t ab, ib;
      const int bh = sel_wave_bin<kSelSampleBins>(L.hist, want_hi, &ab, &ib);
      const int bl = sel_wave_bin<kSelSampleBins>(L.hist, want_lo, &ab, &ib);
      tl = smin + sw * ((float)(bl > 0 ? bl : 0) * (1.f / (float)kSelSampleBins));
      th = bh >= 0 ? fminf(smin + sw * ((float)(bh + 1) * (1.f / (float)kSelSampleBins)), smax) : smax;
    }
    if (lane == 0) {
      L.band[0] = tl;
      L.band[1] = th;
    }
  }
  __syncthreads();
  *t_lo = L.band[0];
  *t_hi = L.band[1];
}

// Pass A's output for one block on NT threads: thread t holds the E entries
// base + E t + e (NaN past the row end), so thread order is index order.  The
// entries >= t_lo go to the block's slots in that order; the counts of them
// and of those above t_hi go to nge / above.  ST(ptr, bits) performs each
// 4-byte workspace store.
template <int NT, int E, typename Store>
__device__ __forceinline__ void sel_compact(SelShared& L, const SelWs& ws, int b, int blk, const float (&x)[E],
                                            int base, float t_lo, float t_hi, Store&& ST) {
  constexpr int NW = NT / 64;
  static_assert(NW <= 16, "wave partials fit L.sh");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t n = 0, above = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    n += x[e] >= t_lo ? 1u : 0u;  // NaN: no
    above += x[e] > t_hi ? 1u : 0u;
  }
  const uint32_t inc = sel_wave_scan(n);
  const uint32_t wab = wave_sum_u32(above);
  if (lane == 63) L.sh[wave] = inc;
  if (lane == 0) L.sh[16 + wave] = wab;
  __syncthreads();
  uint32_t pos = inc - n, total = 0, ab = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t c = L.sh[w];
    pos += w < wave ? c : 0u;
    total += c;
    ab += L.sh[16 + w];
  }
  const long long slot0 = ((long long)b * kSelMaxBlocks + blk) * kSelCap;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (x[e] >= t_lo) {
      if (pos < (uint32_t)kSelCap) {  // past the slots: counted only (pass B falls back)
        ST(reinterpret_cast<uint32_t*>(ws.cv) + slot0 + pos, __float_as_uint(x[e]));
        ST(reinterpret_cast<uint32_t*>(ws.ci) + slot0 + pos, (uint32_t)(base + E * tid + e));
      }
      ++pos;
    }
  }
  if (tid == 0) {
    ST(reinterpret_cast<uint32_t*>(ws.above) + (long long)b * kSelMaxBlocks + blk, ab);
    ST(reinterpret_cast<uint32_t*>(ws.nge) + (long long)b * kSelMaxBlocks + blk, total);
  }
}

// Exact selection over a whole row by one workgroup (short rows, k = 0 or P,
// and rows whose band missed): tau = the k-th largest order key by four radix
// passes of 8 bits from the top, then each thread's contiguous run of the row
// keeps its entries above tau and, in index order, as many entries equal to
// tau as are still needed.  NaN entries are never kept (unless k = P), so a
// row with fewer than k others yields fewer than k indices; `count` says how
// many.  VAL(i) returns entry i of the row.
template <int NT, typename Val>
__device__ __forceinline__ void sel_radix_row(SelShared& L, int P, int k, int k_max, int32_t* __restrict__ out,
                                              int32_t* __restrict__ count, int b, Val&& VAL) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (k == 0 || k == P) {
    for (int i = tid; i < k_max; i += NT) out[i] = i < k ? i : -1;
    if (tid == 0 && count) count[b] = k;
    return;
  }
  uint32_t prefix = 0, pmask = 0, need = (uint32_t)k;
  bool all_valid = false;  // fewer than k non-NaN entries: keep them all
  for (int d = 3; d >= 0; --d) {
    for (int i = tid; i < 256; i += NT) L.hist[i] = 0;
    __syncthreads();
    for (int i0 = tid; i0 < P; i0 += 8 * NT) {
      // eight entries per thread loaded together at clamped places, then counted
      // (one entry per step would be one trip to memory each)
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = VAL(min(i0 + u * NT, P - 1));
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t key = order_key(x[u]);
        sel_hist_add(L.hist, (key >> (8 * d)) & 255u, i0 + u * NT < P && x[u] == x[u] && (key & pmask) == prefix);
      }
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t ab = 0, ib = 0;
      const int q = sel_wave_bin<256>(L.hist, need, &ab, &ib);
      if (lane == 0) {
        L.rq = (uint32_t)q;
        L.rab = ab;
      }
    }
    __syncthreads();
    const int q = (int)L.rq;
    if (q < 0) {  // uniform: every thread reads the same word
      all_valid = true;
      break;
    }
    prefix |= (uint32_t)q << (8 * d);
    pmask |= 0xffu << (8 * d);
    need -= L.rab;
    __syncthreads();  // before the histogram is cleared again
  }
  if (all_valid) {
    prefix = 0;  // every non-NaN key is above 0
    need = 0;
  }
  // thread t's run [r0, r1): entries above tau, entries equal to it
  const int r0 = (int)((long long)tid * P / NT), r1 = (int)((long long)(tid + 1) * P / NT);
  uint32_t gt = 0, eq = 0;
  for (int i0 = r0; i0 < r1; i0 += 8) {  // loads in batches of eight, as above
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = VAL(min(i0 + u, r1 - 1));
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t key = order_key(x[u]);
      const bool in = i0 + u < r1 && x[u] == x[u];
      gt += (in && key > prefix) ? 1u : 0u;
      eq += (in && key == prefix && !all_valid) ? 1u : 0u;
    }
  }
  uint32_t tot;
  const uint32_t eq_before = sel_block_scan<NT>(L, eq, &tot);
  const uint32_t take = eq_before >= need ? 0u : min(eq, need - eq_before);
  __syncthreads();  // L.sh[32..] is reused by the next scan
  uint32_t kept_total;
  uint32_t pos = sel_block_scan<NT>(L, gt + take, &kept_total);
  uint32_t eq_seen = eq_before;
  for (int i0 = r0; i0 < r1; i0 += 8) {  // in index order, loads in batches of eight
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = VAL(min(i0 + u, r1 - 1));
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (i0 + u >= r1) break;
      const uint32_t key = order_key(x[u]);
      bool keep = x[u] == x[u] && key > prefix;
      if (x[u] == x[u] && key == prefix && !all_valid) {
        keep = eq_seen < need;
        ++eq_seen;
      }
      if (keep) {
        if (pos < (uint32_t)k) out[pos] = i0 + u;
        ++pos;
      }
    }
  }
  const int emitted = (int)min(kept_total, (uint32_t)k);
  for (int i = emitted + tid; i < k_max; i += NT) out[i] = -1;
  if (tid == 0 && count) count[b] = emitted;
}

// Pass B for one row on NT threads (wave w holds blocks w, w + NW, ...; lane
// l holds slots l, l + 64, ..., of each, so a block's first n slots fill
// whole slot rounds and empty rounds are skipped).  LD(ptr) performs each
// 4-byte workspace load; VAL(i) returns entry i of the row (radix path only).
// The band path of pass B; false (with nothing written) when the band missed
// or the threshold bin is crowded, and the caller runs the radix path.
template <int NT, typename Load>
__device__ __forceinline__ bool sel_pass_b_band(SelShared& L, const SelWs& ws, int P, int k, int k_max,
                                                int32_t* __restrict__ out, int32_t* __restrict__ count, int b,
                                                Load&& LD) {
  static_assert(kSelCap == 64 * 8, "slot geometry");
  constexpr int NW = NT / 64;
  static_assert(NW <= 16 && kSelMaxBlocks % NW == 0, "wave geometry");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int BL = sel_blk(P, k);
  const int nb = (P + BL - 1) / BL;
  constexpr int M = kSelMaxBlocks / NW;  // blocks per wave
  constexpr int RR = kSelCap / 64;              // slot rounds per block
  const int mw = (nb - wave + NW - 1) / NW;  // this wave's blocks (wave-uniform)
  // ---- one trip to memory: every count and slot of this wave's blocks
  int32_t abv[M], nge[M];
  float v[M][RR];
  int32_t ix[M][RR];
  const long long row0 = (long long)b * kSelMaxBlocks;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int j = wave + NW * m;
    abv[m] = 0;
    nge[m] = 0;
    if (m < mw) {
      abv[m] = (int32_t)LD(reinterpret_cast<const uint32_t*>(ws.above) + row0 + j);
      nge[m] = (int32_t)LD(reinterpret_cast<const uint32_t*>(ws.nge) + row0 + j);
#pragma unroll
      for (int r = 0; r < RR; ++r) {
        const long long sl = (row0 + j) * kSelCap + 64 * r + lane;
        v[m][r] = __uint_as_float(LD(reinterpret_cast<const uint32_t*>(ws.cv) + sl));
        ix[m][r] = (int32_t)LD(reinterpret_cast<const uint32_t*>(ws.ci) + sl);
      }
    }
  }
  const float t_lo = __uint_as_float(LD(reinterpret_cast<const uint32_t*>(&ws.band[b].t_lo)));
  const float t_hi = __uint_as_float(LD(reinterpret_cast<const uint32_t*>(&ws.band[b].t_hi)));
  // ---- totals (entries above the band A, inside it C, slot overflow) and the
  // band histogram (512 value bins over [t_lo, t_hi]) in one phase
  constexpr int kBand = kSelSampleBins;
  const float bw = t_hi - t_lo;
  const float bbs = (float)kBand / bw;
  const bool binned = bw > 0.f && bw < __builtin_inff() && bbs < __builtin_inff();
  auto bbin = [&](float x) {
    if (!binned) return 0;
    const float t = (x - t_lo) * bbs;
    return t < (float)(kBand - 1) ? (int)t : kBand - 1;
  };
  auto in_band = [&](int m, int r) { return 64 * r + lane < nge[m] && v[m][r] <= t_hi; };
  for (int i = tid; i < kSelSampleBins; i += NT) L.hist[i] = 0;
  if (tid == 0) L.ctr = 0;
  __syncthreads();
  {
    uint32_t a = 0, c = 0, over = 0;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      if (m < mw) {
        a += (uint32_t)abv[m];
        c += (uint32_t)(nge[m] - abv[m]);
        over |= nge[m] > kSelCap ? 1u : 0u;
#pragma unroll
        for (int r = 0; r < RR; ++r)
          if (64 * r < nge[m] && in_band(m, r)) atomicAdd(&L.hist[bbin(v[m][r])], 1u);
      }
    }
    if (lane == 0) {
      L.sh[wave] = a;
      L.sh[16 + wave] = c;
      L.sh[48 + wave] = over;
    }
  }
  __syncthreads();
  uint32_t A = 0, C = 0, over = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    A += L.sh[w];
    C += L.sh[16 + w];
    over |= L.sh[48 + w];
  }
  if (over || !(A < (uint32_t)k && A + C >= (uint32_t)k)) return false;  // the band missed
  // ---- cut: the (k - A)-th largest band entry by (value descending, index
  // ascending): every wave finds the threshold bin itself, its entries are
  // gathered and ranked by one wave
  const uint32_t kk = (uint32_t)k - A;
  uint32_t ab = 0, Cb = 0;
  const int beta = sel_wave_bin<kBand>(L.hist, kk, &ab, &Cb);
  const uint32_t krem = kk - ab;
  if (Cb > (uint32_t)kSelRankMax) return false;  // a crowded bin (many equal scores)
  // every entry of a bin above the threshold bin (or above the band) is kept:
  // their number per block, and the threshold bin's entries gathered
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if (m < mw) {
      uint32_t t = 0;
#pragma unroll
      for (int r = 0; r < RR; ++r) {
        if (64 * r < nge[m]) {
          const bool live = 64 * r + lane < nge[m];
          t += (uint32_t)__builtin_popcountll(
              __ballot(live && (v[m][r] > t_hi || (in_band(m, r) && bbin(v[m][r]) > beta))));
          if (live && in_band(m, r) && bbin(v[m][r]) == beta) {
            const uint32_t at = atomicAdd(&L.ctr, 1u);
            L.cand_key[at] = order_key(v[m][r]);
            L.cand_idx[at] = ix[m][r];
          }
        }
      }
      if (lane == 0) L.bsel[wave + NW * m] = t;
    }
  }
  __syncthreads();
  if (wave == 0) {
    // lane j ranks entry j of the threshold bin against all Cb (register broadcasts);
    // the entries ranked below krem are kept
    const bool act = lane < (int)Cb;
    const uint32_t kj = act ? L.cand_key[lane] : 0u;
    const int ij = act ? L.cand_idx[lane] : 0;
    uint32_t rank = 0;
    for (int i = 0; i < (int)Cb; ++i) {
      const uint32_t ki = (uint32_t)__builtin_amdgcn_readlane((int)kj, i);
      const int ii = __builtin_amdgcn_readlane(ij, i);
      rank += (ki > kj || (ki == kj && ii < ij)) ? 1u : 0u;
    }
    if (act && rank == krem - 1) {
      L.tau_key = kj;
      L.tau_idx = ij;
    }
    // block offsets: lane j takes block j's count plus its kept threshold-bin entries
    uint64_t km = __ballot(act && rank < krem);
    uint32_t bj = lane < nb ? L.bsel[lane] : 0u;
    while (km) {
      const int i = __builtin_ctzll(km);
      km &= km - 1;
      bj += (lane < nb && __builtin_amdgcn_readlane(ij, i) / BL == lane) ? 1u : 0u;
    }
    const uint32_t binc = sel_wave_scan(bj);
    if (lane < nb) L.bsel[lane] = binc - bj;
    if (lane == 63) L.total = binc;
  }
  __syncthreads();
  const float tf = key_value(L.tau_key);
  const int i_tie = L.tau_idx;
  const uint32_t total = L.total;
  // ---- emit: per block, the kept slots in order at the block's offset
  auto kept = [&](int m, int r) {
    return 64 * r + lane < nge[m] && (v[m][r] > tf || (v[m][r] == tf && ix[m][r] <= i_tie));
  };
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if (m >= mw) break;
    const int j = wave + NW * m;
    uint32_t pos = L.bsel[j];
#pragma unroll
    for (int r = 0; r < RR; ++r) {
      if (64 * r >= nge[m]) break;
      const bool kp = kept(m, r);
      const uint64_t km = __ballot(kp);
      const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(km >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)km, 0u));
      if (kp && pos + below < (uint32_t)k) out[pos + below] = ix[m][r];
      pos += (uint32_t)__builtin_popcountll(km);
    }
  }
  const int emitted = (int)min(total, (uint32_t)k);
  for (int i = emitted + tid; i < k_max; i += NT) out[i] = -1;
  if (tid == 0 && count) count[b] = emitted;
  return true;
}

// Pass B for one row: the band path, or the exact radix path for short rows,
// k = 0 or P, a missed band and a crowded threshold bin.  The radix path has
// one call site, after the band path: a pass-B launch executes its code once,
// so its instruction-cache misses are a large part of its time, and a single,
// trailing copy of the fallback keeps the common path short and contiguous.
template <int NT, typename Load, typename Val>
__device__ __forceinline__ void sel_pass_b_row(SelShared& L, const SelWs& ws, int P, int k, int k_max,
                                               int32_t* __restrict__ out, int32_t* __restrict__ count, int b,
                                               Load&& LD, Val&& VAL) {
  if (sel_multi(P, k) && sel_pass_b_band<NT>(L, ws, P, k, k_max, out, count, b, LD)) return;
  __syncthreads();  // the band path's LDS is reused
  sel_radix_row<NT>(L, P, k, k_max, out, count, b, VAL);
}

}  // namespace sv
