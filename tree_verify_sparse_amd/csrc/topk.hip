// Top-k selection of prefix entries by score, one 1024-thread workgroup per
// sequence (Vegas §2 step 2 and §2.A: the k-subset with the largest summed
// score is the set of the k largest scores).
//
// Scores map to order-preserving 32-bit keys (-0.0 folded onto +0.0).  The
// offsets x = key - min_key are then radix-selected from the most significant
// bit of (max_key - min_key) downward, 11 bits per pass, which finds the exact
// key tau of the k-th largest entry and how many entries equal to tau are
// still needed.  Starting the digits at the top of the occupied key range
// (rather than at bit 31, where sign and exponent bits put nearly all scores
// into a few bins) keeps the LDS histogram atomics spread out.  A final pass
// in index order keeps every key > tau and the lowest-index keys == tau, and a
// block-wide scan writes them in increasing index order.  Histograms use
// integer LDS atomics, so the result does not depend on thread timing.  Rows
// of up to kCache entries are read from memory once and kept in LDS.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

constexpr int kTopkThreads = 1024;
constexpr int kCache = 32768;
constexpr int kBins = 2048;  // 11-bit digits: 2 bins per thread in the bucket scan

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0) u = 0;  // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan over the workgroup; `sh` holds at least 17 words.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* sh, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  uint32_t inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) sh[w] = inc;
  __syncthreads();
  if (w == 0) {
    const uint32_t t = lane < nw ? sh[lane] : 0u;
    uint32_t ti = t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(ti, o);
      if (lane >= o) ti += y;
    }
    if (lane < nw) sh[lane] = ti - t;
    if (lane == nw - 1) sh[16] = ti;
  }
  __syncthreads();
  const uint32_t r = sh[w] + inc - x;
  *total = sh[16];
  __syncthreads();
  return r;
}

// Keys of elements [base, base + kTopkThreads * 32) are handled 32 per thread:
// element base + 4 * (tid + kTopkThreads * j) + e, j < 8, e < 4 (coalesced float4 loads).
constexpr int kPerThread = 32;
constexpr int kRound = kTopkThreads * kPerThread;

__global__ void __launch_bounds__(kTopkThreads) topk_kernel(const float* __restrict__ scores, int P_max,
                                                           const int32_t* __restrict__ prefix_len,
                                                           const int32_t* __restrict__ kreq, int k_max,
                                                           int32_t* __restrict__ idx, int32_t* __restrict__ count) {
  // key i lives at cache[i + i / 32]: a thread reading its 32 consecutive keys
  // and the 64 lanes of a wave then hit 64 different banks
  __shared__ uint32_t cache[kCache + kCache / 32];
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t sh[24];
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
  const bool cached = P <= kCache;
  const bool vec = ((reinterpret_cast<uintptr_t>(s) & 15) == 0);

  // 32 keys per thread per round: element base + 4 * (tid + kTopkThreads * j) + e (coalesced)
  auto elem = [&](int base, int j, int e) { return base + 4 * (tid + kTopkThreads * j) + e; };
  auto load_round = [&](int base, uint32_t (&u)[kPerThread]) {
#pragma unroll
    for (int j = 0; j < kPerThread / 4; ++j) {
      const int i0 = elem(base, j, 0);
      if (vec && i0 + 4 <= P) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(s + i0);
#pragma unroll
        for (int e = 0; e < 4; ++e) u[4 * j + e] = order_key(x[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) u[4 * j + e] = (i0 + e < P) ? order_key(s[i0 + e]) : 0u;
      }
    }
  };

  // ---- pass 0: load (and cache) the keys, find their range
  if (tid == 0) {
    sh[20] = 0xffffffffu;
    sh[21] = 0u;
  }
  __syncthreads();
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int base = 0; base < P; base += kRound) {
    uint32_t u[kPerThread];
    load_round(base, u);
#pragma unroll
    for (int j = 0; j < kPerThread / 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = elem(base, j, e);
        if (i < P) {
          if (cached) cache[i + (i >> 5)] = u[4 * j + e];
          kmin = min(kmin, u[4 * j + e]);
          kmax = max(kmax, u[4 * j + e]);
        }
      }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
  }
  if ((tid & 63) == 0) {
    atomicMin(&sh[20], kmin);
    atomicMax(&sh[21], kmax);
  }
  __syncthreads();
  kmin = sh[20];
  kmax = sh[21];
  const uint32_t range = kmax - kmin;
  const int nbits = range == 0 ? 0 : 32 - __builtin_clz(range);

  // ---- radix passes over x = key - kmin, 11 bits at a time from bit nbits down
  uint32_t prefix = 0, pmask = 0, krem = (uint32_t)k;  // x & pmask == prefix selects the live bucket
  for (int hi = nbits; hi > 0;) {
    const int lo = hi > 11 ? hi - 11 : 0;
    const uint32_t dmask = (1u << (hi - lo)) - 1u;
    for (int i = tid; i < kBins; i += kTopkThreads) hist[i] = 0;
    if (tid == 0) {
      sh[18] = prefix;
      sh[19] = krem;
    }
    __syncthreads();
    for (int base = 0; base < P; base += kRound) {
      uint32_t u[kPerThread];
      if (cached) {
        const int i0 = base + tid * kPerThread;
#pragma unroll
        for (int e = 0; e < kPerThread; ++e) {
          const int i = i0 + e;
          const uint32_t x = (i < P ? cache[i + (i >> 5)] : kmin) - kmin;
          if (i < P && (x & pmask) == prefix) atomicAdd(&hist[(x >> lo) & dmask], 1u);
        }
      } else {
        load_round(base, u);
#pragma unroll
        for (int j = 0; j < kPerThread / 4; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t x = u[4 * j + e] - kmin;
            if (elem(base, j, e) < P && (x & pmask) == prefix) atomicAdd(&hist[(x >> lo) & dmask], 1u);
          }
      }
    }
    __syncthreads();
    {
      // suffix scan over the bins: thread t holds bins kBins-1-2t and kBins-2-2t
      const uint32_t c0 = hist[kBins - 1 - 2 * tid], c1 = hist[kBins - 2 - 2 * tid];
      uint32_t tot;
      const uint32_t exc = block_excl_scan(c0 + c1, sh, &tot);
      if (exc < krem && krem <= exc + c0 + c1) {
        const bool first = exc + c0 >= krem;
        const uint32_t bucket = first ? (uint32_t)(kBins - 1 - 2 * tid) : (uint32_t)(kBins - 2 - 2 * tid);
        const uint32_t above = first ? exc : exc + c0;
        sh[18] = prefix | (bucket << lo);
        sh[19] = krem - above;
      }
    }
    __syncthreads();
    prefix = sh[18];
    krem = sh[19];
    pmask |= dmask << lo;
    __syncthreads();
    hi = lo;
  }
  const uint32_t tau = prefix + kmin;  // key of the k-th largest score
  const uint32_t need_eq = krem;       // entries equal to tau to keep, lowest index first

  // ---- emit in increasing index order: thread t owns indices [base + 32 t, base + 32 t + 32)
  uint32_t eq_carry = 0, sel_carry = 0;
  for (int base = 0; base < P; base += kRound) {
    const int i0 = base + tid * kPerThread;
    uint32_t u[kPerThread];
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int i = i0 + e;
      u[e] = i < P ? (cached ? cache[i + (i >> 5)] : order_key(s[i])) : 0u;
    }
    uint32_t n_eq = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) n_eq += (i0 + e < P && u[e] == tau) ? 1u : 0u;
    uint32_t tot;
    uint32_t eq_before = eq_carry + block_excl_scan(n_eq, sh, &tot);
    eq_carry += tot;
    uint32_t selmask = 0, n_sel = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      bool sel = false;
      if (i0 + e < P) {
        if (u[e] > tau) {
          sel = true;
        } else if (u[e] == tau) {
          sel = eq_before < need_eq;
          ++eq_before;
        }
      }
      if (sel) {
        selmask |= 1u << e;
        ++n_sel;
      }
    }
    uint32_t pos = sel_carry + block_excl_scan(n_sel, sh, &tot);
    sel_carry += tot;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e)
      if ((selmask & (1u << e)) && pos < (uint32_t)k) out[pos++] = i0 + e;
  }
  for (int i = k + tid; i < k_max; i += kTopkThreads) out[i] = -1;
}

int launch_topk(const float* scores, int B, int P_max, const int32_t* prefix_len, const int32_t* k,
                int k_max, int32_t* idx, int32_t* count, void* stream) {
  (void)hipGetLastError();
  if (B > 0)
    hipLaunchKernelGGL(topk_kernel, dim3(B), dim3(kTopkThreads), 0, reinterpret_cast<hipStream_t>(stream),
                       scores, P_max, prefix_len, k, k_max, idx, count);
  return (int)hipGetLastError();
}

}  // namespace sv
