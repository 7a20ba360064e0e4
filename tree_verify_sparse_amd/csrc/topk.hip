// Top-k selection of prefix entries by score, one 1024-thread workgroup per
// sequence (Vegas §2 step 2 and §2.A: the k-subset with the largest summed
// score is the set of the k largest scores).
//
// Scores map to order-preserving 32-bit keys (-0.0 folded onto +0.0).  Four
// 8-bit radix passes over the keys find the exact key tau of the k-th largest
// entry and how many entries equal to tau are still needed; a final pass in
// index order keeps every key > tau and the lowest-index keys == tau, and a
// block-wide scan writes the kept indices in increasing order.  Histograms
// use integer LDS atomics, so the result does not depend on thread timing.
// Rows of up to kCache entries are read from memory once and kept in LDS.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

constexpr int kTopkThreads = 1024;
constexpr int kCache = 32768;

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

__global__ void __launch_bounds__(kTopkThreads) topk_kernel(const float* __restrict__ scores, int P_max,
                                                           const int32_t* __restrict__ prefix_len,
                                                           const int32_t* __restrict__ kreq, int k_max,
                                                           int32_t* __restrict__ idx, int32_t* __restrict__ count) {
  __shared__ uint32_t cache[kCache];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh[20];
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

  uint32_t prefix = 0, pmask = 0, krem = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    if (tid == 0) {
      sh[18] = prefix;
      sh[19] = krem;
    }
    __syncthreads();
    for (int i = tid; i < P; i += kTopkThreads) {
      uint32_t u;
      if (cached && shift != 24) {
        u = cache[i];
      } else {
        u = order_key(s[i]);
        if (cached) cache[i] = u;
      }
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane 0 holds the top four bins, lane 63 the bottom four
      uint32_t c[4], loc = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = hist[255 - 4 * tid - e];
        loc += c[e];
      }
      uint32_t inc = loc;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(inc, o);
        if (tid >= o) inc += y;
      }
      const uint32_t exc = inc - loc;
      if (exc < krem && krem <= inc) {
        uint32_t cum = exc;
        int bucket = 0;
        uint32_t above = 0;
        for (int e = 0; e < 4; ++e) {
          if (cum + c[e] >= krem) {
            bucket = 255 - 4 * tid - e;
            above = cum;
            break;
          }
          cum += c[e];
        }
        sh[18] = prefix | ((uint32_t)bucket << shift);
        sh[19] = krem - above;
      }
    }
    __syncthreads();
    prefix = sh[18];
    krem = sh[19];
    pmask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t tau = prefix;  // key of the k-th largest score
  const uint32_t need_eq = krem;  // entries equal to tau to keep, lowest index first

  constexpr int E = 8;
  uint32_t eq_carry = 0, sel_carry = 0;
  for (int base = 0; base < P; base += kTopkThreads * E) {
    const int i0 = base + tid * E;
    uint32_t u[E];
    uint32_t n_eq = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = i0 + e;
      u[e] = (i < P) ? (cached ? cache[i] : order_key(s[i])) : 0u;
      n_eq += (i < P && u[e] == tau) ? 1u : 0u;
    }
    uint32_t tot;
    uint32_t eq_before = eq_carry + block_excl_scan(n_eq, sh, &tot);
    eq_carry += tot;
    uint32_t selmask = 0, n_sel = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = i0 + e;
      bool sel = false;
      if (i < P) {
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
    for (int e = 0; e < E; ++e)
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
