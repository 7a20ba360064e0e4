// Top-k selection of prefix entries by score (Vegas §2 step 2 and §2.A: the
// k-subset with the largest summed score is the set of the k largest scores;
// ties go to the lower index), as two kernels over rows held in memory:
//   sel_pass_a  one workgroup per block of a row: the row's band from a
//               sample, the block's entries at or above it into fixed slots;
//   sel_pass_b  one workgroup per row: the cut inside the band and the kept
//               indices in increasing order (or the exact radix path).
// The passes themselves are in select_dev.h, shared with the verify merge
// kernel, which runs them on the scores it has just summed.
#include "select_dev.h"
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

// Pass A of block blk of a row read from memory: thread t holds the E
// entries blk * E * 256 + E t + e.
template <int E>
__device__ __forceinline__ void sel_pass_a_block(SelShared& L, const float* __restrict__ s, int P, int k, int b,
                                                 int blk, const SelWs& ws) {
  const int tid = threadIdx.x;
  const bool vec = (reinterpret_cast<uintptr_t>(s) & 15) == 0;
  auto load4 = [&](int i, float* x) {  // entries i .. i + 3 (NaN past the row end)
    if (vec && i + 4 <= P) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(s + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = v[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = i + e < P ? s[i + e] : __builtin_nanf("");
    }
  };
  // the sample first (it is needed first): segment t of 256, sel_seg(P) entries
  constexpr int SEGMAX = 16;
  const int seg = sel_seg(P);
  float smp[SEGMAX];
  const int p0 = sel_seg_start(tid, P, seg, kSelThreads);
#pragma unroll
  for (int q = 0; q < SEGMAX / 4; ++q) {
    if (4 * q < seg) {
      load4(p0 + 4 * q, smp + 4 * q);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) smp[4 * q + e] = __builtin_nanf("");
    }
  }
  const int base = blk * E * kSelThreads;
  float x[E];
#pragma unroll
  for (int q = 0; q < E / 4; ++q) load4(base + E * tid + 4 * q, x + 4 * q);
  float t_lo, t_hi;
  sel_band<kSelThreads>(L, smp, kSelThreads * seg, P, k, &t_lo, &t_hi);
  if (blk == 0 && tid == 0) ws.band[b] = SelBand{t_lo, t_hi, {0, 0}};
  sel_compact<kSelThreads, E>(L, ws, b, blk, x, base, t_lo, t_hi, [](uint32_t* p, uint32_t v) { *p = v; });
}

// Grid (blocks, rows), 256 threads.
__global__ void __launch_bounds__(kSelThreads) sel_pass_a(const float* __restrict__ scores, int P_max,
                                                          const int32_t* __restrict__ prefix_len,
                                                          const int32_t* __restrict__ kreq, int k_max, SelWs ws) {
  __shared__ SelShared L;
  const int blk = blockIdx.x, b = blockIdx.y;
  int P, k;
  sel_row_sizes(prefix_len, kreq, b, P_max, k_max, &P, &k);
  if (!sel_multi(P, k) || blk * sel_blk(P, k) >= P) return;
  const float* s = scores + (long long)b * P_max;
  if (sel_blk(P, k) == 4096) sel_pass_a_block<16>(L, s, P, k, b, blk, ws);
  else if (sel_blk(P, k) == 2048) sel_pass_a_block<8>(L, s, P, k, b, blk, ws);
  else sel_pass_a_block<4>(L, s, P, k, b, blk, ws);
}

// Grid (rows), 1024 threads.
__global__ void __launch_bounds__(kSelThreadsB) sel_pass_b(const float* __restrict__ scores, int P_max,
                                                          const int32_t* __restrict__ prefix_len,
                                                          const int32_t* __restrict__ kreq, int k_max, SelWs ws,
                                                          int32_t* __restrict__ idx, int32_t* __restrict__ count) {
  __shared__ SelShared L;
  const int b = blockIdx.x;
  int P, k;
  sel_row_sizes(prefix_len, kreq, b, P_max, k_max, &P, &k);
  const float* s = scores + (long long)b * P_max;
  sel_pass_b_row<kSelThreadsB>(L, ws, P, k, k_max, idx + (long long)b * k_max, count, b,
                 [](const uint32_t* p) { return *p; }, [s](int i) { return s[i]; });
}

size_t topk_workspace_bytes(int B, int P_max) {
  (void)P_max;
  return sel_ws_bytes(B);
}

int launch_select_pass_b(const float* scores, int B, int P_max, const int32_t* prefix_len, const int32_t* k,
                         int k_max, int32_t* idx, int32_t* count, const SelWs& w, hipStream_t st);

int launch_topk(const float* scores, int B, int P_max, const int32_t* prefix_len, const int32_t* k,
                int k_max, int32_t* idx, int32_t* count, void* ws, void* stream) {
  (void)hipGetLastError();
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (B <= 0) return 0;
  const SelWs w = sel_ws_at(ws, B);
  if (P_max > kSelMinP) {
    // the most blocks any row up to P_max has: 1024-entry blocks up to 32768
    // entries, 2048 up to 65536, 4096 above (at most kSelMaxBlocks each way)
    int nb = (min(P_max, 32768) + 1023) / 1024;
    if (P_max > 32768) nb = max(nb, (min(P_max, 65536) + 2047) / 2048);
    if (P_max > 65536) nb = max(nb, (min(P_max, kSelMaxP) + 4095) / 4096);
    hipLaunchKernelGGL(sel_pass_a, dim3(min(nb, kSelMaxBlocks), B), dim3(kSelThreads), 0, st, scores, P_max,
                       prefix_len, k, k_max, w);
  }
  return launch_select_pass_b(scores, B, P_max, prefix_len, k, k_max, idx, count, w, st);
}

int launch_select_pass_b(const float* scores, int B, int P_max, const int32_t* prefix_len, const int32_t* k,
                         int k_max, int32_t* idx, int32_t* count, const SelWs& w, hipStream_t st) {
  hipLaunchKernelGGL(sel_pass_b, dim3(B), dim3(kSelThreadsB), 0, st, scores, P_max, prefix_len, k, k_max, w, idx,
                     count);
  return (int)hipGetLastError();
}

bool topk_supported(int P_max) { return P_max >= 0; }

}  // namespace sv
