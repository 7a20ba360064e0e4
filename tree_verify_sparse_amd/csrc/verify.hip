// Verification attention with fused criticality scores, for gfx950.
//
// What is computed (Vegas §2 step 1, §2.A, §3; JETFLOW §2 tree mask): for
// every sequence b, verify node t and query head h (KV head g = h / G),
//   o[b][t][h] = softmax_j(scale * q . k_j) v_j   over j in prefix U {P_b + a : a ancestor-or-self of t}
//   s[b][i]    = sum_{t in score rows} sum_h scale * q[b][t][h] . k[b][i][g(h)],   i < P_b.
//
// Work split: the KV range [0, P_b + N) of each (sequence, KV head) is cut
// into chunks; one 256-thread workgroup (4 waves) owns one chunk, one KV head
// and a block of query rows (row = node * G + head-in-group, so one KV head's
// G query heads share every K/V tile).  K/V tiles of TK keys are staged
// through LDS with a one-tile register prefetch; waves split the tile's 32-key
// blocks and/or the row tiles.  Per 32-key block a wave runs
//   S^T = K Q^T     (MFMA; the C layout puts one query row per lane column),
//   online softmax  (fp32, log2 domain),
//   O^T += V^T P^T  (MFMA; P^T is S^T's accumulator converted in place, V^T
//                    comes straight from the row-major tile via transpose reads).
// The score needs sum over rows and heads of the logits, which is linear in
// q: s_i = scale * k_i . qbar_g with qbar_g the fp32 sum of the scoring rows'
// queries of KV head g.  It is computed in the same K pass as extra MFMA
// columns of S^T holding qbar split into three bf16 parts (hi + mid + lo
// carries qbar to fp32 precision; bf16 x bf16 products are exact in fp32), so
// only one fp32 per prefix key and KV head leaves the kernel.
// Partial (m, l, o) per chunk are merged with log-sum-exp weights by a second
// kernel, which also sums the per-KV-head score partials in a fixed order.
#include "sv_device.h"
#include "sv_internal.h"

#include <algorithm>
#include <type_traits>

namespace sv {

template <typename T, int D>
struct Tile {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int TK = (!kBf16 && D == 128) ? 64 : 128;  // keys per LDS tile
  static constexpr int NB = TK / 32;                         // 32-key blocks per tile
  // LDS row strides (elements), chosen so the MFMA operand reads hit distinct banks.
  static constexpr int KSTR = kBf16 ? (D == 128 ? 136 : 72) : (D == 128 ? 132 : 68);
  static constexpr int VSTR = kBf16 ? (D == 128 ? 160 : 96) : (D == 128 ? 136 : 72);
  static constexpr int ROWB = D * (int)sizeof(T);  // bytes of one head's K (or V) row
  static constexpr int CPR = ROWB / 16;            // 16-byte chunks per row
  static constexpr int LOADS = TK * CPR / 256;     // 16-byte loads per thread per tensor
  static constexpr int KS_BYTES = TK * KSTR * (int)sizeof(T);
  static constexpr int VS_BYTES = TK * VSTR * (int)sizeof(T);
  static constexpr int EPI_BYTES = 4 * 32 * (D + 1) * 4 + 4 * 32 * 2 * 4;
  static constexpr int LDS_BYTES = (KS_BYTES + VS_BYTES) > EPI_BYTES ? (KS_BYTES + VS_BYTES) : EPI_BYTES;
};

struct VerifyArgs {
  const void* q;
  void* out;
  KvView kv;
  const int32_t* prefix_len;
  float* ws_o;
  f32x2* ws_ml;
  float* ws_s;
  float* ws_qbar;
  uint32_t* ws_anc;
  const int32_t* parent;
  float* scores;
  int B, N, Hq, Hkv, G, R, RB, Rpad, P_max, chunk, n_chunks, n_units;
  int tree, do_scores, prep_qbar;
  float scale, scale_log2;
  int n_score_rows;
  uint16_t score_rows[kMaxNodes];
};

// key offset (within a 32-key block) of accumulator element v for lane half h
__device__ __forceinline__ int kappa(int v, int h) { return mfma_row(v, h); }

template <typename T, int D, int RT, int WR>
__global__ void __launch_bounds__(256) verify_main(const VerifyArgs a) {
  using TL = Tile<T, D>;
  constexpr int WK = 4 / WR;
  constexpr bool kBf16 = TL::kBf16;
  constexpr int DB = D / 32;  // 32-wide column blocks of the head dim
  __shared__ __attribute__((aligned(16))) char smem[TL::LDS_BYTES];
  T* Ks = reinterpret_cast<T*>(smem);
  T* Vs = reinterpret_cast<T*>(smem + TL::KS_BYTES);

  // ---- workgroup -> (sequence, KV head, chunk, row block); consecutive logical
  // ids (same head, neighbouring chunks, all row blocks) land on one XCD.
  const int per = gridDim.x >> 3;
  const int lid = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (lid >= a.n_units) return;
  const int rb = lid % a.RB;
  int rest = lid / a.RB;
  const int c = rest % a.n_chunks;
  rest /= a.n_chunks;
  const int g = rest % a.Hkv;
  const int b = rest / a.Hkv;

  int Pb = a.prefix_len[b];
  Pb = Pb < 0 ? 0 : (Pb > a.P_max ? a.P_max : Pb);
  const int L = Pb + a.N;
  const int c0 = c * a.chunk;
  if (c0 >= L) return;
  const int c1 = min(c0 + a.chunk, L);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lane32 = lane & 31, h = lane >> 5;
  const int wk = wave % WK, wr = wave / WK;

  // ---- query fragments (B operand of S^T = K Q^T): lane column = query row
  typedef typename std::conditional<kBf16, bf16x8, float>::type QElem;
  constexpr int QN = kBf16 ? D / 16 : D / 2;
  QElem qf[RT][QN];
  int row_node[RT];
  bool row_ok[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = ((rb * WR + wr) * RT + rt) * 32 + lane32;
    row_ok[rt] = r < a.R;
    const int t = row_ok[rt] ? r / a.G : a.N - 1;
    row_node[rt] = t;
    const int j = row_ok[rt] ? r % a.G : 0;
    const T* qrow = reinterpret_cast<const T*>(a.q) + ((long long)(b * a.N + t) * a.Hq + g * a.G + j) * D;
    if constexpr (kBf16) {
#pragma unroll
      for (int ks = 0; ks < QN; ++ks) {
        bf16x8 x = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks + 8 * h);
        qf[rt][ks] = row_ok[rt] ? x : bf16x8{};
      }
    } else {
#pragma unroll
      for (int cc = 0; cc < D / 8; ++cc) {
        f32x4 x = *reinterpret_cast<const f32x4*>(qrow + 8 * cc + 4 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e) qf[rt][4 * cc + e] = row_ok[rt] ? x[e] : 0.f;
      }
    }
  }

  // ---- score operand: qbar_g split into bf16 hi/mid/lo in MFMA columns 0..2
  const bool wg_scores = a.do_scores && rb == 0 && c0 < Pb;
  QElem qb[QN];
  if (wg_scores) {
    float* qs = reinterpret_cast<float*>(smem);
    if (a.prep_qbar) {
      for (int d = tid; d < D; d += 256) qs[d] = a.ws_qbar[(b * a.Hkv + g) * D + d];
    } else {
      constexpr int NP = 256 / D;
      const int d = tid % D, part = tid / D;
      const int npairs = a.n_score_rows * a.G;
      float acc = 0.f;
      for (int i = part; i < npairs; i += NP) {
        const int t = a.score_rows[i / a.G], j = i % a.G;
        const T* qrow = reinterpret_cast<const T*>(a.q) + ((long long)(b * a.N + t) * a.Hq + g * a.G + j) * D;
        acc += (float)qrow[d];
      }
      qs[D + part * D + d] = acc;
      __syncthreads();
      if (tid < D) {
        float s = 0.f;
        for (int p = 0; p < NP; ++p) s += qs[D + p * D + tid];
        qs[tid] = s;
      }
    }
    __syncthreads();
    if constexpr (kBf16) {
#pragma unroll
      for (int ks = 0; ks < QN; ++ks) {
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = qs[16 * ks + 8 * h + e];
          const bf16 hi = (bf16)x;
          const float r1 = x - (float)hi;
          const bf16 mid = (bf16)r1;
          const float r2 = r1 - (float)mid;
          const bf16 lo = (bf16)r2;
          v[e] = lane32 == 0 ? hi : (lane32 == 1 ? mid : (lane32 == 2 ? lo : (bf16)0.f));
        }
        qb[ks] = v;
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < QN; ++kk) {
        const int d = 8 * (kk >> 2) + 4 * h + (kk & 3);
        qb[kk] = lane32 == 0 ? qs[d] : 0.f;
      }
    }
    __syncthreads();
  }

  // ---- ancestor bitsets of this lane's rows (tree, chunk reaching the verify tokens)
  uint32_t anc[RT][kAncWords];
  const bool has_tail = c1 > Pb;
  if (a.tree && has_tail) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int w = 0; w < kAncWords; ++w) anc[rt][w] = a.ws_anc[((long long)b * a.N + row_node[rt]) * kAncWords + w];
  }

  // ---- running softmax state
  f32x16 o[RT][DB];
  float m[RT], l[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = kNegInf;
    l[rt] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[rt][db] = f32x16{};
  }

  // ---- tile pipeline: registers hold tile it+1 while LDS holds tile it
  const char* kbase = reinterpret_cast<const char*>(a.kv.k) + (long long)g * TL::ROWB;
  const char* vbase = reinterpret_cast<const char*>(a.kv.v) + (long long)g * TL::ROWB;
  const long long slot_bytes = (long long)a.Hkv * TL::ROWB;
  uint4 kr[TL::LOADS], vr[TL::LOADS];
  auto load_tile = [&](int ts) {
#pragma unroll
    for (int i = 0; i < TL::LOADS; ++i) {
      const int ci = tid + 256 * i, key = ci / TL::CPR, col = ci % TL::CPR;
      const int pos = ts + key;
      long long s = pos < c1 ? a.kv.slot(b, pos) : -1;
      if (s >= 0) {
        kr[i] = *reinterpret_cast<const uint4*>(kbase + s * slot_bytes + col * 16);
        vr[i] = *reinterpret_cast<const uint4*>(vbase + s * slot_bytes + col * 16);
      } else {
        kr[i] = make_uint4(0, 0, 0, 0);
        vr[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < TL::LOADS; ++i) {
      const int ci = tid + 256 * i, key = ci / TL::CPR, col = ci % TL::CPR;
      *reinterpret_cast<uint4*>(smem + key * TL::KSTR * (int)sizeof(T) + col * 16) = kr[i];
      *reinterpret_cast<uint4*>(smem + TL::KS_BYTES + key * TL::VSTR * (int)sizeof(T) + col * 16) = vr[i];
    }
  };

  const int n_tiles = (c1 - c0 + TL::TK - 1) / TL::TK;
  load_tile(c0);
  for (int it = 0; it < n_tiles; ++it) {
    const int ts = c0 + it * TL::TK;
    __syncthreads();
    store_tile();
    __syncthreads();
    if (it + 1 < n_tiles) load_tile(ts + TL::TK);

    for (int kb = wk; kb < TL::NB; kb += WK) {
      const int kb0 = ts + 32 * kb;
      if (kb0 >= c1) break;
      const bool do_score = wg_scores && kb0 < Pb && ((kb / WK) % WR) == wr;
      f32x16 s[RT];
      f32x16 sc = f32x16{};
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) s[rt] = f32x16{};

      // S^T = K Q^T (and the score columns)
      const T* krow = Ks + (32 * kb + lane32) * TL::KSTR;
      if constexpr (kBf16) {
#pragma unroll
        for (int ks = 0; ks < QN; ++ks) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(krow + 16 * ks + 8 * h);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) s[rt] = mfma_bf16(ka, qf[rt][ks], s[rt]);
          if (do_score) sc = mfma_bf16(ka, qb[ks], sc);
        }
      } else {
#pragma unroll
        for (int cc = 0; cc < D / 8; ++cc) {
          const f32x4 ka = *reinterpret_cast<const f32x4*>(krow + 8 * cc + 4 * h);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) s[rt] = mfma_f32(ka[e], qf[rt][4 * cc + e], s[rt]);
            if (do_score) sc = mfma_f32(ka[e], qb[4 * cc + e], sc);
          }
        }
      }

      if (do_score) {
        // column sum hi + mid + lo (lanes 0..2 / 32..34), written by lanes 0 and 32
        float tv[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float x = sc[v];
          if constexpr (kBf16) x = x + __shfl_down(sc[v], 1) + __shfl_down(sc[v], 2);
          tv[v] = x * a.scale;
        }
        if (lane32 == 0) {
          const int lim = min(Pb, c1);
          float* dst = a.ws_s + ((long long)b * a.Hkv + g) * a.P_max;
#pragma unroll
          for (int qd = 0; qd < 4; ++qd) {
            const int k0 = kb0 + 8 * qd + 4 * h;
            if (k0 + 4 <= lim) {
              *reinterpret_cast<f32x4*>(dst + k0) = f32x4{tv[4 * qd], tv[4 * qd + 1], tv[4 * qd + 2], tv[4 * qd + 3]};
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (k0 + e < lim) dst[k0 + e] = tv[4 * qd + e];
            }
          }
        }
      }

      // mask: keys past the chunk end, and verify tokens that are not ancestors-or-self
      if (kb0 + 32 > min(Pb, c1)) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int t = row_node[rt];
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = kb0 + kappa(v, h);
            bool vis = key < c1;
            if (vis && key >= Pb) {
              const int an = key - Pb;
              if (a.tree) {
                uint32_t word = 0;
#pragma unroll
                for (int w = 0; w < kAncWords; ++w) word = ((an >> 5) == w) ? anc[rt][w] : word;
                vis = (word >> (an & 31)) & 1u;
              } else {
                vis = an <= t;
              }
            }
            if (!vis) s[rt][v] = kNegInf;
          }
        }
      }

      // online softmax (log2 domain)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float mx = kNegInf;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          s[rt][v] *= a.scale_log2;
          mx = fmaxf(mx, s[rt][v]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(m[rt], mx);
        const bool live = mn != kNegInf;
        const float alpha = live ? fast_exp2(m[rt] - mn) : 1.f;
        float ps = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = live ? fast_exp2(s[rt][v] - mn) : 0.f;
          s[rt][v] = p;
          ps += p;
        }
        l[rt] = l[rt] * alpha + ps;
        m[rt] = mn;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[rt][db] *= alpha;
      }

      // O^T += V^T P^T
      if constexpr (kBf16) {
        const int e = (lane & 15) >> 2, cq = lane & 3, dh = (lane >> 4) & 1;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          bf16x8 pb[RT];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int u = 0; u < 8; ++u) pb[rt][u] = (bf16)s[rt][8 * jj + u];
          const T* v0 = Vs + (32 * kb + 16 * jj + 4 * h + e) * TL::VSTR + 16 * dh + 4 * cq;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x4 lo = lds_read_tr16(v0 + 32 * db);
            const bf16x4 hi = lds_read_tr16(v0 + 8 * TL::VSTR + 32 * db);
            const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) o[rt][db] = mfma_bf16(va, pb[rt], o[rt][db]);
          }
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const T* vrow = Vs + (32 * kb + kappa(v, h)) * TL::VSTR + lane32;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const float va = vrow[32 * db];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) o[rt][db] = mfma_f32(va, s[rt][v], o[rt][db]);
          }
        }
      }
    }
  }

  // ---- epilogue: combine the WK waves that share rows, write (m, l, o) partials
  constexpr int OS = D + 1;
  float* lo_ = reinterpret_cast<float*>(smem);            // [4 waves][32 rows][D+1]
  float* lml = lo_ + 4 * 32 * OS;                          // [4 waves][32 rows][2]
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float lt = l[rt] + __shfl_xor(l[rt], 32);
    __syncthreads();
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) lo_[(wave * 32 + lane32) * OS + 32 * db + kappa(v, h)] = o[rt][db][v];
    if (h == 0) {
      lml[(wave * 32 + lane32) * 2 + 0] = m[rt];
      lml[(wave * 32 + lane32) * 2 + 1] = lt;
    }
    __syncthreads();
    for (int idx = tid; idx < WR * 32 * D; idx += 256) {
      const int d = idx % D, r = (idx / D) % 32, wq = idx / (32 * D);
      const int row = ((rb * WR + wq) * RT + rt) * 32 + r;
      if (row >= a.R) continue;
      float M = kNegInf;
#pragma unroll
      for (int k2 = 0; k2 < WK; ++k2) M = fmaxf(M, lml[((wq * WK + k2) * 32 + r) * 2]);
      float acc = 0.f, lsum = 0.f;
#pragma unroll
      for (int k2 = 0; k2 < WK; ++k2) {
        const int w = wq * WK + k2;
        const float mw = lml[(w * 32 + r) * 2];
        const float wt = (M == kNegInf) ? 0.f : fast_exp2(mw - M);
        acc += wt * lo_[(w * 32 + r) * OS + d];
        lsum += wt * lml[(w * 32 + r) * 2 + 1];
      }
      const long long rec = ((long long)(b * a.Hkv + g) * a.Rpad + row) * a.n_chunks + c;
      a.ws_o[rec * D + d] = acc;
      if (d == 0) a.ws_ml[rec] = f32x2{M, lsum};
    }
  }
}

// Split-KV merge (log-sum-exp weights) + per-KV-head score sum.
template <typename T, int D>
__global__ void __launch_bounds__(256) verify_merge(const VerifyArgs a, int n_row_wgs) {
  const int tid = threadIdx.x;
  if ((int)blockIdx.x < n_row_wgs) {
    const int wave = tid >> 6, lane = tid & 63;
    const int gr = blockIdx.x * 4 + wave;  // (b, g, row)
    if (gr >= a.B * a.Hkv * a.R) return;
    const int row = gr % a.R, bg = gr / a.R, g = bg % a.Hkv, b = bg / a.Hkv;
    int Pb = a.prefix_len[b];
    Pb = Pb < 0 ? 0 : (Pb > a.P_max ? a.P_max : Pb);
    const int nc = min((Pb + a.N + a.chunk - 1) / a.chunk, a.n_chunks);
    const long long rec0 = ((long long)(b * a.Hkv + g) * a.Rpad + row) * a.n_chunks;
    float M = kNegInf;
    for (int c = 0; c < nc; ++c) M = fmaxf(M, a.ws_ml[rec0 + c][0]);
    constexpr int PER = D / 64;
    float acc[PER] = {};
    float lsum = 0.f;
    for (int c = 0; c < nc; ++c) {
      const f32x2 ml = a.ws_ml[rec0 + c];
      const float wt = (M == kNegInf) ? 0.f : fast_exp2(ml[0] - M);
      lsum += wt * ml[1];
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += wt * a.ws_o[(rec0 + c) * D + lane * PER + e];
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const int t = row / a.G, j = row % a.G;
    T* dst = reinterpret_cast<T*>(a.out) + ((long long)(b * a.N + t) * a.Hq + g * a.G + j) * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) dst[e] = (T)(acc[e] * inv);
  } else {
    const long long i0 = (long long)(blockIdx.x - n_row_wgs) * 256 + tid;
    if (i0 >= (long long)a.B * a.P_max) return;
    const int b = (int)(i0 / a.P_max), i = (int)(i0 % a.P_max);
    int Pb = a.prefix_len[b];
    Pb = Pb < 0 ? 0 : (Pb > a.P_max ? a.P_max : Pb);
    if (i >= Pb) return;
    float s = 0.f;
    for (int g = 0; g < a.Hkv; ++g) s += a.ws_s[((long long)b * a.Hkv + g) * a.P_max + i];
    a.scores[i0] = s;
  }
}

// Per-sequence precomputation: qbar_g (fp32 sum of the scoring rows' queries of
// each KV head) and ancestor-or-self bitsets of the draft tree by pointer jumping.
template <typename T, int D>
__global__ void __launch_bounds__(256) verify_prep(const VerifyArgs a, int n_qbar_wgs) {
  const int tid = threadIdx.x;
  __shared__ float part[256];
  __shared__ uint32_t ancs[2][kMaxNodes][kAncWords];
  __shared__ int jmp[2][kMaxNodes];
  if ((int)blockIdx.x < n_qbar_wgs) {
    const int g = blockIdx.x % a.Hkv, b = blockIdx.x / a.Hkv;
    constexpr int NP = 256 / D;
    const int d = tid % D, p = tid / D;
    const int npairs = a.n_score_rows * a.G;
    float acc = 0.f;
    for (int i = p; i < npairs; i += NP) {
      const int t = a.score_rows[i / a.G], j = i % a.G;
      acc += (float)reinterpret_cast<const T*>(a.q)[((long long)(b * a.N + t) * a.Hq + g * a.G + j) * D + d];
    }
    part[tid] = acc;
    __syncthreads();
    if (tid < D) {
      float s = 0.f;
      for (int k = 0; k < NP; ++k) s += part[k * D + tid];
      a.ws_qbar[(b * a.Hkv + g) * D + tid] = s;
    }
    return;
  }
  const int b = blockIdx.x - n_qbar_wgs;
  const int N = a.N;
  for (int t = tid; t < N; t += 256) {
    int p = a.parent[(long long)b * N + t];
    if (p < 0 || p >= t) p = -1;  // malformed parents are treated as roots
    jmp[0][t] = p;
#pragma unroll
    for (int w = 0; w < kAncWords; ++w) {
      uint32_t x = (w == (t >> 5)) ? (1u << (t & 31)) : 0u;
      if (p >= 0 && w == (p >> 5)) x |= 1u << (p & 31);
      ancs[0][t][w] = x;
    }
  }
  __syncthreads();
  int cur = 0;
  for (int round = 0; round < 9; ++round) {
    int any = 0;
    for (int e = tid; e < N * kAncWords; e += 256) {
      const int t = e / kAncWords, w = e % kAncWords;
      const int j = jmp[cur][t];
      ancs[cur ^ 1][t][w] = ancs[cur][t][w] | (j >= 0 ? ancs[cur][j][w] : 0u);
      if (w == 0) {
        const int jj = j >= 0 ? jmp[cur][j] : -1;
        jmp[cur ^ 1][t] = jj;
        any |= jj >= 0;
      }
    }
    cur ^= 1;
    if (!__syncthreads_or(any)) break;
  }
  for (int e = tid; e < N * kAncWords; e += 256)
    a.ws_anc[(long long)b * N * kAncWords + e] = ancs[cur][e / kAncWords][e % kAncWords];
}

// ------------------------------------------------------------------------- host side

VerifyPlan plan_verify(int B, int N, int Hq, int Hkv, int D, int P_max, int dtype, bool tree,
                       int n_score_rows) {
  VerifyPlan p{};
  p.B = B; p.N = N; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv; p.D = D; p.P_max = P_max; p.dtype = dtype;
  p.R = N * p.G;
  const int rtiles = (p.R + 31) / 32;
  if (rtiles <= 1) { p.RT = 1; p.WR = 1; }
  else if (rtiles <= 2) { p.RT = 2; p.WR = 1; }
  else if (rtiles <= 4) { p.RT = 2; p.WR = 2; }
  else { p.RT = 2; p.WR = 4; }
  p.WK = 4 / p.WR;
  p.rows_per_block = p.RT * p.WR * 32;
  p.RB = (p.R + p.rows_per_block - 1) / p.rows_per_block;
  p.Rpad = p.RB * p.rows_per_block;
  p.TK = (dtype == SV_F32 && D == 128) ? 64 : 128;
  const long long Lmax = (long long)P_max + N;
  const long long units = (long long)B * Hkv * p.RB;
  const long long target = 512;  // about two resident workgroups per CU
  long long want = (target + units - 1) / units;
  if (want < 1) want = 1;
  long long chunk = (Lmax + want - 1) / want;
  chunk = (chunk + 31) / 32 * 32;
  if (chunk < 32) chunk = 32;
  p.chunk = (int)chunk;
  p.n_chunks = (int)((Lmax + chunk - 1) / chunk);
  long long n_units = units * p.n_chunks;
  p.n_wg = (int)((n_units + 7) / 8 * 8);
  p.tree = tree;
  p.scores = n_score_rows > 0;
  p.prep_qbar = p.scores && (long long)n_score_rows * p.G > kInlineQbarRows;
  p.prep = p.prep_qbar || tree;
  size_t off = 0;
  p.off_o = off; off = align_up(off + (size_t)B * Hkv * p.Rpad * p.n_chunks * D * 4);
  p.off_ml = off; off = align_up(off + (size_t)B * Hkv * p.Rpad * p.n_chunks * 8);
  p.off_s = off; off = align_up(off + (p.scores ? (size_t)B * Hkv * P_max * 4 : 0));
  p.off_qbar = off; off = align_up(off + (p.prep_qbar ? (size_t)B * Hkv * D * 4 : 0));
  p.off_anc = off; off = align_up(off + (tree ? (size_t)B * N * kAncWords * 4 : 0));
  p.bytes = off;
  return p;
}

template <typename T, int D, int RT, int WR>
static void launch_main(const VerifyPlan& p, const VerifyArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((verify_main<T, D, RT, WR>), dim3(p.n_wg), dim3(256), 0, st, a);
}

template <typename T, int D>
static int launch_typed(const VerifyPlan& p, VerifyArgs& a, hipStream_t st, void* ev0, void* ev1) {
  if (p.prep) {
    const int nq = p.prep_qbar ? p.B * p.Hkv : 0;
    const int nt = p.tree ? p.B : 0;
    hipLaunchKernelGGL((verify_prep<T, D>), dim3(nq + nt), dim3(256), 0, st, a, nq);
  }
  if (ev0) (void)hipEventRecord((hipEvent_t)ev0, st);
  if (p.RT == 1 && p.WR == 1) launch_main<T, D, 1, 1>(p, a, st);
  else if (p.RT == 2 && p.WR == 1) launch_main<T, D, 2, 1>(p, a, st);
  else if (p.RT == 2 && p.WR == 2) launch_main<T, D, 2, 2>(p, a, st);
  else launch_main<T, D, 2, 4>(p, a, st);
  if (ev1) (void)hipEventRecord((hipEvent_t)ev1, st);
  const int n_row_wgs = (p.B * p.Hkv * p.R + 3) / 4;
  const long long n_s = p.scores ? ((long long)p.B * p.P_max + 255) / 256 : 0;
  hipLaunchKernelGGL((verify_merge<T, D>), dim3(n_row_wgs + (int)n_s), dim3(256), 0, st, a, n_row_wgs);
  return (int)hipGetLastError();
}

int launch_verify(const VerifyPlan& p, const void* q, const KvArgs& kv, const int32_t* prefix_len,
                  const int32_t* parent, const int32_t* score_rows, int n_score_rows, float scale,
                  void* out, float* scores, void* ws, void* stream, void* ev_start, void* ev_stop) {
  VerifyArgs a{};
  a.q = q;
  a.out = out;
  a.kv = KvView{kv.k, kv.v, kv.page_table, kv.page_size, kv.max_pages, kv.seq_stride, kv.num_slots};
  a.prefix_len = prefix_len;
  char* w = reinterpret_cast<char*>(ws);
  a.ws_o = reinterpret_cast<float*>(w + p.off_o);
  a.ws_ml = reinterpret_cast<f32x2*>(w + p.off_ml);
  a.ws_s = reinterpret_cast<float*>(w + p.off_s);
  a.ws_qbar = reinterpret_cast<float*>(w + p.off_qbar);
  a.ws_anc = reinterpret_cast<uint32_t*>(w + p.off_anc);
  a.parent = parent;
  a.scores = scores;
  a.B = p.B; a.N = p.N; a.Hq = p.Hq; a.Hkv = p.Hkv; a.G = p.G; a.R = p.R; a.RB = p.RB; a.Rpad = p.Rpad;
  a.P_max = p.P_max; a.chunk = p.chunk; a.n_chunks = p.n_chunks;
  a.n_units = p.B * p.Hkv * p.RB * p.n_chunks;
  a.tree = p.tree; a.do_scores = p.scores; a.prep_qbar = p.prep_qbar;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  a.n_score_rows = n_score_rows;
  for (int i = 0; i < n_score_rows && i < kMaxNodes; ++i) a.score_rows[i] = (uint16_t)score_rows[i];
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (p.dtype == SV_BF16) {
    if (p.D == 128) return launch_typed<bf16, 128>(p, a, st, ev_start, ev_stop);
    return launch_typed<bf16, 64>(p, a, st, ev_start, ev_stop);
  }
  if (p.D == 128) return launch_typed<float, 128>(p, a, st, ev_start, ev_stop);
  return launch_typed<float, 64>(p, a, st, ev_start, ev_stop);
}

}  // namespace sv
