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
// queries of KV head g.  It is computed in the same K pass, so only one fp32
// per prefix key and KV head leaves the kernel: as extra MFMA columns of S^T
// holding qbar split into three bf16 parts (hi + mid + lo carries qbar to fp32
// precision; bf16 x bf16 products are exact in fp32) in the generic and the
// streaming kernels, and as fp32 dot products on the vector unit, spread over
// all eight waves, in the tree kernel.
// Partial (m, l, o) per chunk are merged with log-sum-exp weights by a second
// kernel, which also sums the per-KV-head score partials in a fixed order.
#include "select_dev.h"
#include "sv_device.h"
#include "sv_internal.h"

#include <hip/hip_ext.h>

#include <algorithm>
#include <type_traits>

namespace sv {

// LDS ring geometry.  K and V rows are stored unpadded; 16-byte chunks of a
// row are permuted by an XOR swizzle so that the MFMA operand reads (16-byte
// K reads, 8-byte transpose reads of V) spread over all LDS banks, while every
// global->LDS copy instruction still reads whole rows (four 256-byte rows per
// 1 KB wave instruction for bf16, D = 128).
template <typename T, int D>
struct Ring {
  static constexpr bool kBf16 = sizeof(T) == 2;
  static constexpr int ROWB = D * (int)sizeof(T);  // bytes of one head's K (or V) row
  static constexpr int CPR = ROWB / 16;            // 16-byte chunks per row
  static constexpr int SK = ROWB > 256 ? 32 : 64;  // keys per stage
  static constexpr int NB = SK / 32;               // 32-key MFMA blocks per stage
  static constexpr int TILE = SK * ROWB;           // bytes of K (or V) per stage
  static constexpr int STAGE = 2 * TILE;
  static constexpr int NS = 4;                     // stages in the ring
  static constexpr int PD = NS - 1;                // stages in flight ahead of compute
  static constexpr int SEGS = STAGE / 1024;        // 1 KB copy instructions per stage
  static constexpr int LPW = SEGS / 4;             // ... per wave
  static constexpr int RPS = 1024 / ROWB;          // rows per copy instruction
  static constexpr int RING = NS * STAGE;
  static constexpr int EPI = 4 * 32 * (D + 1) * 4 + 4 * 32 * 2 * 4;
  static constexpr int MAIN = RING > EPI ? RING : EPI;
  static constexpr int PT_CAP = 1024;              // cached page-table entries per chunk
  static constexpr int AUX_FLOATS = 512;           // qbar scratch
  static constexpr int QBT = 3 * D * (int)sizeof(T);  // score operand table: qbar hi/mid/lo (bf16) or qbar (f32)
  static constexpr int LDS = MAIN + PT_CAP * 4 + AUX_FLOATS * 4 + QBT;
  static_assert(LPW * 4 == SEGS && RPS * ROWB == 1024, "ring geometry");
};

// chunk swizzle of row r (see Ring); the derivation per layout is in the design notes
template <typename T, int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (sizeof(T) == 2 && D == 128) return ((r & 3) << 2) ^ ((r >> 2) & 3);
  else if constexpr (sizeof(T) == 2) return (((r >> 1) & 1) << 2) ^ ((r >> 2) & 3);
  else return (r & 7) ^ (((r >> 2) & 1) << 3);
}
template <typename T, int D>
__device__ __forceinline__ int tile_off(int r, int c) {
  return r * Ring<T, D>::ROWB + ((c ^ swz<T, D>(r)) << 4);
}

struct VerifyArgs {
  const void* q;
  void* out;
  KvView kv;
  float* ws_o;
  f32x2* ws_ml;
  float* ws_s;
  float* ws_qbar;
  uint32_t* ws_anc;
  const int32_t* parent;
  float* scores;
  const int32_t* sel_k;  // device [B] requested k, or null: no selection (see below)
  // bytes 128..191: what a verify kernel reads before its first copies, in one
  // 64-byte line of the argument block (with kv above: two lines in all)
  const int32_t* prefix_len;
  int B, N, Hq, Hkv, G, R, RB, Rpad, P_max, chunk, n_chunks, n_units;
  int len_bias;  // 0 for verification; -1 for a decode over rows [0, prefix_len[b]) (see seq_prefix)
  int tree, do_scores, prep_qbar;
  int qsplit;  // prep_qbar: partial sums per (sequence, KV head), each over kQbarPairs (row, head) pairs
  int s_stride;  // row stride of the per-KV-head score partials: P_max + 32 (whole blocks are stored), rounded up to 4
  int all_chunks;  // every chunk writes a partial (streaming kernel), else only chunks below P_b + N
  int ps_shift;  // log2(page_size) if it is a power of two, else -1
  float scale, scale_log2;
  int n_score_rows;
  int head_scores;  // 1: scores are per KV head, [B][Hkv][P_max] (no sum over the groups)
  // fused selection (sv_verify_select): the merge's score workgroups run the
  // two selection passes on the scores they sum (select_dev.h)
  int sel_kmax;
  int32_t* sel_idx;      // [B][sel_kmax]
  int32_t* sel_count;    // [B] or null
  SelWs selws;
  uint16_t score_rows[kMaxNodes];
};



static_assert(offsetof(VerifyArgs, prefix_len) == 128 && offsetof(VerifyArgs, len_bias) + 4 <= 192,
              "the fields read first share one 64-byte line");
// P_b of sequence b, clamped to [0, P_max], and in *L the length of its KV
// range P_b + N.  A decode over the first n rows of a dense buffer passes n
// with len_bias -1 and N = 1: the query is the last row's token and sees
// [0, n); n = 0 then means no rows at all (L = 0, a zero output).
__device__ __forceinline__ int seq_prefix(const VerifyArgs& a, int b, int* L) {
  int Pb = a.prefix_len[b] + a.len_bias;
  const bool empty = a.len_bias < 0 && Pb < 0;
  Pb = Pb < 0 ? 0 : (Pb > a.P_max ? a.P_max : Pb);
  *L = empty ? 0 : Pb + a.N;
  return Pb;
}

// key offset (within a 32-key block) of accumulator element v for lane half h
__device__ __forceinline__ int kappa(int v, int h) { return mfma_row(v, h); }

// Tree visibility of a 32-key block for one node: bit j of the result is set
// iff key kb0 + j is a prefix entry (an = kb0 + j - P_b < 0) or the verify
// token an is an ancestor-or-self of the node (bit an of its ancestor set).
// an0 = kb0 - P_b > -32; tokens at or past N (<= 256) have no bits, so keys
// past the sequence end are never visible.  Two words of the set are picked
// once per block and funnel-shifted, so each key costs one bit test.
__device__ __forceinline__ uint32_t anc_window(const uint32_t (&anc)[kAncWords], int an0) {
  const int w0 = an0 >> 5;  // -1 .. kAncWords - 1
  uint32_t lo = w0 < 0 ? 0xffffffffu : 0u, hi = 0u;
#pragma unroll
  for (int w = 0; w < kAncWords; ++w) {
    lo = (w == w0) ? anc[w] : lo;
    hi = (w == w0 + 1) ? anc[w] : hi;
  }
  return (uint32_t)(((((unsigned long long)hi) << 32) | lo) >> (an0 & 31));
}
// Visibility of lane (v, h)'s key kappa(v, h) in a block with window `win`.
__device__ __forceinline__ bool win_vis(uint32_t win, int v, int h) { return (win >> kappa(v, h)) & 1u; }

// 2-lane-shifted copies within a row of 16 lanes (DPP): lane i gets lane i + N's x (0 past the row end)
template <int N>
__device__ __forceinline__ float row_shl(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x100 + N, 0xf, 0xf, true));
}

template <typename T, int D, int RT, int WR, bool PAGED>
__global__ void __launch_bounds__(256) verify_main(const VerifyArgs a) {
  using RG = Ring<T, D>;
  constexpr int WK = 4 / WR;
  constexpr bool kBf16 = RG::kBf16;
  constexpr int DB = D / 32;  // 32-wide column blocks of the head dim
  constexpr int QN = kBf16 ? D / 16 : D / 2;
  constexpr int KRD = kBf16 ? D / 16 : D / 8;  // 16-byte K reads per 32-key block
  __shared__ __attribute__((aligned(1024))) char smem[RG::LDS];
  char* ring = smem;
  int* pt_lds = reinterpret_cast<int*>(smem + RG::MAIN);
  float* qs = reinterpret_cast<float*>(smem + RG::MAIN + RG::PT_CAP * 4);
  T* qbt = reinterpret_cast<T*>(smem + RG::MAIN + RG::PT_CAP * 4 + RG::AUX_FLOATS * 4);

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

  int L;
  const int Pb = seq_prefix(a, b, &L);
  // chunk c covers stages [c * nst / n_chunks, (c + 1) * nst / n_chunks) of
  // this sequence (balanced; an empty chunk still writes an empty partial)
  const int nst_seq = (L + RG::SK - 1) / RG::SK;
  const int c0 = (int)((long long)c * nst_seq / a.n_chunks) * RG::SK;
  const int c1 = min((int)((long long)(c + 1) * nst_seq / a.n_chunks) * RG::SK, L);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, lane32 = lane & 31, h = lane >> 5;
  const int wk = wave % WK, wr = wave / WK;

  // ---- page-table slice of this chunk -> LDS
  const int ps = a.kv.page_size;
  int pg0 = 0;
  bool pt_fits = true;  // every page of the chunk is in the cached slice
  if constexpr (PAGED) {
    pg0 = a.ps_shift >= 0 ? (c0 >> a.ps_shift) : c0 / ps;
    const int pg1 = a.ps_shift >= 0 ? ((c1 - 1) >> a.ps_shift) : (c1 - 1) / ps;
    pt_fits = pg1 - pg0 < RG::PT_CAP;
    for (int j = tid; j <= pg1 - pg0 && j < RG::PT_CAP; j += 256) {
      const int pg = pg0 + j;
      pt_lds[j] = pg < a.kv.max_pages ? a.kv.page_table[(long long)b * a.kv.max_pages + pg] : -1;
    }
    __syncthreads();
  }
  const long long seq_base = (long long)b * a.kv.seq_stride;
  // slot of a position: page entries from the cached slice (FROM_MEM: pages
  // past it are read from memory; the copy paths keep the two apart, so the
  // common one never waits on a memory read, which would also wait for every
  // copy already in flight)
  auto slot_of = [&](int pos, auto from_mem) -> long long {
    long long s;
    if constexpr (PAGED) {
      const int pg = a.ps_shift >= 0 ? (pos >> a.ps_shift) : pos / ps;
      const int jp = pg - pg0;
      int e;
      if constexpr (decltype(from_mem)::value)
        e = jp < RG::PT_CAP ? pt_lds[jp]
                            : (pg < a.kv.max_pages ? a.kv.page_table[(long long)b * a.kv.max_pages + pg] : -1);
      else
        e = pt_lds[jp < RG::PT_CAP ? jp : 0];
      s = e < 0 ? -1 : (long long)e * ps + (pos - pg * ps);
    } else {
      s = seq_base + pos;
    }
    return (s >= 0 && s < a.kv.num_slots) ? s : 0;  // unmapped positions read slot 0 (never visible)
  };

  // ---- global -> LDS copies of one stage.  A wave's LPW copies all go to the
  // same tensor (waves 0..1 fill K, 2..3 fill V); each lane's row and swizzled
  // column within the stage are the same for every stage, so they are set once.
  const bool wave_v = wave * RG::LPW >= RG::SEGS / 2;
  const char* tbase = reinterpret_cast<const char*>(wave_v ? a.kv.v : a.kv.k) + (long long)g * RG::ROWB;
  const long long slot_bytes = (long long)a.Hkv * RG::ROWB;
  int dma_row[RG::LPW], dma_off[RG::LPW];
#pragma unroll
  for (int j = 0; j < RG::LPW; ++j) {
    const int sgt = (wave * RG::LPW + j) % (RG::SEGS / 2);
    dma_row[j] = sgt * RG::RPS + lane / RG::CPR;
    const int cl = (lane % RG::CPR) ^ swz<T, D>(dma_row[j]);
    dma_off[j] = (int)(dma_row[j] * slot_bytes) + cl * 16;
  }
  const int n_st = c1 > c0 ? (c1 - c0 + RG::SK - 1) / RG::SK : 0;
  auto issue = [&](int i) {
    const int key0 = c0 + i * RG::SK;
    char* dst = ring + (i % RG::NS) * RG::STAGE + wave * RG::LPW * 1024;
    if (!PAGED && key0 + RG::SK <= c1 && seq_base + key0 + RG::SK <= a.kv.num_slots) {
      const char* base = tbase + (seq_base + key0) * slot_bytes;  // wave-uniform
#pragma unroll
      for (int j = 0; j < RG::LPW; ++j) global_to_lds16(base + dma_off[j], dst + j * 1024);
    } else if (pt_fits) {
#pragma unroll
      for (int j = 0; j < RG::LPW; ++j) {
        const int pos = key0 + dma_row[j];
        const long long sl = slot_of(pos < c1 ? pos : c0, std::false_type{});
        global_to_lds16(tbase + sl * slot_bytes + (dma_off[j] - (int)(dma_row[j] * slot_bytes)), dst + j * 1024);
      }
    } else {
#pragma unroll
      for (int j = 0; j < RG::LPW; ++j) {
        const int pos = key0 + dma_row[j];
        const long long sl = slot_of(pos < c1 ? pos : c0, std::true_type{});
        global_to_lds16(tbase + sl * slot_bytes + (dma_off[j] - (int)(dma_row[j] * slot_bytes)), dst + j * 1024);
      }
    }
  };
  for (int i = 0; i < RG::PD && i < n_st; ++i) issue(i);

  // ---- query fragments (B operand of S^T = K Q^T): lane column = query row
  typedef typename std::conditional<kBf16, bf16x8, float>::type QElem;
  QElem qf[RT][QN];
  int row_node[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = ((rb * WR + wr) * RT + rt) * 32 + lane32;
    const bool ok = r < a.R;
    const int t = ok ? r / a.G : a.N - 1;
    row_node[rt] = t;
    const int j = ok ? r % a.G : 0;
    const T* qrow = reinterpret_cast<const T*>(a.q) + ((long long)(b * a.N + t) * a.Hq + g * a.G + j) * D;
    if constexpr (kBf16) {
#pragma unroll
      for (int ks = 0; ks < QN; ++ks) {
        bf16x8 x = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks + 8 * h);
        qf[rt][ks] = ok ? x : bf16x8{};
      }
    } else {
#pragma unroll
      for (int cc = 0; cc < D / 8; ++cc) {
        f32x4 x = *reinterpret_cast<const f32x4*>(qrow + 8 * cc + 4 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e) qf[rt][4 * cc + e] = ok ? x[e] : 0.f;
      }
    }
  }

  // ---- score operand: qbar_g (fp32) split into bf16 hi + mid + lo, kept in
  // LDS as three rows; they become MFMA columns 0..2 of S^T's companion tile
  const bool wg_scores = a.do_scores && c0 < Pb;  // key blocks are shared out over the row blocks
  if (wg_scores) {
    if (a.prep_qbar) {
      for (int d = tid; d < D; d += 256) {
        const float* part = a.ws_qbar + (long long)(b * a.Hkv + g) * a.qsplit * D + d;
        float acc = 0.f;
        for (int sp0 = 0; sp0 < a.qsplit; sp0 += 16) {
          // sixteen loads at clamped places issued together, then summed in order (a
          // bounded loop's load per step would be one trip to memory each)
          float x[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) x[u] = part[min(sp0 + u, a.qsplit - 1) * D];
#pragma unroll
          for (int u = 0; u < 16; ++u) acc += sp0 + u < a.qsplit ? x[u] : 0.f;
        }
        qs[d] = acc;
      }
    } else {
      constexpr int NP = 256 / D;
      const int d = tid % D, part = tid / D;
      const int npairs = a.n_score_rows * a.G;
      float acc = 0.f;
      for (int i0 = part; i0 < npairs; i0 += 8 * NP) {
        // eight pairs at a time: their row indices, then their query elements, each
        // step's loads issued together at clamped places, then summed in order
        int t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) t[u] = a.score_rows[min(i0 + u * NP, npairs - 1) / a.G];
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int j = min(i0 + u * NP, npairs - 1) % a.G;
          x[u] = (float)reinterpret_cast<const T*>(a.q)[((long long)(b * a.N + t[u]) * a.Hq + g * a.G + j) * D + d];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += i0 + u * NP < npairs ? x[u] : 0.f;
      }
      qs[D + part * D + d] = acc;
      __syncthreads();
      if (tid < D) {
        float sacc = 0.f;
        for (int p = 0; p < NP; ++p) sacc += qs[D + p * D + tid];
        qs[tid] = sacc;
      }
    }
    __syncthreads();
    for (int d = tid; d < D; d += 256) {
      const float x = qs[d];
      if constexpr (kBf16) {
        const bf16 hi = (bf16)x;
        const float r1 = x - (float)hi;
        const bf16 mid = (bf16)r1;
        const bf16 lo = (bf16)(r1 - (float)mid);
        qbt[d] = hi;
        qbt[D + d] = mid;
        qbt[2 * D + d] = lo;
      } else {
        qbt[d] = x;
      }
    }
    __syncthreads();
  }
  // B-operand fragment of the score tile for k-step ks (nonzero only in lanes of columns 0..2)
  auto qb_frag = [&](int ks) -> QElem {
    if constexpr (kBf16) {
      bf16x8 v = bf16x8{};
      if (lane32 < 3) v = *reinterpret_cast<const bf16x8*>(qbt + lane32 * D + 16 * ks + 8 * h);
      return v;
    } else {
      const int d = 8 * (ks >> 2) + 4 * h + (ks & 3);
      return lane32 == 0 ? qbt[d] : 0.f;
    }
  };

  // ---- ancestor bitsets of this lane's rows (tree, chunk reaching the verify tokens)
  uint32_t anc[RT][kAncWords] = {};
  if (a.tree && c1 > Pb) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int w = 0; w < kAncWords; ++w) anc[rt][w] = a.ws_anc[((long long)b * a.N + row_node[rt]) * kAncWords + w];
  }

  // ---- per-lane LDS offsets of the MFMA operand reads inside a 32-key block;
  // the swizzle depends on row & 15 only, so blocks and stages just add a base
  int koff[KRD];
#pragma unroll
  for (int kr = 0; kr < KRD; ++kr) koff[kr] = tile_off<T, D>(lane32, 2 * kr + h);
  const int e4 = (lane & 15) >> 2, cq = lane & 3, dh = (lane >> 4) & 1;
  int voff[kBf16 ? DB : 1][2];
  if constexpr (kBf16) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int hl = 0; hl < 2; ++hl)
        voff[db][hl] = tile_off<T, D>(4 * h + e4 + 8 * hl, 4 * db + 2 * dh + (cq >> 1)) + (cq & 1) * 8;
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

  for (int i = 0; i < n_st; ++i) {
    // stage i has landed once at most (stages issued after it) x LPW copies are outstanding
    const int after = min(RG::PD - 1, n_st - 1 - i);
    if (after >= 2) wait_vm_lgkm0<2 * RG::LPW>();
    else if (after == 1) wait_vm_lgkm0<RG::LPW>();
    else wait_vm_lgkm0<0>();
    barrier_only();
    // the buffer of stage i + PD was last read in iteration i - 1, which every wave has finished
    if (i + RG::PD < n_st) issue(i + RG::PD);

    const char* Kt = ring + (i % RG::NS) * RG::STAGE;
    const char* Vt = Kt + RG::TILE;
    // S^T of block kb of this stage (and, for one wave of one row block per
    // key block, the score columns)
    auto qk_block = [&](int kb, f32x16 (&s)[RT]) {
      const int gb = i * RG::NB + kb;
      const int kb0 = c0 + 32 * gb;
      const int jblk = kb0 >> 5;  // key block index within the sequence
      const bool do_score = wg_scores && kb0 < Pb && (jblk % a.RB) == rb && ((jblk / a.RB) % WR) == wr;
      const char* Kb = Kt + kb * 32 * RG::ROWB;
      // S^T = K Q^T in two independent accumulation chains (and the score columns)
      f32x16 s2[RT];
      f32x16 sc = f32x16{};
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        s[rt] = f32x16{};
        s2[rt] = f32x16{};
      }
      if constexpr (kBf16) {
        bf16x8 ka[QN];
#pragma unroll
        for (int ks = 0; ks < QN; ++ks) ka[ks] = *reinterpret_cast<const bf16x8*>(Kb + koff[ks]);
#pragma unroll
        for (int ks = 0; ks < QN; ++ks) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            if (ks & 1) s2[rt] = mfma_bf16(ka[ks], qf[rt][ks], s2[rt]);
            else s[rt] = mfma_bf16(ka[ks], qf[rt][ks], s[rt]);
          }
          if (do_score) sc = mfma_bf16(ka[ks], qb_frag(ks), sc);
        }
      } else {
#pragma unroll
        for (int cc = 0; cc < D / 8; ++cc) {
          const f32x4 ka = *reinterpret_cast<const f32x4*>(Kb + koff[cc]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
              if (e & 1) s2[rt] = mfma_f32(ka[e], qf[rt][4 * cc + e], s2[rt]);
              else s[rt] = mfma_f32(ka[e], qf[rt][4 * cc + e], s[rt]);
            }
            if (do_score) sc = mfma_f32(ka[e], qb_frag(4 * cc + e), sc);
          }
        }
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) s[rt] += s2[rt];

      if (do_score) {
        // column sum hi + mid + lo (lanes 0..2 / 32..34 of their 16-lane rows), written by lanes 0 and 32
        float tv[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float x = sc[v];
          if constexpr (kBf16) x = x + row_shl<1>(sc[v]) + row_shl<2>(sc[v]);
          tv[v] = x * a.scale;
        }
        if (lane32 == 0) {  // whole block (rows are padded by 32; entries past P_b are never read)
          float* dst = a.ws_s + ((long long)b * a.Hkv + g) * a.s_stride;
#pragma unroll
          for (int qd = 0; qd < 4; ++qd)
            *reinterpret_cast<f32x4*>(dst + kb0 + 8 * qd + 4 * h) =
                f32x4{tv[4 * qd], tv[4 * qd + 1], tv[4 * qd + 2], tv[4 * qd + 3]};
        }
      }

    };
    // mask, online softmax and O^T += V^T P^T of block kb
    auto finish_block = [&](int kb, f32x16 (&s)[RT]) {
      const int gb = i * RG::NB + kb;
      const int kb0 = c0 + 32 * gb;
      const char* Vb = Vt + kb * 32 * RG::ROWB;
      // mask: keys past the chunk end, and verify tokens that are not ancestors-or-self
      if (kb0 + 32 > min(Pb, c1)) {
        if (a.tree) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const uint32_t win = kb0 + 32 > Pb ? anc_window(anc[rt], kb0 - Pb) : 0xffffffffu;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const bool vis = kb0 + kappa(v, h) < c1 && win_vis(win, v, h);
              s[rt][v] = vis ? s[rt][v] : kNegInf;
            }
          }
        } else {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int key = kb0 + kappa(v, h);
              s[rt][v] = (key < c1 && key - Pb <= row_node[rt]) ? s[rt][v] : kNegInf;
            }
        }
      }

      // online softmax (log2 domain); the O rescale is skipped when no row's max moved
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float mx = kNegInf;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          s[rt][v] *= a.scale_log2;
          mx = fmaxf(mx, s[rt][v]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool grew = mx > m[rt];
        const float mn = grew ? mx : m[rt];
        const bool live = mn != kNegInf;
        float psum = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = live ? fast_exp2(s[rt][v] - mn) : 0.f;
          s[rt][v] = p;
          psum += p;
        }
        if (__any(grew)) {
          const float alpha = grew ? fast_exp2(m[rt] - mn) : 1.f;
          l[rt] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) o[rt][db] *= alpha;
        }
        l[rt] += psum;
        m[rt] = mn;
      }

      // O^T += V^T P^T
      if constexpr (kBf16) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          bf16x8 pb[RT];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int u = 0; u < 8; ++u) pb[rt][u] = (bf16)s[rt][8 * jj + u];
          const char* Vj = Vb + jj * 16 * RG::ROWB;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x4 lo = lds_read_tr16(reinterpret_cast<const T*>(Vj + voff[db][0]));
            const bf16x4 hi = lds_read_tr16(reinterpret_cast<const T*>(Vj + voff[db][1]));
            const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) o[rt][db] = mfma_bf16(va, pb[rt], o[rt][db]);
          }
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int vr = kappa(v, h);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const float va = *reinterpret_cast<const float*>(
                Vb + tile_off<T, D>(vr, 8 * db + (lane32 >> 2)) + (lane32 & 3) * 4);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) o[rt][db] = mfma_f32(va, s[rt][v], o[rt][db]);
          }
        }
      }
    };
    if constexpr (WK == 1) {
      // every wave takes every block of the stage: issue both blocks' S^T
      // products before the first softmax so the matrix cores stay busy
      // while the vector unit works
      f32x16 sb[RG::NB][RT];
#pragma unroll
      for (int kb = 0; kb < RG::NB; ++kb)
        if (c0 + 32 * (i * RG::NB + kb) < c1) qk_block(kb, sb[kb]);
#pragma unroll
      for (int kb = 0; kb < RG::NB; ++kb)
        if (c0 + 32 * (i * RG::NB + kb) < c1) finish_block(kb, sb[kb]);
    } else {
#pragma unroll
      for (int kb = 0; kb < RG::NB; ++kb) {
        const int gb = i * RG::NB + kb;
        if ((gb % WK) != wk) continue;
        if (c0 + 32 * gb >= c1) break;
        f32x16 s[RT];
        qk_block(kb, s);
        finish_block(kb, s);
      }
    }
  }

  // ---- epilogue: combine the WK waves that share rows, write (m, l, o) partials
  wait_vm_lgkm0<0>();
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

// ---------------------------------------------------------------------------
// Streaming kernel for few query rows per KV head (bf16, N * G <= 64: chains
// and small trees).  All rows of a KV head fit one or two 32-column MFMA
// tiles, so the four waves of a workgroup split the keys instead of the rows:
// each wave owns a contiguous run of 32-key blocks and a private LDS ring that
// only it fills (global->LDS copies) and reads.  Nothing is shared between
// waves until the epilogue, so the loop has no workgroup barrier and every
// wave streams at its own pace.  Per block the wave computes S^T = K Q^T
// (plus the score columns), the online softmax and O^T += V^T P^T exactly as
// verify_main does.
template <int D>
struct WaveRing {
  static constexpr int ROWB = D * 2;             // bytes of one head's bf16 row
  static constexpr int CPR = ROWB / 16;          // 16-byte chunks per row
  static constexpr int RPI = 1024 / ROWB;        // rows per 1 KB copy instruction
  static constexpr int TILE = 32 * ROWB;         // K (or V) bytes of a 32-key block
  static constexpr int LPT = TILE / 1024;        // copy instructions per tile
  static constexpr int BLK = 2 * TILE;           // K + V of a block
  static constexpr int NSW = D == 128 ? 2 : 4;   // blocks in a wave's ring
  static constexpr int WAVE = NSW * BLK;
  static constexpr int RING = 4 * WAVE;
  static constexpr int EPI_OS = D + 4;          // epilogue row stride (floats): 16-byte pad spreads banks
  static constexpr int EPI = 4 * 32 * EPI_OS * 4 + 4 * 32 * 4 * 4;
  static constexpr int MAIN = RING > EPI ? RING : EPI;
  static constexpr int PT_CAP = 1024;            // cached page-table entries per chunk
  static constexpr int AUX_FLOATS = 512;
  static constexpr int QBT = 3 * D * 2;
  static constexpr int LDS = MAIN + PT_CAP * 4 + AUX_FLOATS * 4 + QBT;
  static_assert(LPT * 1024 == TILE && RPI * ROWB == 1024, "wave ring geometry");
};

// One 16-byte-per-lane global->LDS copy (1 KB per wave).  `lds` is the
// wave-uniform LDS byte address, `off` a per-lane 32-bit offset from the
// wave-uniform base `base` (the scalar-base form of the instruction).  The
// copies carry the non-temporal hint: K/V is streamed, and the hint took the
// 32k step from 63.6 to 59.2 us (the 4 x 128k batch from 769 to 697 us).
// The LDS address (m0) and the scalar base must sit in scalar registers: both
// are wave-uniform by construction, and readfirstlane says so to the compiler
// (which otherwise may keep a uniform value in a vector register).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const unsigned long long u = reinterpret_cast<unsigned long long>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return reinterpret_cast<const void*>(((unsigned long long)hi << 32) | lo);
}
__device__ __forceinline__ void dma16_sbase(uint32_t lds, uint32_t off, const void* base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(__builtin_amdgcn_readfirstlane(lds)),
               "v"(off), "s"(uniform_ptr(base)) : "memory");
}
__device__ __forceinline__ void dma16_vaddr(uint32_t lds, const void* addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(__builtin_amdgcn_readfirstlane(lds)),
               "v"(addr) : "memory");
}
// s_waitcnt vmcnt(n) lgkmcnt(0) for a run-time n in {0, step, 2 step, 3 step}
template <int STEP>
__device__ __forceinline__ void wait_blocks_after(int blocks) {
  if (blocks >= 3) wait_vm_lgkm0<3 * STEP>();
  else if (blocks == 2) wait_vm_lgkm0<2 * STEP>();
  else if (blocks == 1) wait_vm_lgkm0<STEP>();
  else wait_vm_lgkm0<0>();
}

// Combine lane l with lane l ^ 32.  v_permlane32_swap with both operands equal
// returns {x of lanes 0-31 in both halves, x of lanes 32-63 in both halves}.
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// Lazy rescale threshold (log2 units): the running max is only moved when a
// block's max exceeds it by more than this, so p <= 2^8 and O is rescaled a
// handful of times per chunk instead of per block.
constexpr float kRescaleSlack = 8.f;

template <int D, int RT, bool PAGED>
__global__ void __launch_bounds__(256) verify_stream(const VerifyArgs a) {
  using WRg = WaveRing<D>;
  using T = bf16;
  constexpr int DB = D / 32;
  constexpr int QN = D / 16;
  constexpr int STEP = 2 * WRg::LPT;  // copy instructions per block
  __shared__ __attribute__((aligned(1024))) char smem[WRg::LDS];
  int* pt_lds = reinterpret_cast<int*>(smem + WRg::MAIN);
  float* qs = reinterpret_cast<float*>(smem + WRg::MAIN + WRg::PT_CAP * 4);
  T* qbt = reinterpret_cast<T*>(smem + WRg::MAIN + WRg::PT_CAP * 4 + WRg::AUX_FLOATS * 4);

  // ---- workgroup -> (sequence, KV head, chunk).  Batches: chunk c runs on XCD
  // c % 8 (blockIdx % 8 picks the XCD), so every XCD gets a slice of every
  // sequence and head whatever the lengths.  One sequence: each XCD streams
  // whole heads (consecutive chunks), which measured slightly faster.
  // Every argument the first copies need is read here, before anything
  // branches, so the loads go out together: each one first read behind a
  // branch or a division was its own trip to memory (the argument block is
  // not in the scalar cache when a launch starts).
  const int aB = a.B, aHkv = a.Hkv, ach = a.n_chunks, anu = a.n_units, aN = a.N, aPmax = a.P_max,
            alb = a.len_bias;
  const int32_t* apl = a.prefix_len;
  const char* kbase = reinterpret_cast<const char*>(a.kv.k);
  const char* vbase = reinterpret_cast<const char*>(a.kv.v);
  const long long sstr = a.kv.seq_stride, nslots = a.kv.num_slots;
  // used here, so that their line of the argument block comes with the first
  // trip (the test never fires: the host rejects null caches)
  if (kbase == nullptr || nslots <= 0 || aB <= 0 || ach <= 0) return;
  int c, g, b;
  if (aB > 1) {
    c = (int)(blockIdx.x >> 3) / (aB * aHkv) * 8 + (int)(blockIdx.x & 7);
    g = (int)(blockIdx.x >> 3) % aHkv;
    b = (int)(blockIdx.x >> 3) / aHkv % aB;
    if (c >= ach) return;
  } else {
    // one sequence: the grid holds the units rounded up to whole XCD rows
    const int lid = (int)(blockIdx.x & 7) * ((anu + 7) >> 3) + (int)(blockIdx.x >> 3);
    if (lid >= anu) return;
    c = lid % ach;
    g = lid / ach;
    b = 0;
  }
  int L, Pb;
  {
    int x = apl[b] + alb;
    const bool empty = alb < 0 && x < 0;
    Pb = x < 0 ? 0 : (x > aPmax ? aPmax : x);
    L = empty ? 0 : Pb + aN;
  }
  const int nbk = (L + 31) >> 5;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lane32 = lane & 31, h = lane >> 5;

  // balanced split of the sequence's blocks over all waves of all its chunks
  const long long WT = (long long)ach * 4;
  const int blk0 = (int)((long long)(c * 4 + wave) * nbk / WT);
  const int blk1 = (int)((long long)(c * 4 + wave + 1) * nbk / WT);
  const int cblk0 = (int)((long long)c * 4 * nbk / WT);
  const int cblk1 = (int)((long long)(c * 4 + 4) * nbk / WT);

  // ---- page-table slice of this chunk -> LDS
  const int ps = a.kv.page_size;
  int pg0 = 0;
  bool pt_fits = true;  // every page of the chunk is in the cached slice
  if constexpr (PAGED) {
    const int k0 = cblk0 * 32, k1 = min(cblk1 * 32, L);
    if (k1 > k0) {
      pg0 = a.ps_shift >= 0 ? (k0 >> a.ps_shift) : k0 / ps;
      const int pg1 = a.ps_shift >= 0 ? ((k1 - 1) >> a.ps_shift) : (k1 - 1) / ps;
      pt_fits = pg1 - pg0 < WRg::PT_CAP;
      for (int j = tid; j <= pg1 - pg0 && j < WRg::PT_CAP; j += 256) {
        const int pg = pg0 + j;
        pt_lds[j] = pg < a.kv.max_pages ? a.kv.page_table[(long long)b * a.kv.max_pages + pg] : -1;
      }
    }
    __syncthreads();
  }
  const long long seq_base = (long long)b * sstr;
  // slot of a position: page entries from the cached slice (FROM_MEM: pages
  // past it are read from memory; the copy paths keep the two apart, so the
  // common one never waits on a memory read, which would also wait for every
  // copy already in flight)
  auto slot_of = [&](int pos, auto from_mem) -> long long {
    long long sl;
    if constexpr (PAGED) {
      const int pg = a.ps_shift >= 0 ? (pos >> a.ps_shift) : pos / ps;
      const int jp = pg - pg0;
      int e;
      if constexpr (decltype(from_mem)::value)
        e = jp < WRg::PT_CAP ? pt_lds[jp]
                             : (pg < a.kv.max_pages ? a.kv.page_table[(long long)b * a.kv.max_pages + pg] : -1);
      else
        e = pt_lds[jp < WRg::PT_CAP ? jp : 0];
      sl = e < 0 ? -1 : (long long)e * ps + (pos - pg * ps);
    } else {
      sl = seq_base + pos;
    }
    return (sl >= 0 && sl < a.kv.num_slots) ? sl : 0;  // unmapped positions read slot 0 (never visible)
  };

  // ---- copies of one block into ring slot `st` (K tile, then V tile)
  const uint32_t ring_l =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem) +
      (uint32_t)(wave * WRg::WAVE);
  const long long slot_bytes = (long long)a.Hkv * WRg::ROWB;
  const char* kg = kbase + (long long)g * WRg::ROWB;
  const char* vg = vbase + (long long)g * WRg::ROWB;
  uint32_t doff[WRg::LPT];  // per-lane offset of copy j inside a contiguous block
  int drow[WRg::LPT], dcol[WRg::LPT];
#pragma unroll
  for (int j = 0; j < WRg::LPT; ++j) {
    drow[j] = j * WRg::RPI + lane / WRg::CPR;
    dcol[j] = ((lane % WRg::CPR) ^ swz<T, D>(drow[j])) * 16;
    doff[j] = (uint32_t)(drow[j] * slot_bytes) + (uint32_t)dcol[j];
  }
  // copies of one tile (K if !is_v, else V) of block `blk` into ring slot `st`
  auto issue = [&](int blk, int st, bool is_v) {
    const int key0 = blk * 32;
    const uint32_t ld = ring_l + (uint32_t)(st * WRg::BLK + (is_v ? WRg::TILE : 0));
    const char* tg = is_v ? vg : kg;
    if (!PAGED && key0 + 32 <= L && seq_base + key0 + 32 <= nslots) {
      const char* bt = tg + (seq_base + key0) * slot_bytes;
#pragma unroll
      for (int j = 0; j < WRg::LPT; ++j) dma16_sbase(ld + j * 1024, doff[j], bt);
    } else if (pt_fits) {
#pragma unroll
      for (int j = 0; j < WRg::LPT; ++j) {
        const int pos = key0 + drow[j];
        dma16_vaddr(ld + j * 1024, tg + slot_of(pos < L ? pos : key0, std::false_type{}) * slot_bytes + dcol[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < WRg::LPT; ++j) {
        const int pos = key0 + drow[j];
        dma16_vaddr(ld + j * 1024, tg + slot_of(pos < L ? pos : key0, std::true_type{}) * slot_bytes + dcol[j]);
      }
    }
  };
  // the first block's copies, then the query loads, then the other ring slot's
  // copies: the query fragments arrive ahead of the second block (measured 0.6 us
  // faster at 32k than both blocks first)
  const int nb = blk1 - blk0;
  if (nb > 0) {
    issue(blk0, 0, false);
    issue(blk0, 0, true);
  }

  // ---- query fragments (B operand of S^T = K Q^T): lane column = query row
  bf16x8 qf[RT][QN];
  int row_node[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = rt * 32 + lane32;
    const bool ok = r < a.R;
    const int t = ok ? r / a.G : a.N - 1;
    row_node[rt] = t;
    const int j = ok ? r % a.G : 0;
    const T* qrow = reinterpret_cast<const T*>(a.q) + ((long long)(b * a.N + t) * a.Hq + g * a.G + j) * D;
#pragma unroll
    for (int ks = 0; ks < QN; ++ks) {
      bf16x8 x = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks + 8 * h);
      qf[rt][ks] = ok ? x : bf16x8{};
    }
  }

  for (int i = 1; i < WRg::NSW && i < nb; ++i) {
    issue(blk0 + i, i, false);
    issue(blk0 + i, i, true);
  }

  // ---- score operand: scale * qbar_g split into bf16 hi + mid + lo = B columns 0..2
  const bool wg_scores = a.do_scores && cblk0 * 32 < Pb;
  bf16x8 qbf[QN];
  if (wg_scores) {
    if (a.prep_qbar) {
      for (int d = tid; d < D; d += 256) {
        const float* part = a.ws_qbar + (long long)(b * a.Hkv + g) * a.qsplit * D + d;
        float acc = 0.f;
        for (int sp0 = 0; sp0 < a.qsplit; sp0 += 16) {
          // sixteen loads at clamped places issued together, then summed in order (a
          // bounded loop's load per step would be one trip to memory each)
          float x[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) x[u] = part[min(sp0 + u, a.qsplit - 1) * D];
#pragma unroll
          for (int u = 0; u < 16; ++u) acc += sp0 + u < a.qsplit ? x[u] : 0.f;
        }
        qs[d] = acc;
      }
    } else {
      constexpr int NP = 256 / D;
      const int d = tid % D, part = tid / D;
      const int npairs = a.n_score_rows * a.G;
      float acc = 0.f;
      for (int i0 = part; i0 < npairs; i0 += 8 * NP) {
        // eight pairs at a time: their row indices, then their query elements, each
        // step's loads issued together at clamped places, then summed in order
        int t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) t[u] = a.score_rows[min(i0 + u * NP, npairs - 1) / a.G];
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int j = min(i0 + u * NP, npairs - 1) % a.G;
          x[u] = (float)reinterpret_cast<const T*>(a.q)[((long long)(b * a.N + t[u]) * a.Hq + g * a.G + j) * D + d];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += i0 + u * NP < npairs ? x[u] : 0.f;
      }
      qs[D + part * D + d] = acc;
      __syncthreads();
      if (tid < D) {
        float sacc = 0.f;
        for (int p = 0; p < NP; ++p) sacc += qs[D + p * D + tid];
        qs[tid] = sacc;
      }
    }
    __syncthreads();
    for (int d = tid; d < D; d += 256) {
      const float x = qs[d] * a.scale;
      const bf16 hi = (bf16)x;
      const float r1 = x - (float)hi;
      const bf16 mid = (bf16)r1;
      const bf16 lo = (bf16)(r1 - (float)mid);
      qbt[d] = hi;
      qbt[D + d] = mid;
      qbt[2 * D + d] = lo;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < QN; ++ks)
      qbf[ks] = lane32 < 3 ? *reinterpret_cast<const bf16x8*>(qbt + lane32 * D + 16 * ks + 8 * h) : bf16x8{};
  } else {
#pragma unroll
    for (int ks = 0; ks < QN; ++ks) qbf[ks] = bf16x8{};
  }

  // ---- ancestor bitsets of this lane's rows (trees, for blocks holding verify tokens)
  uint32_t anc[RT][kAncWords] = {};
  if (a.tree && blk1 * 32 > Pb) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int w = 0; w < kAncWords; ++w) anc[rt][w] = a.ws_anc[((long long)b * a.N + row_node[rt]) * kAncWords + w];
    // wait for the words here (all loads in flight together), not inside the loop
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
      asm volatile("" ::"v"(anc[rt][0]), "v"(anc[rt][1]), "v"(anc[rt][2]), "v"(anc[rt][3]), "v"(anc[rt][4]),
                   "v"(anc[rt][5]), "v"(anc[rt][6]), "v"(anc[rt][7]));
  }

  // ---- per-lane LDS offsets of the operand reads inside a block
  int koff[QN];
#pragma unroll
  for (int kr = 0; kr < QN; ++kr) koff[kr] = tile_off<T, D>(lane32, 2 * kr + h);
  const int e4 = (lane & 15) >> 2, cq = lane & 3, dh = (lane >> 4) & 1;
  int voff[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int hl = 0; hl < 2; ++hl)
      voff[db][hl] = tile_off<T, D>(4 * h + e4 + 8 * hl, 4 * db + 2 * dh + (cq >> 1)) + (cq & 1) * 8;

  f32x16 o[RT][DB];
  float m[RT], l[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = kNegInf;
    l[rt] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[rt][db] = f32x16{};
  }
  float* sdst = a.ws_s + ((long long)b * a.Hkv + g) * a.s_stride;
  float pend[16];
  int pend_key = -1;  // first key of the block whose scores are pending (wave-uniform)
  auto flush_scores = [&]() {  // whole block (rows are padded by 32; entries past P_b are never read)
    if (pend_key >= 0 && lane32 == 0) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        *reinterpret_cast<f32x4*>(sdst + pend_key + 8 * qd + 4 * h) =
            f32x4{pend[4 * qd], pend[4 * qd + 1], pend[4 * qd + 2], pend[4 * qd + 3]};
    }
  };
  const char* wring = smem + wave * WRg::WAVE;

  for (int i = 0; i < nb; ++i) {
    // block i has landed once only the copies of later blocks (and the score
    // stores issued before them, see flush_scores) can still be outstanding;
    // loads complete in order, so vmcnt <= later copies means block i is in LDS
    wait_blocks_after<STEP>(min(WRg::NSW - 1, nb - 1 - i));
    flush_scores();
    const int st = i % WRg::NSW;
    const int blk = blk0 + i;
    const int key0 = blk * 32;
    const char* Kb = wring + st * WRg::BLK;
    const char* Vb = Kb + WRg::TILE;
    const bool do_score = wg_scores && key0 < Pb;

    f32x16 s[RT];
    f32x16 sc = f32x16{};
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) s[rt] = f32x16{};
    {
      bf16x8 ka[QN];
#pragma unroll
      for (int ks = 0; ks < QN; ++ks) ka[ks] = *reinterpret_cast<const bf16x8*>(Kb + koff[ks]);
      if (do_score) {
#pragma unroll
        for (int ks = 0; ks < QN; ++ks) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) s[rt] = mfma_bf16(ka[ks], qf[rt][ks], s[rt]);
          sc = mfma_bf16(ka[ks], qbf[ks], sc);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < QN; ++ks)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) s[rt] = mfma_bf16(ka[ks], qf[rt][ks], s[rt]);
      }
    }
    // the K tile of this slot is consumed: refill it with block i + NSW (the
    // wait makes sure every LDS read of it has returned before the copy starts)
    if (i + WRg::NSW < nb) {
      wait_lgkm0();
      issue(blk + WRg::NSW, st, false);
    }

    if (do_score) {
#pragma unroll
      for (int v = 0; v < 16; ++v) pend[v] = sc[v] + row_shl<1>(sc[v]) + row_shl<2>(sc[v]);
      pend_key = key0;
    } else {
      pend_key = -1;
    }

    // mask (blocks reaching the verify tokens): key j is visible iff j < P_b or
    // j - P_b is an ancestor-or-self of the row's node (chains: j - P_b <= t);
    // positions at or past P_b + N are never ancestors, so they drop out too
    if (key0 + 32 > Pb) {
      if (a.tree) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const uint32_t win = anc_window(anc[rt], key0 - Pb);
#pragma unroll
          for (int v = 0; v < 16; ++v) s[rt][v] = win_vis(win, v, h) ? s[rt][v] : kNegInf;
        }
      } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int an = key0 + kappa(v, h) - Pb;
            s[rt][v] = an <= row_node[rt] ? s[rt][v] : kNegInf;
          }
      }
    }

    // online softmax, log2 domain, lazy rescale
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float mx = s[rt][0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, s[rt][v]);
      mx = half_max(mx) * a.scale_log2;
      const bool grew = mx > m[rt] + kRescaleSlack;
      if (__any(grew)) {
        const float mn = grew ? mx : m[rt];
        const float alpha = grew ? fast_exp2(m[rt] - mn) : 1.f;
        l[rt] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[rt][db] *= alpha;
        m[rt] = mn;
      }
      const float mneg = m[rt] == kNegInf ? 0.f : -m[rt];
      float psum = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = fast_exp2(__builtin_fmaf(s[rt][v], a.scale_log2, mneg));
        s[rt][v] = p;
        psum += p;
      }
      l[rt] += psum;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      bf16x8 pb[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int u = 0; u < 8; ++u) pb[rt][u] = (bf16)s[rt][8 * jj + u];
      const char* Vj = Vb + jj * 16 * WRg::ROWB;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const bf16x4 lo = lds_read_tr16(reinterpret_cast<const T*>(Vj + voff[db][0]));
        const bf16x4 hi = lds_read_tr16(reinterpret_cast<const T*>(Vj + voff[db][1]));
        const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) o[rt][db] = mfma_bf16(va, pb[rt], o[rt][db]);
      }
    }
    if (i + WRg::NSW < nb) {  // likewise for the V tile
      wait_lgkm0();
      issue(blk + WRg::NSW, st, true);
    }
  }
  flush_scores();

  // ---- epilogue: combine the four waves (same rows, disjoint keys), write (m, l, o) partials.
  // No copy is in flight any more (the last block waited for all of them); the
  // score stores may be, and nothing here needs them, so only LDS is waited for.
  // Each wave rescales its own accumulators to the rows' common maximum, the
  // rescaled tiles meet in LDS, and all threads sum them in wave order.
  wait_lgkm0();
  barrier_only();
  constexpr int OS = WRg::EPI_OS;
  float* lo_ = reinterpret_cast<float*>(smem);  // [4 waves][32 rows][OS]
  float* lml = lo_ + 4 * 32 * OS;                // [4 waves][32 rows][m, l, -, -]
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float lt = half_sum(l[rt]);
    if (rt > 0) {  // the previous tile's reads are done before its LDS is reused
      wait_lgkm0();
      barrier_only();
    }
    if (h == 0) lml[(wave * 32 + lane32) * 4] = m[rt];
    wait_lgkm0();
    barrier_only();
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, lml[(w * 32 + lane32) * 4]);
    const float wt = (M == kNegInf || m[rt] == kNegInf) ? 0.f : fast_exp2(m[rt] - M);
    float* orow = lo_ + (wave * 32 + lane32) * OS;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * qd + 4 * h) =
            f32x4{wt * o[rt][db][4 * qd], wt * o[rt][db][4 * qd + 1], wt * o[rt][db][4 * qd + 2], wt * o[rt][db][4 * qd + 3]};
    if (h == 0) lml[(wave * 32 + lane32) * 4 + 1] = wt * lt;
    wait_lgkm0();
    barrier_only();
    // thread -> (row, 16 columns): four float4 groups, each summed over the waves in order
    {
      constexpr int TPR = 256 / 32;      // threads per row
      constexpr int CPT = D / TPR;       // columns per thread
      const int r = tid / TPR, cg = tid % TPR;
      const int row = rt * 32 + r;
      f32x4 acc[CPT / 4];
#pragma unroll
      for (int i = 0; i < CPT / 4; ++i) {
        const int d = cg * CPT + 4 * i;
        acc[i] = *reinterpret_cast<const f32x4*>(lo_ + (0 * 32 + r) * OS + d);
#pragma unroll
        for (int w = 1; w < 4; ++w) acc[i] += *reinterpret_cast<const f32x4*>(lo_ + (w * 32 + r) * OS + d);
      }
      if (row < a.R) {
        const long long rec = ((long long)(b * a.Hkv + g) * a.Rpad + row) * a.n_chunks + c;
#pragma unroll
        for (int i = 0; i < CPT / 4; ++i)  // bf16 partials, as the tree kernel's
          *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(a.ws_o) + rec * D + cg * CPT + 4 * i) =
              bf16x4{(bf16)acc[i][0], (bf16)acc[i][1], (bf16)acc[i][2], (bf16)acc[i][3]};
        if (cg == 0) {
          float Mr = kNegInf, Lr = 0.f;
#pragma unroll
          for (int w = 0; w < 4; ++w) Mr = fmaxf(Mr, lml[(w * 32 + r) * 4]);
#pragma unroll
          for (int w = 0; w < 4; ++w) Lr += lml[(w * 32 + r) * 4 + 1];
          a.ws_ml[rec] = f32x2{Mr, Lr};
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Tree kernel for many query rows per KV head (bf16, N * G > 64: draft trees
// and long chains).  Eight waves per workgroup, each owning one 32-row tile of
// a block of 256 rows; all waves read the same K/V tiles from a 4-stage LDS
// ring that they fill together (global->LDS copies, one barrier per stage).
// Two waves share each SIMD, so one wave's softmax runs on the vector unit
// while the other's products run on the matrix cores, and within a wave both
// blocks' S^T products of a stage are issued before the first softmax.  No two
// waves hold the same rows, so each writes its own (m, l, o) partials.
constexpr int kTreeWaves = 8;

// Inclusive prefix sum over the 64 lanes (DPP row shifts, then the row
// broadcasts of lanes 15 and 31).
__device__ __forceinline__ int wave_incl_sum(int x) {
  x += (int)__builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);
  x += (int)__builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);
  x += (int)__builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);
  x += (int)__builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);
  x += (int)__builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);
  x += (int)__builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);
  return x;
}
// The lowest lane whose x exceeds v (x non-decreasing over the lanes; 64 if none).
__device__ __forceinline__ int first_lane_above(int x, int v) {
  const unsigned long long m = __ballot(x > v);
  return m ? __builtin_ctzll(m) : 64;
}

template <int D, bool PAGED>
__global__ void __launch_bounds__(64 * kTreeWaves) verify_tree(const VerifyArgs a) {
  using T = bf16;
  using RG = Ring<T, D>;
  constexpr int NW = kTreeWaves, NT = 64 * NW;
  constexpr int DB = D / 32, QN = D / 16;
  constexpr int LPW = RG::SEGS / NW;  // 1 KB copies per wave per stage
  static_assert(LPW * NW == RG::SEGS && LPW >= 1, "ring split over the waves");
  constexpr int QSF = D + (NT / D) * D;  // qbar scratch: the sum, then one partial per pair phase
  constexpr int LDS = RG::MAIN + RG::PT_CAP * 4 + QSF * 4;
  __shared__ __attribute__((aligned(1024))) char smem[LDS];
  int* pt_lds = reinterpret_cast<int*>(smem + RG::MAIN);
  float* qs = reinterpret_cast<float*>(smem + RG::MAIN + RG::PT_CAP * 4);
  // one field from each line of the argument block the prologue reads, so the
  // lines arrive in one trip instead of one after another (each first read
  // behind a branch or a division waited for its own)
  asm volatile("" ::"v"(a.B), "v"((uint32_t)(uintptr_t)a.q), "v"((uint32_t)(uintptr_t)a.ws_anc), "v"(a.do_scores));

  // ---- workgroup -> (sequence, KV head, chunk, row block); blockIdx % 8
  // picks the XCD, and the row blocks of a chunk, which read the same K/V,
  // share that XCD's L2.
  int rb, g, b, c;
  if (a.B <= 64) {
    // Batches of up to 64 sequences: every sequence's whole chunks first, then
    // the shorter last chunks.  The dispatcher starts workgroups in grid order,
    // so the short ones run last and fill the final round instead of leaving
    // CUs idle behind the last whole chunks.  Item j = (blockIdx / 8 / RB) * 8
    // + blockIdx % 8 runs on XCD j % 8, and the RB row blocks of one item share
    // that XCD's L2.
    const int s8 = (int)(blockIdx.x >> 3);
    rb = s8 % a.RB;
    const int j = s8 / a.RB * 8 + (int)(blockIdx.x & 7);
    const int ln = (int)(threadIdx.x & 63);
    int Lb = 0;
    if (ln < a.B) seq_prefix(a, ln, &Lb);
    const int nf = Lb / a.chunk;                         // whole chunks of sequence ln
    const int tl = Lb > nf * a.chunk ? 1 : 0;            // and a shorter last one
    const int fi = wave_incl_sum(nf * a.Hkv);
    const int F = __builtin_amdgcn_readlane(fi, 63);
    if (j < F) {
      b = first_lane_above(fi, j);
      const int r = j - (__builtin_amdgcn_readlane(fi, b) - __builtin_amdgcn_readlane(nf, b) * a.Hkv);
      c = r / a.Hkv;
      g = (r - c * a.Hkv + c) % a.Hkv;  // heads rotated by the chunk: each XCD sees every head
    } else {
      const int ti = wave_incl_sum(tl * a.Hkv);
      const int jt = j - F;
      if (jt >= __builtin_amdgcn_readlane(ti, 63)) return;
      b = first_lane_above(ti, jt);
      g = jt - (__builtin_amdgcn_readlane(ti, b) - __builtin_amdgcn_readlane(tl, b) * a.Hkv);
      c = __builtin_amdgcn_readlane(nf, b);
    }
  } else {
    // Larger batches: chunk c of (b, g) runs on XCD (c + b Hkv + g) % 8, so
    // every XCD gets a slice of every sequence and head, and the chunks past a
    // multiple of 8 start on a different XCD for each (sequence, head) (chunk c
    // on XCD c % 8 gave XCD 0 45% more work than XCD 7 on a batch of 16 mixed
    // lengths).
    int wk = (int)(blockIdx.x >> 3);
    rb = wk % a.RB;
    wk /= a.RB;
    g = wk % a.Hkv;
    wk /= a.Hkv;
    b = wk % a.B;
    c = wk / a.B * 8 + (((int)(blockIdx.x & 7) - b * a.Hkv - g) & 7);
    if (c >= a.n_chunks) return;
  }
  int L;
  const int Pb = seq_prefix(a, b, &L);
  // fixed-length chunks (a whole number of stages): a sequence shorter than the
  // longest has fewer chunks, and its chunks past the end do nothing (the merge
  // reads only chunks below P_b + N), so workgroups are of similar length
  const int c0 = c * a.chunk;
  if (c0 >= L) return;
  const int c1 = min(c0 + a.chunk, L);
  const int n_st = (c1 - c0 + RG::SK - 1) / RG::SK;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lane32 = lane & 31, h = lane >> 5;

  // ---- this wave's query tile (B operand of S^T = K Q^T): lane column = query row
  bf16x8 qf[QN];
  const int row = (rb * NW + wave) * 32 + lane32;
  const bool row_ok = row < a.R;
  const int t_node = row_ok ? row / a.G : a.N - 1;
  {
    const int j = row_ok ? row % a.G : 0;
    const T* qrow = reinterpret_cast<const T*>(a.q) + ((long long)(b * a.N + t_node) * a.Hq + g * a.G + j) * D;
#pragma unroll
    for (int ks = 0; ks < QN; ++ks) {
      bf16x8 x = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks + 8 * h);
      qf[ks] = row_ok ? x : bf16x8{};
    }
  }
  // ancestor bitset of this lane's node (tree, chunk reaching the verify
  // tokens), in flight together with the query tile and the loads below
  uint32_t anc[kAncWords] = {};
  const bool need_anc = a.tree && c1 > Pb;
  if (need_anc) {
#pragma unroll
    for (int w = 0; w < kAncWords; ++w) anc[w] = a.ws_anc[((long long)b * a.N + t_node) * kAncWords + w];
  }

  // ---- page-table slice of this chunk -> LDS
  const int ps = a.kv.page_size;
  int pg0 = 0;
  bool pt_fits = true;  // every page of the chunk is in the cached slice
  if constexpr (PAGED) {
    if (c1 > c0) {
      pg0 = a.ps_shift >= 0 ? (c0 >> a.ps_shift) : c0 / ps;
      const int pg1 = a.ps_shift >= 0 ? ((c1 - 1) >> a.ps_shift) : (c1 - 1) / ps;
      pt_fits = pg1 - pg0 < RG::PT_CAP;
      for (int j = tid; j <= pg1 - pg0 && j < RG::PT_CAP; j += NT) {
        const int pg = pg0 + j;
        pt_lds[j] = pg < a.kv.max_pages ? a.kv.page_table[(long long)b * a.kv.max_pages + pg] : -1;
      }
    }
    __syncthreads();
  }
  const long long seq_base = (long long)b * a.kv.seq_stride;
  // slot of a position: page entries from the cached slice (FROM_MEM: pages
  // past it are read from memory; the copy paths keep the two apart, so the
  // common one never waits on a memory read, which would also wait for every
  // copy already in flight)
  auto slot_of = [&](int pos, auto from_mem) -> long long {
    long long sl;
    if constexpr (PAGED) {
      const int pg = a.ps_shift >= 0 ? (pos >> a.ps_shift) : pos / ps;
      const int jp = pg - pg0;
      int e;
      if constexpr (decltype(from_mem)::value)
        e = jp < RG::PT_CAP ? pt_lds[jp]
                             : (pg < a.kv.max_pages ? a.kv.page_table[(long long)b * a.kv.max_pages + pg] : -1);
      else
        e = pt_lds[jp < RG::PT_CAP ? jp : 0];
      sl = e < 0 ? -1 : (long long)e * ps + (pos - pg * ps);
    } else {
      sl = seq_base + pos;
    }
    return (sl >= 0 && sl < a.kv.num_slots) ? sl : 0;  // unmapped positions read slot 0 (never visible)
  };

  // ---- copies of a stage: segment wave * LPW + j; the first SEGS / 2 segments are K rows, the rest V.
  // (The row blocks of a chunk read each tile too; copies without the
  // non-temporal hint, meant to keep the tiles in L2 for them, measured 4x
  // slower with 4x the HBM traffic on the 256-node tree.)
  const uint32_t ring_l =
      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)smem);
  const long long slot_bytes = (long long)a.Hkv * RG::ROWB;
  const bool wave_v = wave * LPW >= RG::SEGS / 2;
  const char* tg = reinterpret_cast<const char*>(wave_v ? a.kv.v : a.kv.k) + (long long)g * RG::ROWB;
  const int seg0 = (wave * LPW) % (RG::SEGS / 2);
  // lane's row of copy j and its swizzled 16-byte column (recomputed per copy: few registers)
  auto drow = [&](int j) { return (seg0 + j) * RG::RPS + lane / RG::CPR; };
  auto dcol = [&](int j) { return ((lane % RG::CPR) ^ swz<T, D>(drow(j))) * 16; };
  auto issue = [&](int i) {
    const int key0 = c0 + i * RG::SK;
    const uint32_t ld = ring_l + (uint32_t)((i % RG::NS) * RG::STAGE + (wave_v ? RG::TILE : 0) + seg0 * 1024);
    if (!PAGED && key0 + RG::SK <= c1 && seq_base + key0 + RG::SK <= a.kv.num_slots) {
      const char* bt = tg + (seq_base + key0) * slot_bytes;
#pragma unroll
      for (int j = 0; j < LPW; ++j) dma16_sbase(ld + j * 1024, (uint32_t)(drow(j) * slot_bytes) + dcol(j), bt);
    } else if (pt_fits) {
#pragma unroll
      for (int j = 0; j < LPW; ++j) {
        const int pos = key0 + drow(j);
        dma16_vaddr(ld + j * 1024, tg + slot_of(pos < c1 ? pos : c0, std::false_type{}) * slot_bytes + dcol(j));
      }
    } else {
#pragma unroll
      for (int j = 0; j < LPW; ++j) {
        const int pos = key0 + drow(j);
        dma16_vaddr(ld + j * 1024, tg + slot_of(pos < c1 ? pos : c0, std::true_type{}) * slot_bytes + dcol(j));
      }
    }
  };

  // ---- score operand: scale * qbar_g in fp32 (qs[0 .. D))
  const bool wg_scores = a.do_scores && c0 < Pb;
  if (wg_scores) {
    if (a.prep_qbar) {
      for (int d = tid; d < D; d += NT) {
        const float* part = a.ws_qbar + (long long)(b * a.Hkv + g) * a.qsplit * D + d;
        float acc = 0.f;
        for (int sp0 = 0; sp0 < a.qsplit; sp0 += 16) {
          // sixteen loads at clamped places issued together, then summed in order (a
          // bounded loop's load per step would be one trip to memory each)
          float x[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) x[u] = part[min(sp0 + u, a.qsplit - 1) * D];
#pragma unroll
          for (int u = 0; u < 16; ++u) acc += sp0 + u < a.qsplit ? x[u] : 0.f;
        }
        qs[d] = acc;
      }
    } else {
      constexpr int NP = NT / D;
      const int d = tid % D, part = tid / D;
      const int npairs = a.n_score_rows * a.G;
      float acc = 0.f;
      for (int i0 = part; i0 < npairs; i0 += 8 * NP) {
        // eight pairs at a time: their row indices, then their query elements, each
        // step's loads issued together at clamped places, then summed in order
        int t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) t[u] = a.score_rows[min(i0 + u * NP, npairs - 1) / a.G];
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int j = min(i0 + u * NP, npairs - 1) % a.G;
          x[u] = (float)reinterpret_cast<const T*>(a.q)[((long long)(b * a.N + t[u]) * a.Hq + g * a.G + j) * D + d];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += i0 + u * NP < npairs ? x[u] : 0.f;
      }
      qs[D + part * D + d] = acc;
      __syncthreads();
      if (tid < D) {
        float sacc = 0.f;
        for (int p = 0; p < NP; ++p) sacc += qs[D + p * D + tid];
        qs[tid] = sacc;
      }
    }
    if (tid < D) qs[tid] *= a.scale;  // the entry this thread wrote
    __syncthreads();
  }

  if (need_anc) {
    asm volatile("" ::"v"(anc[0]), "v"(anc[1]), "v"(anc[2]), "v"(anc[3]), "v"(anc[4]), "v"(anc[5]), "v"(anc[6]),
                 "v"(anc[7]));  // wait for the loads here (all in flight together), not inside the loop
  }
#pragma unroll
  for (int ks = 0; ks < QN; ++ks) asm volatile("" ::"v"(qf[ks]));  // the query tile has landed
  // Only now fill the ring: a load the compiler waits for, issued after the
  // copies, would wait for every copy too (the counter completes in order),
  // so the first stage would start only once the whole ring had landed
  // (256-node tree: step 70.8 -> 69.9 us with the copies issued last).
  for (int i = 0; i < RG::PD && i < n_st; ++i) issue(i);

  // ---- per-lane LDS offsets of the operand reads inside a 32-key block
  int koff[QN];
#pragma unroll
  for (int kr = 0; kr < QN; ++kr) koff[kr] = tile_off<T, D>(lane32, 2 * kr + h);
  const int e4 = (lane & 15) >> 2, cq = lane & 3, dh = (lane >> 4) & 1;
  int voff[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int hl = 0; hl < 2; ++hl)
      voff[db][hl] = tile_off<T, D>(4 * h + e4 + 8 * hl, 4 * db + 2 * dh + (cq >> 1)) + (cq & 1) * 8;

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m = kNegInf, l = 0.f;
  float* sdst = a.ws_s + ((long long)b * a.Hkv + g) * a.s_stride;

  // Stage i: wait for its copies, start the copies of stage i + PD, then the
  // two blocks' S^T products, one max and one rescale decision for the
  // stage's 64 keys, and both blocks' exponentials and P V products in one
  // branch-free stretch (so the second block's exponentials can issue while
  // the first block's P V products run on the matrix cores).  The stage's
  // scores come last, eight keys per wave, when this row block owns the
  // stage (K rows read again from the ring).  Stages
  // whose keys all lie in the prefix need no mask and run a copy of the body
  // without it; stages past the chunk end (the last one of a chunk) skip
  // their missing blocks.
  auto stage = [&](int i, auto masked, auto full) {
    constexpr bool MASKED = decltype(masked)::value;
    constexpr bool FULL = decltype(full)::value;
    // stage i has landed once only the copies of later stages can be outstanding
    const int after = min(RG::PD - 1, n_st - 1 - i);
    if (after >= 2) wait_vm_lgkm0<2 * LPW>();
    else if (after == 1) wait_vm_lgkm0<LPW>();
    else wait_vm_lgkm0<0>();
    barrier_only();
    // the buffer of stage i + PD was last read in iteration i - 1, which every wave has finished
    if (i + RG::PD < n_st) issue(i + RG::PD);
    const char* Kt = smem + (i % RG::NS) * RG::STAGE;
    const char* Vt = Kt + RG::TILE;
    const int kst = c0 + i * RG::SK;  // first key of the stage
    const int nb = FULL ? RG::NB : min(RG::NB, (c1 - kst + 31) / 32);

    f32x16 sb[RG::NB];
#pragma unroll
    for (int kb = 0; kb < RG::NB; ++kb) {
      if (!FULL && kb >= nb) break;
      const char* Kb = Kt + kb * 32 * RG::ROWB;
      bf16x8 ka[QN];
#pragma unroll
      for (int ks = 0; ks < QN; ++ks) ka[ks] = *reinterpret_cast<const bf16x8*>(Kb + koff[ks]);
      f32x16 s = f32x16{};
#pragma unroll
      for (int ks = 0; ks < QN; ++ks) s = mfma_bf16(ka[ks], qf[ks], s);
      sb[kb] = s;
    }

    // mask (blocks reaching the verify tokens): visible iff j < P_b or j - P_b is
    // an ancestor-or-self; then the stage max
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < RG::NB; ++kb) {
      if (!FULL && kb >= nb) break;
      const int kb0 = kst + 32 * kb;
      f32x16& s = sb[kb];
      if (MASKED && kb0 + 32 > Pb) {
        if (a.tree) {
          const uint32_t win = anc_window(anc, kb0 - Pb);
#pragma unroll
          for (int v = 0; v < 16; ++v) s[v] = win_vis(win, v, h) ? s[v] : kNegInf;
        } else {
#pragma unroll
          for (int v = 0; v < 16; ++v) s[v] = (kb0 + kappa(v, h) - Pb <= t_node) ? s[v] : kNegInf;
        }
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[v]);
    }
    // online softmax, log2 domain, lazy rescale (one decision per stage)
    mx = half_max(mx) * a.scale_log2;
    const bool grew = mx > m + kRescaleSlack;
    if (__any(grew)) {
      const float mn = grew ? mx : m;
      const float alpha = grew ? fast_exp2(m - mn) : 1.f;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      m = mn;
    }
    const float mneg = m == kNegInf ? 0.f : -m;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < RG::NB; ++kb) {
      if (!FULL && kb >= nb) break;
      f32x16& s = sb[kb];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = fast_exp2(__builtin_fmaf(s[v], a.scale_log2, mneg));
        s[v] = p;
        psum += p;
      }
      // O^T += V^T P^T
      const char* Vb = Vt + kb * 32 * RG::ROWB;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        bf16x8 pb;
#pragma unroll
        for (int u = 0; u < 8; ++u) pb[u] = (bf16)s[8 * jj + u];
        const char* Vj = Vb + jj * 16 * RG::ROWB;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x4 lo = lds_read_tr16(reinterpret_cast<const T*>(Vj + voff[db][0]));
          const bf16x4 hi = lds_read_tr16(reinterpret_cast<const T*>(Vj + voff[db][1]));
          const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          o[db] = mfma_bf16(va, pb, o[db]);
        }
      }
    }
    l += psum;

    // scores of the stage's prefix keys, by one row block per stage (stage s by
    // row block s mod RB) and spread over all its waves, so no wave waits for
    // another at the next barrier: wave w takes keys 8w .. 8w + 7 of the
    // stage, each key's CPR lanes dot 8 of its dimensions with scale * qbar in
    // fp32, the row shifts sum the CPR products, and the key's last lane writes
    // the score (keys past P_b land in the row's padding and are never read)
    if (wg_scores && (kst / RG::SK) % a.RB == rb) {
      constexpr int CPR = D / 8, KPR = 64 / CPR;  // lanes per key, keys per 16-byte read
      static_assert(NW * 8 == RG::SK && KPR <= 8 && 8 % KPR == 0, "eight keys per wave");
      const int kw = kst + 8 * wave;
      if (kw < Pb && kw < c1) {
        const int cc = lane % CPR;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(qs + 8 * cc);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(qs + 8 * cc + 4);
        float acc[8 / KPR];
#pragma unroll
        for (int j = 0; j < 8 / KPR; ++j) {
          const bf16x8 kv = *reinterpret_cast<const bf16x8*>(Kt + tile_off<T, D>(8 * wave + KPR * j + lane / CPR, cc));
          float d = (float)kv[0] * x0[0];
          d = __builtin_fmaf((float)kv[1], x0[1], d);
          d = __builtin_fmaf((float)kv[2], x0[2], d);
          d = __builtin_fmaf((float)kv[3], x0[3], d);
          d = __builtin_fmaf((float)kv[4], x1[0], d);
          d = __builtin_fmaf((float)kv[5], x1[1], d);
          d = __builtin_fmaf((float)kv[6], x1[2], d);
          acc[j] = __builtin_fmaf((float)kv[7], x1[3], d);
        }
#pragma unroll
        for (int j = 0; j < 8 / KPR; ++j) {
          float v = acc[j];  // inclusive sums over the row of 16 lanes, 1 + 2 + 4 (+ 8)
          v += dpp_f<0x111, 0xf>(0.f, v);
          v += dpp_f<0x112, 0xf>(0.f, v);
          v += dpp_f<0x114, 0xf>(0.f, v);
          if constexpr (CPR == 16) v += dpp_f<0x118, 0xf>(0.f, v);
          if (cc == CPR - 1) sdst[kw + KPR * j + lane / CPR] = v;
        }
      }
    }
  };
  // stages entirely inside the prefix need no mask; only the last stage of a
  // chunk can reach past its end
  const int n_full = (c1 - c0) / RG::SK;
  const int n_plain = min(max((Pb - c0) / RG::SK, 0), n_full);
  for (int i = 0; i < n_plain; ++i) stage(i, std::false_type{}, std::true_type{});
  for (int i = n_plain; i < n_full; ++i) stage(i, std::true_type{}, std::true_type{});
  if (n_full < n_st) stage(n_full, std::true_type{}, std::false_type{});

  // ---- epilogue: this wave's rows are its own -> (m, l, o) partials straight to
  // the workspace (no copy is in flight; the score stores need no wait)
  const float lt = half_sum(l);
  if (row_ok) {
    const long long rec = ((long long)(b * a.Hkv + g) * a.Rpad + row) * a.n_chunks + c;
    // o partials in bf16 (relative rounding 2^-9, far inside the output
    // tolerance): the merge then reads half the bytes
    bf16* dst = reinterpret_cast<bf16*>(a.ws_o) + rec * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        *reinterpret_cast<bf16x4*>(dst + 32 * db + 8 * qd + 4 * h) =
            bf16x4{(bf16)o[db][4 * qd], (bf16)o[db][4 * qd + 1], (bf16)o[db][4 * qd + 2], (bf16)o[db][4 * qd + 3]};
    if (h == 0) a.ws_ml[rec] = f32x2{m, lt};
  }
}

// Split-KV merge (log-sum-exp weights) + per-KV-head score sum.  wpr waves
// (1 or 4) per (sequence, KV head, query row), 4 / wpr rows per workgroup.
// The two halves of each of the row's waves take every (2 wpr)-th chunk
// (lane q of a half holds columns 4q..4q+3) and merge them in one pass, eight
// chunks' (m, l, o) loads in flight per lane: each batch's max rescales the
// running sums once.  Halves, then waves (through LDS), are combined in a
// fixed order with their own log-sum-exp weights, so results do not depend
// on timing.  Four waves per row when rows have many chunks (few, long
// rows), one otherwise.  Workgroups past the row ones sum the per-head score
// partials of 256 prefix entries each.
constexpr int kMaxChunks = 1024;

// (m, l, o) partial of a merge lane; merging two is log-sum-exp weighting
struct MergeAcc {
  float m, l;
  f32x4 o;
};
__device__ __forceinline__ MergeAcc merge_acc(const MergeAcc& x, const MergeAcc& y) {
  const float M = fmaxf(x.m, y.m);
  const float wx = x.m == kNegInf ? 0.f : fast_exp2(x.m - M);
  const float wy = y.m == kNegInf ? 0.f : fast_exp2(y.m - M);
  return MergeAcc{M, wx * x.l + wy * y.l, wx * x.o + wy * y.o};
}

// Fused selection, pass A on the merge's score workgroups (NT threads, one
// per (sequence, block of sel_blk(P, k) prefix entries)): the block's scores are
// summed from the per-KV-head partials (head order, as every score) and
// written, then pass A runs on them (band from a sample of summed scores, the
// block's entries at or above it to the selection workspace).  Pass B is the
// next kernel.  Thread t sums the E entries base + E t + e and, for t < 256,
// the SEG sample entries of segment t, each a 16-byte load per KV head: a
// sample of 1024 entries (2048 for rows above 65536), half what a selection
// over rows in memory takes, since every workgroup of the row sums it from
// the partials of all KV heads.
template <int NT, int E, int SEG>
__device__ __forceinline__ void merge_select_block(SelShared& L, const VerifyArgs& a, int b, int blk, int P, int k) {
  static_assert(E % 2 == 0 && SEG % 4 == 0, "8- or 16-byte pieces");
  constexpr int PC = E % 4 == 0 ? 4 : 2;  // floats per block piece
  const int tid = threadIdx.x;
  const int base = blk * E * NT;
  const float* part = a.ws_s + (long long)b * a.Hkv * a.s_stride;  // rows of s_stride (a multiple of 4)
  constexpr int NSEG = 256;  // sample segments
  const bool samp = sel_multi(P, k);
  const bool seg_t = samp && tid < NSEG;
  const int p0 = seg_t ? sel_seg_start(tid, P, SEG, NSEG) : 0;
  float x[E], smp[SEG];
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = 0.f;
#pragma unroll
  for (int e = 0; e < SEG; ++e) smp[e] = 0.f;
  // every load of a group of KV heads before its sums (in head order, as
  // every score is formed); a piece starting below P_b ends inside the row
  // (rows hold P_max + 32 entries, rounded up to whole pieces).  Groups hold at
  // most 64 values in flight per thread (8 heads, or 4 for 8-entry pieces), so
  // the kernel's row merges keep their occupancy.
  constexpr int HG = (E + SEG) * 8 > 64 ? 4 : 8;
  for (int g0 = 0; g0 < a.Hkv; g0 += HG) {
    float xv[HG][E];
    f32x4 sv[HG][SEG / 4];
#pragma unroll
    for (int j = 0; j < HG; ++j) {
      const bool live = g0 + j < a.Hkv;
      const float* pg = part + (long long)(live ? g0 + j : 0) * a.s_stride;
#pragma unroll
      for (int q = 0; q < E / PC; ++q) {
        const int i = base + E * tid + PC * q;
        if constexpr (PC == 4) {
          const f32x4 v = live && i < P ? *reinterpret_cast<const f32x4*>(pg + i) : f32x4{};
#pragma unroll
          for (int e = 0; e < 4; ++e) xv[j][4 * q + e] = v[e];
        } else {
          const f32x2 v = live && i < P ? *reinterpret_cast<const f32x2*>(pg + i) : f32x2{};
          xv[j][2 * q] = v[0];
          xv[j][2 * q + 1] = v[1];
        }
      }
#pragma unroll
      for (int q = 0; q < SEG / 4; ++q)
        sv[j][q] = live && seg_t ? *reinterpret_cast<const f32x4*>(pg + p0 + 4 * q) : f32x4{};
    }
#pragma unroll
    for (int j = 0; j < HG; ++j) {
      if (g0 + j < a.Hkv) {
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] += xv[j][e];
#pragma unroll
        for (int q = 0; q < SEG / 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) smp[4 * q + e] += sv[j][q][e];
      }
    }
  }
  float* srow = a.scores + (long long)b * a.P_max;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = base + E * tid + e;
    if (i < P) srow[i] = x[e];
    else x[e] = __builtin_nanf("");
  }
  if (!samp) return;
  if (!seg_t)
#pragma unroll
    for (int e = 0; e < SEG; ++e) smp[e] = __builtin_nanf("");
  float t_lo, t_hi;
  sel_band<NT>(L, smp, NSEG * SEG, P, k, &t_lo, &t_hi);
  if (blk == 0 && tid == 0) a.selws.band[b] = SelBand{t_lo, t_hi, {0, 0}};
  sel_compact<NT, E>(L, a.selws, b, blk, x, base, t_lo, t_hi, [](uint32_t* p, uint32_t v) { *p = v; });
}

template <typename T, int D, bool OB, bool SEL>
__global__ void __launch_bounds__(SEL ? 512 : 256) verify_merge(const VerifyArgs a, int n_score_wgs, int wpr) {
  constexpr int NT = SEL ? 512 : 256;
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  // the score workgroups come first: they start with the row merges instead
  // of after all of them (as a tail, on batches with many rows)
  if ((int)blockIdx.x >= n_score_wgs) {
    __shared__ MergeAcc red[NW][32];
    const int lane = tid & 63, wave = tid >> 6;
    const int sub = wave % wpr;
    const int gr = ((int)blockIdx.x - n_score_wgs) * (NW / wpr) + wave / wpr;  // (b, g, row); uniform over a row's waves
    if (gr >= a.B * a.Hkv * a.R) return;
    const int row = gr % a.R, bg = gr / a.R, g = bg % a.Hkv, b = bg / a.Hkv;
    // every chunk holds a partial (streaming kernel), else the chunks below P_b + N;
    // the branch keeps the sequence-length load off the first path
    int nc = a.n_chunks;
    if (!a.all_chunks) {
      int L;
      seq_prefix(a, b, &L);
      nc = min((L + a.chunk - 1) / a.chunk, a.n_chunks);
    }
    const long long rec0 = ((long long)(b * a.Hkv + g) * a.Rpad + row) * a.n_chunks;
    static_assert(D / 4 <= 32, "one float4 column group per lane of a half");
    const int half = lane >> 5, q = lane & 31;
    const int qc = q < D / 4 ? q : 0;  // lanes past the row width repeat column group 0 (not stored)
    MergeAcc acc{kNegInf, 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
    constexpr int BATCH = 8;
    for (int c0 = 2 * sub + half; c0 < nc; c0 += 2 * wpr * BATCH) {
      f32x2 ml[BATCH];
      f32x4 ov[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int c = c0 + 2 * wpr * u;
        const bool ok = c < nc;
        ml[u] = ok ? a.ws_ml[rec0 + c] : f32x2{kNegInf, 0.f};
        if constexpr (OB) {
          const bf16x4 x = ok ? *reinterpret_cast<const bf16x4*>(reinterpret_cast<const bf16*>(a.ws_o) +
                                                                  (rec0 + c) * D + 4 * qc)
                              : bf16x4{};
          ov[u] = f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
        } else {
          ov[u] = ok ? *reinterpret_cast<const f32x4*>(a.ws_o + (rec0 + c) * D + 4 * qc) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      float bm = acc.m;
#pragma unroll
      for (int u = 0; u < BATCH; ++u) bm = fmaxf(bm, ml[u][0]);
      const float wa = acc.m == kNegInf ? 0.f : fast_exp2(acc.m - bm);
      acc.l *= wa;
      acc.o *= wa;
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const float w = ml[u][0] == kNegInf ? 0.f : fast_exp2(ml[u][0] - bm);
        acc.l += w * ml[u][1];
        acc.o += w * ov[u];
      }
      acc.m = bm;
    }
    // halves: lane q of half 1 joins lane q of half 0 (same columns, other chunks)
    {
      MergeAcc oth;
      oth.m = __shfl_xor(acc.m, 32);
      oth.l = __shfl_xor(acc.l, 32);
#pragma unroll
      for (int e = 0; e < 4; ++e) oth.o[e] = __shfl_xor(acc.o[e], 32);
      acc = half == 0 ? merge_acc(acc, oth) : merge_acc(oth, acc);
    }
    if (wpr > 1) {  // the row's waves share one workgroup: merge their results in wave order
      if (half == 0) red[wave][q] = acc;
      __syncthreads();
      if (sub == 0) {
        acc = red[wave][q];
        for (int w = 1; w < wpr; ++w) acc = merge_acc(acc, red[wave + w][q]);
      }
    }
    if (sub == 0 && half == 0 && q < D / 4) {
      const float inv = acc.l > 0.f ? 1.f / acc.l : 0.f;
      const int tn = row / a.G, j = row % a.G;
      T* dst = reinterpret_cast<T*>(a.out) + ((long long)(b * a.N + tn) * a.Hq + g * a.G + j) * D + 4 * q;
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = (T)(acc.o[e] * inv);
    }
  } else if constexpr (SEL) {
    __shared__ SelShared L;
    const int sw = (int)blockIdx.x;
    const int b = sw / kSelMaxBlocks, blk = sw % kSelMaxBlocks;
    if (b >= a.B) return;
    int P, k;
    sel_row_sizes(a.prefix_len, a.sel_k, b, a.P_max, a.sel_kmax, &P, &k);
    if (blk * sel_blk(P, k) >= P) return;
    if (sel_blk(P, k) == 4096) merge_select_block<NT, 4096 / NT, 8>(L, a, b, blk, P, k);
    else if (sel_blk(P, k) == 2048) merge_select_block<NT, 2048 / NT, 4>(L, a, b, blk, P, k);
    else merge_select_block<NT, 1024 / NT, 4>(L, a, b, blk, P, k);
  } else {
    const long long i0 = (long long)blockIdx.x * 256 + tid;
    if (i0 >= (long long)a.B * a.P_max) return;
    const int b = (int)(i0 / a.P_max), i = (int)(i0 % a.P_max);
    int Pb = a.prefix_len[b];
    Pb = Pb < 0 ? 0 : (Pb > a.P_max ? a.P_max : Pb);
    if (i >= Pb) return;
    // the KV heads' partials eight at a time, loaded together at clamped places
    // (a load per step of a bounded loop would be one trip to memory each)
    if (a.head_scores) {  // each KV head's own sum over its query heads and the scoring rows
      for (int g0 = 0; g0 < a.Hkv; g0 += 8) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = a.ws_s[((long long)b * a.Hkv + min(g0 + u, a.Hkv - 1)) * a.s_stride + i];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (g0 + u < a.Hkv) a.scores[((long long)b * a.Hkv + g0 + u) * a.P_max + i] = x[u];
      }
      return;
    }
    float s = 0.f;  // summed in head order
    for (int g0 = 0; g0 < a.Hkv; g0 += 8) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = a.ws_s[((long long)b * a.Hkv + min(g0 + u, a.Hkv - 1)) * a.s_stride + i];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += g0 + u < a.Hkv ? x[u] : 0.f;
    }
    a.scores[i0] = s;
  }
}

// Per-sequence precomputation: qbar_g (fp32 sum of the scoring rows' queries of
// each KV head) and ancestor-or-self bitsets of the draft tree by pointer jumping.
template <typename T, int D>
__global__ void __launch_bounds__(256) verify_prep(const VerifyArgs a, int n_qbar_wgs) {
  const int tid = threadIdx.x;
  __shared__ float part[256];
  __shared__ __attribute__((aligned(16))) uint32_t ancs[kMaxNodes][kAncWords];
  __shared__ int jmp[kMaxNodes];
  // one field from each line of the argument block either path reads first,
  // so the lines arrive in one trip instead of one after another
  asm volatile("" ::"v"(n_qbar_wgs), "v"(a.N), "v"((uint32_t)(uintptr_t)a.q), "v"((uint32_t)(uintptr_t)a.ws_anc),
               "v"(a.qsplit));
  if ((int)blockIdx.x < n_qbar_wgs) {
    // partial qbar of (b, g) over pairs [sp * kQbarPairs, (sp + 1) * kQbarPairs):
    // D columns x (256 / D) pair phases; every load of the thread is issued
    // before the first is used (one trip to memory)
    const int sp = blockIdx.x % a.qsplit, bg = blockIdx.x / a.qsplit;
    const int g = bg % a.Hkv, b = bg / a.Hkv;
    constexpr int NP = 256 / D;
    constexpr int PT = kQbarPairs / NP;  // pairs per thread
    static_assert(D % 64 == 0, "a pair phase is a whole number of waves");
    // the pair phase is wave-uniform: score_rows is then read with scalar loads
    const int d = tid % D, p = __builtin_amdgcn_readfirstlane(tid / D);
    const int npairs = a.n_score_rows * a.G;
    const int i_end = min(npairs, (sp + 1) * kQbarPairs);
    // pair indices clamped into range so every load is unconditional (no
    // branch between a row index and its load); pairs past the range add 0
    int off[PT];
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int i = min(sp * kQbarPairs + p + NP * u, npairs - 1);
      const int t = a.score_rows[i / a.G], j = i % a.G;
      off[u] = ((b * a.N + t) * a.Hq + g * a.G + j) * D;
    }
    T x[PT];
#pragma unroll
    for (int u = 0; u < PT; ++u) x[u] = reinterpret_cast<const T*>(a.q)[(long long)off[u] + d];
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < PT; ++u) acc += sp * kQbarPairs + p + NP * u < i_end ? (float)x[u] : 0.f;
    part[tid] = acc;
    __syncthreads();
    if (tid < D) {
      float sum = 0.f;
      for (int k = 0; k < NP; ++k) sum += part[k * D + tid];
      a.ws_qbar[((long long)bg * a.qsplit + sp) * D + tid] = sum;
    }
    return;
  }
  // ancestor-or-self sets by pointer doubling: thread t owns node t (N <= 256),
  // holding its set and jump in registers; each round publishes them to LDS
  // and ORs in the set of the node it jumps to, whose jump it then takes
  static_assert(kMaxNodes <= 256 && kAncWords == 8, "one node per thread, two 16-byte words per set");
  const int b = blockIdx.x - n_qbar_wgs;
  const int N = a.N;
  const int t = tid;
  const bool act = t < N;
  int jp = act ? a.parent[(long long)b * N + t] : -1;
  if (jp < 0 || jp >= t) jp = -1;  // malformed parents are treated as roots
  uint32_t anc[kAncWords];
#pragma unroll
  for (int w = 0; w < kAncWords; ++w) {
    uint32_t x = (act && w == (t >> 5)) ? (1u << (t & 31)) : 0u;
    if (jp >= 0 && w == (jp >> 5)) x |= 1u << (jp & 31);
    anc[w] = x;
  }
  for (int round = 0; round < 9; ++round) {
    if (!__syncthreads_or(jp >= 0)) break;  // also: every read of the previous round is done
    if (act) {
      *reinterpret_cast<uint4*>(&ancs[t][0]) = uint4{anc[0], anc[1], anc[2], anc[3]};
      *reinterpret_cast<uint4*>(&ancs[t][4]) = uint4{anc[4], anc[5], anc[6], anc[7]};
      jmp[t] = jp;
    }
    __syncthreads();
    if (jp >= 0) {
      const uint4 lo = *reinterpret_cast<const uint4*>(&ancs[jp][0]);
      const uint4 hi = *reinterpret_cast<const uint4*>(&ancs[jp][4]);
      jp = jmp[jp];
      anc[0] |= lo.x; anc[1] |= lo.y; anc[2] |= lo.z; anc[3] |= lo.w;
      anc[4] |= hi.x; anc[5] |= hi.y; anc[6] |= hi.z; anc[7] |= hi.w;
    }
  }
  if (act) {
    uint4* dst = reinterpret_cast<uint4*>(a.ws_anc + ((long long)b * N + t) * kAncWords);
    dst[0] = uint4{anc[0], anc[1], anc[2], anc[3]};
    dst[1] = uint4{anc[4], anc[5], anc[6], anc[7]};
  }
}

// ------------------------------------------------------------------------- host side

size_t select_workspace_bytes(int B) { return sel_ws_bytes(B); }
int launch_select_pass_b(const float* scores, int B, int P_max, const int32_t* prefix_len, const int32_t* k,
                         int k_max, int32_t* idx, int32_t* count, const SelWs& w, hipStream_t st);

VerifyPlan plan_verify(int B, int N, int Hq, int Hkv, int D, int P_max, int dtype, bool tree,
                       int n_score_rows, int page_size) {
  VerifyPlan p{};
  p.B = B; p.N = N; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv; p.D = D; p.P_max = P_max; p.dtype = dtype;
  p.R = N * p.G;
  const int es = dtype == SV_BF16 ? 2 : 4;
  const long long Lmax = (long long)P_max + N;
  p.tree = tree;
  p.scores = n_score_rows > 0;
  p.prep_qbar = p.scores && (long long)n_score_rows * p.G > kInlineQbarRows;
  p.qsplit = p.prep_qbar ? (n_score_rows * p.G + kQbarPairs - 1) / kQbarPairs : 0;
  p.prep = p.prep_qbar || tree;
  p.stream = dtype == SV_BF16 && p.R <= 64;
  p.treek = dtype == SV_BF16 && p.R > 64;
  if (p.stream) {
    // streaming kernel: waves split the keys of one (sequence, KV head) chunk
    p.RT = p.R <= 32 ? 1 : 2;
    p.WR = 1;
    p.WK = 4;
    p.rows_per_block = p.RT * 32;
    p.RB = 1;
    p.Rpad = p.rows_per_block;
    p.TK = 32;
    const long long units = (long long)B * Hkv;
    const long long nbk = (Lmax + 31) / 32;
    long long want = (256 + units / 2) / units;
    if (want < 1) want = 1;
    if (want > (nbk + 3) / 4) want = (nbk + 3) / 4;  // at least one block per wave on average
    if (page_size > 0) {  // a chunk's page-table slice should fit the LDS copy (PT_CAP entries; pages past it are read from memory)
      const long long cap_blocks = ((long long)(WaveRing<128>::PT_CAP - 2) * page_size) / 32 - 1;
      const long long need = (nbk + cap_blocks - 1) / (cap_blocks > 0 ? cap_blocks : 1);
      if (want < need) want = need;
    }
    if (want > kMaxChunks) want = kMaxChunks;
    if (want < 1) want = 1;
    p.n_chunks = (int)want;
    p.chunk = (int)(((nbk + want - 1) / want + 1) * 32);  // longest chunk, in keys
    // batches put chunk c on XCD c % 8; one sequence keeps whole heads on an XCD
    p.n_wg = B > 1 ? (int)(units * 8 * ((p.n_chunks + 7) / 8)) : (int)((units * p.n_chunks + 7) / 8 * 8);
  }
  const int rtiles = (p.R + 31) / 32;
  if (p.treek) {
    // tree kernel: kTreeWaves waves, one 32-row tile each
    p.RT = 1;
    p.WR = kTreeWaves;
    p.WK = 1;
    p.rows_per_block = 32 * kTreeWaves;
    p.RB = (p.R + p.rows_per_block - 1) / p.rows_per_block;
    p.Rpad = p.RB * p.rows_per_block;
  } else if (!p.stream) {
    if (rtiles <= 1) { p.RT = 1; p.WR = 1; }
    else if (rtiles <= 2) { p.RT = 2; p.WR = 1; }
    else if (rtiles <= 4) { p.RT = 2; p.WR = 2; }
    else { p.RT = 2; p.WR = 4; }
    p.WK = 4 / p.WR;
    p.rows_per_block = p.RT * p.WR * 32;
    p.RB = (p.R + p.rows_per_block - 1) / p.rows_per_block;
    p.Rpad = p.RB * p.rows_per_block;
  }
  const int SK = D * es > 256 ? 32 : 64;  // keys per ring stage (Ring<T, D>::SK)
  p.TK = SK;
  // one resident workgroup per CU (two for the smaller bf16, D = 64 ring)
  const int occ = (dtype == SV_BF16 && D == 64) ? 2 : 1;
  const long long units = (long long)B * Hkv * p.RB;
  if (!p.stream) {
    // chunks of whole stages, balanced over the longest sequence; about one
    // wave of workgroups over the 256 CUs (occ per CU)
    const long long nst = (Lmax + SK - 1) / SK;
    long long nc = (256LL * occ + units / 2) / units;
    // chunks of at most 4096 keys (2048 for the tree kernel, whose chunks have a fixed
    // length): the longest workgroups bound the tail of mixed-length batches
    const long long max_st = (p.treek ? 2048 : 4096) / SK;
    if (nc < (nst + max_st - 1) / max_st) nc = (nst + max_st - 1) / max_st;
    if (nc > nst) nc = nst;
    if (nc < 1) nc = 1;
    if (page_size > 0) {  // a chunk's page-table slice should fit the LDS copy (Ring::PT_CAP entries; pages past it are read from memory)
      const long long cap_st = (long long)(Ring<float, 64>::PT_CAP - 2) * page_size / SK - 1;
      const long long need = (nst + (cap_st > 0 ? cap_st : 1) - 1) / (cap_st > 0 ? cap_st : 1);
      if (nc < need) nc = need;
    }
    if (nc > kMaxChunks) nc = kMaxChunks;
    p.n_chunks = (int)nc;
    p.chunk = (int)(((nst + nc - 1) / nc) * SK);  // longest chunk, in keys
    // the tree kernel puts chunk c on XCD c % 8; verify_main keeps neighbouring chunks together
    p.n_wg = p.treek ? (int)(units * 8 * ((p.n_chunks + 7) / 8)) : (int)((units * p.n_chunks + 7) / 8 * 8);
  }
  size_t off = 0;
  p.off_o = off; off = align_up(off + (size_t)B * Hkv * p.Rpad * p.n_chunks * D * 4);
  p.off_ml = off; off = align_up(off + (size_t)B * Hkv * p.Rpad * p.n_chunks * 8);
  p.off_s = off; off = align_up(off + (p.scores ? (size_t)B * Hkv * (((size_t)P_max + 32 + 3) / 4 * 4) * 4 : 0));
  p.off_qbar = off; off = align_up(off + (p.prep_qbar ? (size_t)B * Hkv * p.qsplit * D * 4 : 0));
  p.off_anc = off; off = align_up(off + (tree ? (size_t)B * N * kAncWords * 4 : 0));
  p.bytes = off;
  return p;
}

template <typename T, int D, int RT, int WR, bool PAGED>
static void launch_main2(const VerifyPlan& p, const VerifyArgs& a, hipStream_t st, void* ev0, void* ev1) {
  if (ev0 && ev1)  // timestamps taken by the dispatch itself: no extra marker packets in the stream
    hipExtLaunchKernelGGL((verify_main<T, D, RT, WR, PAGED>), dim3(p.n_wg), dim3(256), 0, st, (hipEvent_t)ev0,
                          (hipEvent_t)ev1, 0, a);
  else
    hipLaunchKernelGGL((verify_main<T, D, RT, WR, PAGED>), dim3(p.n_wg), dim3(256), 0, st, a);
}
template <typename T, int D, int RT, int WR>
static void launch_main(const VerifyPlan& p, const VerifyArgs& a, hipStream_t st, void* ev0, void* ev1) {
  if (a.kv.page_table) launch_main2<T, D, RT, WR, true>(p, a, st, ev0, ev1);
  else launch_main2<T, D, RT, WR, false>(p, a, st, ev0, ev1);
}

template <int D, int RT, bool PAGED>
static void launch_stream2(const VerifyPlan& p, const VerifyArgs& a, hipStream_t st, void* ev0, void* ev1) {
  if (ev0 && ev1)
    hipExtLaunchKernelGGL((verify_stream<D, RT, PAGED>), dim3(p.n_wg), dim3(256), 0, st, (hipEvent_t)ev0,
                          (hipEvent_t)ev1, 0, a);
  else
    hipLaunchKernelGGL((verify_stream<D, RT, PAGED>), dim3(p.n_wg), dim3(256), 0, st, a);
}
template <int D, int RT>
static void launch_stream(const VerifyPlan& p, const VerifyArgs& a, hipStream_t st, void* ev0, void* ev1) {
  if (a.kv.page_table) launch_stream2<D, RT, true>(p, a, st, ev0, ev1);
  else launch_stream2<D, RT, false>(p, a, st, ev0, ev1);
}

template <int D, bool PAGED>
static void launch_tree2(const VerifyPlan& p, const VerifyArgs& a, hipStream_t st, void* ev0, void* ev1) {
  if (ev0 && ev1)
    hipExtLaunchKernelGGL((verify_tree<D, PAGED>), dim3(p.n_wg), dim3(64 * kTreeWaves), 0, st, (hipEvent_t)ev0,
                          (hipEvent_t)ev1, 0, a);
  else
    hipLaunchKernelGGL((verify_tree<D, PAGED>), dim3(p.n_wg), dim3(64 * kTreeWaves), 0, st, a);
}
template <int D>
static void launch_tree(const VerifyPlan& p, const VerifyArgs& a, hipStream_t st, void* ev0, void* ev1) {
  if (a.kv.page_table) launch_tree2<D, true>(p, a, st, ev0, ev1);
  else launch_tree2<D, false>(p, a, st, ev0, ev1);
}

template <typename T, int D>
static int launch_typed(const VerifyPlan& p, VerifyArgs& a, hipStream_t st, void* ev0, void* ev1) {
  if (p.prep) {
    const int nq = p.prep_qbar ? p.B * p.Hkv * p.qsplit : 0;
    const int nt = p.tree ? p.B : 0;
    hipLaunchKernelGGL((verify_prep<T, D>), dim3(nq + nt), dim3(256), 0, st, a, nq);
  }
  if constexpr (std::is_same<T, bf16>::value) {
    if (p.stream) {
      if (p.RT == 1) launch_stream<D, 1>(p, a, st, ev0, ev1);
      else launch_stream<D, 2>(p, a, st, ev0, ev1);
    } else if (p.treek) {
      launch_tree<D>(p, a, st, ev0, ev1);
    }
  }
  if (p.stream || p.treek) {
  } else if (p.RT == 1 && p.WR == 1) launch_main<T, D, 1, 1>(p, a, st, ev0, ev1);
  else if (p.RT == 2 && p.WR == 1) launch_main<T, D, 2, 1>(p, a, st, ev0, ev1);
  else if (p.RT == 2 && p.WR == 2) launch_main<T, D, 2, 2>(p, a, st, ev0, ev1);
  else launch_main<T, D, 2, 4>(p, a, st, ev0, ev1);
  // waves per merged row: four when rows are few and long (one sequence's
  // rows would not fill the GPU otherwise), one when there are many rows
  const int wpr = (p.n_chunks >= 16 && (long long)p.B * p.Hkv * p.R < 2048) ? 4 : 1;
  const bool ob = p.treek || p.stream;        // the bf16 kernels write their o partials in bf16
  if (a.sel_k) {
    // fused selection: 512-thread workgroups, one per (sequence, selection block)
    // (pass A) before the row ones, then the selection's pass B kernel
    const int n_row_wgs = (p.B * p.Hkv * p.R * wpr + 7) / 8;
    const int n_sel = p.B * kSelMaxBlocks;
    const dim3 grid(n_row_wgs + n_sel);
    if (ob) hipLaunchKernelGGL((verify_merge<T, D, true, true>), grid, dim3(512), 0, st, a, n_sel, wpr);
    else hipLaunchKernelGGL((verify_merge<T, D, false, true>), grid, dim3(512), 0, st, a, n_sel, wpr);
    const int e = (int)hipGetLastError();
    if (e) return e;
    return launch_select_pass_b(a.scores, p.B, p.P_max, a.prefix_len, a.sel_k, a.sel_kmax, a.sel_idx, a.sel_count,
                                a.selws, st);
  }
  const int n_row_wgs = (p.B * p.Hkv * p.R * wpr + 3) / 4;
  const long long n_s = p.scores ? ((long long)p.B * p.P_max + 255) / 256 : 0;
  if (ob)
    hipLaunchKernelGGL((verify_merge<T, D, true, false>), dim3(n_row_wgs + (int)n_s), dim3(256), 0, st, a, (int)n_s,
                       wpr);
  else
    hipLaunchKernelGGL((verify_merge<T, D, false, false>), dim3(n_row_wgs + (int)n_s), dim3(256), 0, st, a, (int)n_s,
                       wpr);
  return (int)hipGetLastError();
}

int launch_verify(const VerifyPlan& p, const void* q, const KvArgs& kv, const int32_t* prefix_len,
                  const int32_t* parent, const int32_t* score_rows, int n_score_rows, float scale,
                  void* out, float* scores, void* ws, void* stream, void* ev_start, void* ev_stop,
                  int len_bias, int head_scores, const SelectArgs* sel) {
  VerifyArgs a{};
  if (sel) {
    a.sel_k = sel->k;
    a.sel_kmax = sel->k_max;
    a.sel_idx = sel->idx;
    a.sel_count = sel->count;
    a.selws = sel_ws_at(sel->ws, p.B);
  }
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
  a.s_stride = (p.P_max + 32 + 3) / 4 * 4;  // whole 32-key blocks past P_max; rows 16-byte aligned
  a.n_units = p.B * p.Hkv * p.RB * p.n_chunks;
  a.all_chunks = p.treek ? 0 : 1;  // the tree kernel writes partials only for chunks below P_b + N
  a.ps_shift = -1;
  if (kv.page_table && kv.page_size > 0 && (kv.page_size & (kv.page_size - 1)) == 0) {
    a.ps_shift = 0;
    while ((1 << a.ps_shift) < kv.page_size) ++a.ps_shift;
  }
  a.tree = p.tree; a.do_scores = p.scores; a.prep_qbar = p.prep_qbar; a.qsplit = p.qsplit;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  a.n_score_rows = n_score_rows;
  a.len_bias = len_bias;
  a.head_scores = head_scores;
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
