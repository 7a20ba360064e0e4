// Sparse draft attention: one decode query per sequence attends to exactly a
// gathered list of KV positions (Vegas §2 step 3; §3: a paged attention kernel
// whose pages hold a single token, with token indices used as page indices).
//
// One 256-thread workgroup per (sequence, KV head, chunk of 64 or 128 listed
// positions: 128 when the lists would need many workgroups).  Each wave gathers 16 of the chunk's K and V rows of that head
// straight into registers: a row is CPR = row bytes / 16 consecutive lanes (a
// lane group), each holding one 16-byte piece, so every gather is whole
// 128-byte lines.  The logits of the query heads sharing the KV head are
// per-lane partial dot products summed over the group's lanes (DPP); each
// lane group then forms its own (m, l, o) over its rows, and the groups'
// partials are combined through LDS into one per query head and chunk.  A
// second kernel merges the chunks with log-sum-exp weights.  The work is a
// few FLOP per byte, so it runs on the vector ALUs; the gathers are what
// costs.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

constexpr int kChunk = 64;     // listed positions per workgroup (16 per wave) ...
constexpr int kChunkBig = 128;  // ... or 32 per wave, when 64-position chunks would
constexpr int kBigGrid = 1024;  // need at least this many workgroups
constexpr int kMaxG = 16;      // query heads per KV head
constexpr int kHeadGroup = 4;  // query heads per pass over the gathered rows

struct SparseArgs {
  const void* q;
  void* out;
  KvView kv;
  const int32_t* idx;
  const int32_t* n_idx;
  float* ws_o;
  f32x2* ws_ml;
  int B, Hq, Hkv, G, idx_stride, max_idx, n_chunks;
  int per_head;  // 1: one index list per (sequence, KV head)
  int chunk;     // listed positions per workgroup (the partial kernel's CH)
  float scale_log2;
};

// Sum over each aligned segment of W lanes, every lane getting its segment's
// sum: DPP quad permutations and row mirrors inside a row of 16 lanes (no LDS
// round trip), a lane shuffle across rows.
template <int W>
__device__ __forceinline__ float seg_sum(float x) {
  if constexpr (W >= 2) x += dpp_f<0xB1, 0xf>(0.f, x);   // quad_perm [1, 0, 3, 2]
  if constexpr (W >= 4) x += dpp_f<0x4E, 0xf>(0.f, x);   // quad_perm [2, 3, 0, 1]
  if constexpr (W >= 8) x += dpp_f<0x141, 0xf>(0.f, x);  // row_half_mirror: the other quad of the 8
  if constexpr (W >= 16) x += dpp_f<0x140, 0xf>(0.f, x); // row_mirror: the other 8 of the row
  if constexpr (W >= 32) x += __shfl_xor(x, 16);
  if constexpr (W >= 64) x += __shfl_xor(x, 32);
  return x;
}

// The EPC elements of a 16-byte piece as floats.
template <typename T, int EPC>
__device__ __forceinline__ void piece_f(const uint4& raw, float (&x)[EPC]) {
  const T* t = reinterpret_cast<const T*>(&raw);
#pragma unroll
  for (int u = 0; u < EPC; ++u) x[u] = (float)t[u];
}

template <typename T, int D, int CH>
__global__ void __launch_bounds__(256) sparse_partial(const SparseArgs a) {
  constexpr int ROWB = D * (int)sizeof(T);
  constexpr int CPR = ROWB / 16;   // lanes per gathered row (one 16-byte piece each)
  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int RPW = 64 / CPR;    // rows a wave holds at once (lane groups)
  constexpr int KW = CH / 4;       // listed positions per wave
  constexpr int U = KW / RPW;      // positions per lane group
  constexpr int HG = kHeadGroup;
  static_assert(CPR <= 64 && RPW * U == KW && U >= 1, "gather geometry");
  // one (m, l, o) partial per (wave, lane group, head of the group)
  __shared__ __attribute__((aligned(16))) float red_o[4][RPW][HG][D];
  __shared__ f32x2 red_ml[4][RPW][HG];

  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, col = lane % CPR, r = lane / CPR;
  const long long lst = a.per_head ? (long long)b * a.Hkv + g : b;  // this KV head's list
  const int k0 = c * CH;
  int n = a.n_idx[lst];
  // positions of this lane group's rows: their loads do not wait for the count
  // (the list holds max_idx entries)
  const int32_t* il = a.idx + lst * a.idx_stride + k0;
  int pos[U];
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int key = wave * KW + r + RPW * i;
    pos[i] = k0 + key < a.max_idx ? il[key] : 0;
  }
  n = n < 0 ? 0 : (n > a.max_idx ? a.max_idx : n);
  if (k0 >= n) return;
  const int nk = min(CH, n - k0);
  const int G = a.G;

  // gather: every load issued before any is used
  const char* kb = reinterpret_cast<const char*>(a.kv.k) + (long long)g * ROWB + col * 16;
  const char* vb = reinterpret_cast<const char*>(a.kv.v) + (long long)g * ROWB + col * 16;
  const long long sb = (long long)a.Hkv * ROWB;
  uint4 kx[U], vx[U];
  bool ok[U];
  long long sl[U];
  if (a.kv.page_table != nullptr) {
    // every row's page entry loaded before any is used (a lookup per row in turn
    // would be one trip to memory each)
    int ent[U];
    bool in[U];
#pragma unroll
    for (int i = 0; i < U; ++i) ent[i] = a.kv.page_table[a.kv.entry_index(b, pos[i], &in[i])];
#pragma unroll
    for (int i = 0; i < U; ++i) sl[i] = a.kv.slot_of_entry(pos[i], ent[i], in[i]);
  } else {
#pragma unroll
    for (int i = 0; i < U; ++i) sl[i] = a.kv.slot(b, pos[i]);
  }
#pragma unroll
  for (int i = 0; i < U; ++i) {
    ok[i] = wave * KW + r + RPW * i < nk;
    const long long s = (ok[i] && sl[i] >= 0) ? sl[i] : 0;  // rows past the count read slot 0 and are masked below
    kx[i] = *reinterpret_cast<const uint4*>(kb + s * sb);
    vx[i] = *reinterpret_cast<const uint4*>(vb + s * sb);
  }

  for (int j0 = 0; j0 < G; j0 += HG) {
    // this lane's columns of the group's queries
    float qf[HG][EPC];
#pragma unroll
    for (int jj = 0; jj < HG; ++jj) {
      if (j0 + jj < G) {
        const uint4 raw = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(a.q) +
                                                          (((long long)b * a.Hq + g * G + j0 + jj) * D) * sizeof(T) +
                                                          col * 16);
        piece_f<T, EPC>(raw, qf[jj]);
      } else {
#pragma unroll
        for (int u = 0; u < EPC; ++u) qf[jj][u] = 0.f;
      }
    }
    // logits (log2 domain): partial dot products summed over the lane group
    float lg[U][HG];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      float kf[EPC];
      piece_f<T, EPC>(kx[i], kf);
#pragma unroll
      for (int jj = 0; jj < HG; ++jj) {
        float acc = 0.f;
#pragma unroll
        for (int u = 0; u < EPC; ++u) acc += qf[jj][u] * kf[u];
        lg[i][jj] = seg_sum<CPR>(acc) * a.scale_log2;
      }
    }
    // the lane group's partial over its U rows: every lane of the group holds
    // the same logits, so m and l need no exchange; each lane sums P V for its
    // own columns
    float o[HG][EPC];
#pragma unroll
    for (int jj = 0; jj < HG; ++jj) {
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < U; ++i) mx = ok[i] ? fmaxf(mx, lg[i][jj]) : mx;
      float ls = 0.f;
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const float p = (ok[i] && mx != kNegInf) ? fast_exp2(lg[i][jj] - mx) : 0.f;
        lg[i][jj] = p;
        ls += p;
      }
      if (col == 0) red_ml[wave][r][jj] = f32x2{mx, ls};
#pragma unroll
      for (int u = 0; u < EPC; ++u) o[jj][u] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      float vf[EPC];
      piece_f<T, EPC>(vx[i], vf);
#pragma unroll
      for (int jj = 0; jj < HG; ++jj)
#pragma unroll
        for (int u = 0; u < EPC; ++u) o[jj][u] += lg[i][jj] * vf[u];
    }
#pragma unroll
    for (int jj = 0; jj < HG; ++jj)
#pragma unroll
      for (int u = 0; u < EPC; u += 4)
        *reinterpret_cast<f32x4*>(&red_o[wave][r][jj][col * EPC + u]) =
            f32x4{o[jj][u], o[jj][u + 1], o[jj][u + 2], o[jj][u + 3]};
    __syncthreads();

    // the group's 4 * RPW partials of each (head, column pair), combined in a fixed order
    const int hg = min(HG, G - j0);
    for (int e = tid; e < hg * (D / 2); e += 256) {
      const int jj = e / (D / 2), d = 2 * (e % (D / 2));
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int q = 0; q < RPW; ++q) M = fmaxf(M, red_ml[w][q][jj][0]);
      float L = 0.f, o0 = 0.f, o1 = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int q = 0; q < RPW; ++q) {
          const f32x2 ml = red_ml[w][q][jj];
          const float wt = ml[0] == kNegInf ? 0.f : fast_exp2(ml[0] - M);
          const f32x2 ov = *reinterpret_cast<const f32x2*>(&red_o[w][q][jj][d]);
          L += wt * ml[1];
          o0 += wt * ov[0];
          o1 += wt * ov[1];
        }
      const long long rec = ((long long)b * a.Hq + g * G + j0 + jj) * a.n_chunks + c;
      *reinterpret_cast<f32x2*>(a.ws_o + rec * D + d) = f32x2{o0, o1};
      if (d == 0) a.ws_ml[rec] = f32x2{M, L};
    }
    if (j0 + HG < G) __syncthreads();  // the next group rewrites the partials
  }
}

// Chunk merge: one wave per (sequence, query head).  The pair's partials are
// contiguous ([chunk][D] floats); each lane keeps its own running (m, l, o)
// over the chunks it reads, fetching a batch's (m, l) and o together (one
// trip to memory per batch), and the lanes holding the same columns are
// combined with log-sum-exp weights at the end.
template <typename T, int D>
__global__ void __launch_bounds__(256) sparse_merge(const SparseArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + wave;
  if (bh >= a.B * a.Hq) return;
  const int b = bh / a.Hq;
  const long long rec0 = (long long)bh * a.n_chunks;
  constexpr int Q4 = D / 4;          // float4 column groups per row
  constexpr int CPL = 64 / Q4;       // chunks covered by one wave-wide load step
  constexpr int STEPS = 16;          // load steps in flight per batch
  const int quad = lane % Q4, sub = lane / Q4;
  float m = kNegInf, lsum = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 x[STEPS];
  f32x2 ml[STEPS];
  // a batch of chunks, loaded unconditionally at indices clamped into the
  // workspace (a guarded load would wait for its predecessor); records past
  // the count hold stale data and are selected away below
  auto fetch = [&](int cb) {
#pragma unroll
    for (int j = 0; j < STEPS; ++j) {
      const int c = min(cb + j * CPL + sub, a.n_chunks - 1);
      x[j] = *reinterpret_cast<const f32x4*>(a.ws_o + (rec0 + c) * D + 4 * quad);
      ml[j] = a.ws_ml[rec0 + c];
    }
  };
  // the first batch is requested before the count: the loads do not wait for it
  fetch(0);
  int n = a.n_idx[a.per_head ? (long long)b * a.Hkv + (bh % a.Hq) / a.G : b];
  n = n < 0 ? 0 : (n > a.max_idx ? a.max_idx : n);
  const int nc = (n + a.chunk - 1) / a.chunk;
  for (int cb = 0;;) {
    // records past the count are selected away unread
#pragma unroll
    for (int j = 0; j < STEPS; ++j) {
      if (cb + j * CPL + sub >= nc) {
        x[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        ml[j] = f32x2{kNegInf, 0.f};
      }
    }
    float bm = m;
#pragma unroll
    for (int j = 0; j < STEPS; ++j) bm = fmaxf(bm, ml[j][0]);
    const float wa = m == kNegInf ? 0.f : fast_exp2(m - bm);
    acc *= wa;
    lsum *= wa;
#pragma unroll
    for (int j = 0; j < STEPS; ++j) {
      const float w = ml[j][0] == kNegInf ? 0.f : fast_exp2(ml[j][0] - bm);
      acc += w * x[j];
      lsum += w * ml[j][1];
    }
    m = bm;
    cb += CPL * STEPS;
    if (cb >= nc) break;
    fetch(cb);
  }
  // lanes with the same quad (different sub) hold different chunks
  const float M = wave_max(m);
  const float wl = m == kNegInf ? 0.f : fast_exp2(m - M);
  acc *= wl;
  lsum *= wl;
#pragma unroll
  for (int o = Q4; o < 64; o <<= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], o);
    lsum += __shfl_xor(lsum, o);
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  if (sub == 0) {
    T* dst = reinterpret_cast<T*>(a.out) + (long long)bh * D + 4 * quad;
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = (T)(acc[e] * inv);
  }
}

// Compaction of a selected set: the K and V rows (all KV heads, Hkv * D
// elements each) of the listed logical positions are copied into dense
// per-sequence buffers, so that the draft steps that follow read one
// contiguous stream instead of gathering the set again each time.  One
// workgroup copies kCompactRows rows of one sequence as 16-byte pieces, every
// load of a batch issued before any store.
constexpr int kCompactRows = 16;
using u32x4 = uint32_t __attribute__((ext_vector_type(4)));

struct CompactArgs {
  KvView kv;
  const int32_t* idx;
  const int32_t* n_idx;
  char* ck;
  char* cv;
  int idx_stride, max_idx, cap;
  int row_pieces;  // 16-byte pieces per row: Hkv * D * sizeof(T) / 16
};

__global__ void __launch_bounds__(256) compact_rows(const CompactArgs a) {
  constexpr int U = 4;  // pieces per thread per batch (of K and of V)
  const int b = blockIdx.y, tid = threadIdx.x;
  int n = a.n_idx[b];
  n = n < 0 ? 0 : (n > a.max_idx ? a.max_idx : n);
  n = n > a.cap ? a.cap : n;
  const int j0 = blockIdx.x * kCompactRows;
  if (j0 >= n) return;
  const int nr = min(kCompactRows, n - j0);
  const int total = nr * a.row_pieces;
  const long long row_bytes = (long long)a.row_pieces * 16;
  const char* kb = reinterpret_cast<const char*>(a.kv.k);
  const char* vb = reinterpret_cast<const char*>(a.kv.v);
  for (int base = 0; base < total; base += 256 * U) {
    // loads at clamped (always valid) pieces, all issued before the first store;
    // positions, then page entries, then rows, each step's loads issued together
    u32x4 kx[U], vx[U];
    long long dst[U], sl[U];
    int pos[U], cc[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = base + tid + 256 * u;
      ok[u] = e < total;
      const int ec = ok[u] ? e : total - 1;
      const int r = ec / a.row_pieces;
      cc[u] = ec % a.row_pieces;
      pos[u] = a.idx[(long long)b * a.idx_stride + j0 + r];
      dst[u] = ((long long)b * a.cap + j0 + r) * row_bytes + cc[u] * 16;
    }
    if (a.kv.page_table != nullptr) {
      int ent[U];
      bool in[U];
#pragma unroll
      for (int u = 0; u < U; ++u) ent[u] = a.kv.page_table[a.kv.entry_index(b, pos[u], &in[u])];
#pragma unroll
      for (int u = 0; u < U; ++u) sl[u] = a.kv.slot_of_entry(pos[u], ent[u], in[u]);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) sl[u] = a.kv.slot(b, pos[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long s = sl[u] >= 0 ? sl[u] : 0;  // unmapped positions copy slot 0 (a caller-contract violation)
      kx[u] = *reinterpret_cast<const u32x4*>(kb + s * row_bytes + cc[u] * 16);
      vx[u] = *reinterpret_cast<const u32x4*>(vb + s * row_bytes + cc[u] * 16);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ok[u]) {
        *reinterpret_cast<u32x4*>(a.ck + dst[u]) = kx[u];
        *reinterpret_cast<u32x4*>(a.cv + dst[u]) = vx[u];
      }
    }
  }
}

int launch_compact(int dtype, int B, int Hkv, int D, const KvArgs& kv, const int32_t* idx, int idx_stride,
                   const int32_t* n_idx, int max_idx, void* ck, void* cv, int cap, void* stream) {
  CompactArgs a{};
  a.kv = KvView{kv.k, kv.v, kv.page_table, kv.page_size, kv.max_pages, kv.seq_stride, kv.num_slots};
  a.idx = idx;
  a.n_idx = n_idx;
  a.ck = reinterpret_cast<char*>(ck);
  a.cv = reinterpret_cast<char*>(cv);
  a.idx_stride = idx_stride;
  a.max_idx = max_idx;
  a.cap = cap;
  a.row_pieces = Hkv * D * (dtype == SV_BF16 ? 2 : 4) / 16;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int rows = min(max_idx, cap);
  if (B == 0 || rows <= 0) return 0;
  hipLaunchKernelGGL(compact_rows, dim3((rows + kCompactRows - 1) / kCompactRows, B), dim3(256), 0, st, a);
  return (int)hipGetLastError();
}

// Query-agnostic baseline selection: the first `sink` and the last `window`
// prefix positions, in increasing order, then -1 up to k_max (the same
// output format as the top-k selection).
__global__ void __launch_bounds__(256) sink_window(const int32_t* prefix_len, int P_max, int sink, int window,
                                                   int k_max, int32_t* idx, int32_t* count) {
  const int b = blockIdx.x;
  int P = prefix_len[b];
  P = P < 0 ? 0 : (P > P_max ? P_max : P);
  const int s = min(sink, P);
  const int w0 = max(s, P - window);
  const int n = s + (P - w0);
  for (int j = threadIdx.x; j < k_max; j += 256)
    idx[(long long)b * k_max + j] = j < s ? j : (j < n ? w0 + (j - s) : -1);
  if (threadIdx.x == 0 && count) count[b] = n;
}

int launch_sink_window(int B, int P_max, const int32_t* prefix_len, int sink, int window, int k_max, int32_t* idx,
                       int32_t* count, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (B == 0) return 0;
  hipLaunchKernelGGL(sink_window, dim3(B), dim3(256), 0, st, prefix_len, P_max, sink, window, k_max, idx, count);
  return (int)hipGetLastError();
}

SparsePlan plan_sparse(int B, int Hq, int Hkv, int D, int max_idx) {
  SparsePlan p{};
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv; p.D = D; p.max_idx = max_idx;
  // larger chunks when the grid is large: fewer partials, and the gathers of
  // a workgroup still fit its registers (measured: -24 us over 15 gathered
  // steps of 4 x 4096 positions, +1 us at one sequence of 2048)
  const long long wgs64 = (long long)B * Hkv * ((max_idx + kChunk - 1) / kChunk);
  p.KCH = wgs64 >= kBigGrid ? kChunkBig : kChunk;
  p.n_chunks = (max_idx + p.KCH - 1) / p.KCH;
  if (p.n_chunks < 1) p.n_chunks = 1;
  size_t off = 0;
  p.off_o = off; off = align_up(off + (size_t)B * Hq * p.n_chunks * D * 4);
  p.off_ml = off; off = align_up(off + (size_t)B * Hq * p.n_chunks * 8);
  p.bytes = off;
  return p;
}

template <typename T, int D>
static void launch_sparse_typed(const SparsePlan& p, const SparseArgs& a, hipStream_t st) {
  if (p.max_idx > 0 && p.KCH == kChunkBig)
    hipLaunchKernelGGL((sparse_partial<T, D, kChunkBig>), dim3(p.n_chunks, p.Hkv, p.B), dim3(256), 0, st, a);
  else if (p.max_idx > 0)
    hipLaunchKernelGGL((sparse_partial<T, D, kChunk>), dim3(p.n_chunks, p.Hkv, p.B), dim3(256), 0, st, a);
  hipLaunchKernelGGL((sparse_merge<T, D>), dim3((p.B * p.Hq + 3) / 4), dim3(256), 0, st, a);
}

int launch_sparse(const SparsePlan& p, int dtype, const void* q, const KvArgs& kv, const int32_t* idx,
                  int idx_stride, const int32_t* n_idx, float scale, void* out, void* ws, void* stream,
                  int per_head) {
  SparseArgs a{};
  a.q = q;
  a.out = out;
  a.kv = KvView{kv.k, kv.v, kv.page_table, kv.page_size, kv.max_pages, kv.seq_stride, kv.num_slots};
  a.idx = idx;
  a.n_idx = n_idx;
  char* w = reinterpret_cast<char*>(ws);
  a.ws_o = reinterpret_cast<float*>(w + p.off_o);
  a.ws_ml = reinterpret_cast<f32x2*>(w + p.off_ml);
  a.B = p.B; a.Hq = p.Hq; a.Hkv = p.Hkv; a.G = p.G; a.idx_stride = idx_stride; a.max_idx = p.max_idx;
  a.n_chunks = p.n_chunks;
  a.chunk = p.KCH;
  a.per_head = per_head;
  a.scale_log2 = scale * kLog2e;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (p.B == 0 || p.Hq == 0) return 0;
  if (dtype == SV_BF16) {
    if (p.D == 128) launch_sparse_typed<bf16, 128>(p, a, st);
    else launch_sparse_typed<bf16, 64>(p, a, st);
  } else {
    if (p.D == 128) launch_sparse_typed<float, 128>(p, a, st);
    else launch_sparse_typed<float, 64>(p, a, st);
  }
  return (int)hipGetLastError();
}

}  // namespace sv
