// Sparse draft attention: one decode query per sequence attends to exactly a
// gathered list of KV positions (Vegas §2 step 3; §3: a paged attention kernel
// whose pages hold a single token, with token indices used as page indices).
//
// One 256-thread workgroup per (sequence, KV head, chunk of kChunk listed
// positions): it gathers the chunk's K and V rows of that head (each a
// contiguous D-element row, so every gather is whole 128-byte lines) into LDS,
// forms the logits of the G query heads sharing the KV head, and writes a
// partial (m, l, o) per query head.  A second kernel merges the chunks with
// log-sum-exp weights.  The work is a few FLOP per byte, so it runs on the
// vector ALUs; the gathers are what costs.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

constexpr int kChunk = 64;
constexpr int kMaxG = 16;

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
  float scale_log2;
};

template <typename T, int D>
__global__ void __launch_bounds__(256) sparse_partial(const SparseArgs a) {
  constexpr int ROWB = D * (int)sizeof(T);
  constexpr int CPR = ROWB / 16;              // 16-byte pieces per row
  constexpr int LOADS = kChunk * CPR / 256;   // pieces per thread per tensor
  constexpr int EPC = 16 / (int)sizeof(T);    // elements per piece
  constexpr int KSTR = D + EPC;               // LDS row stride (elements): +16 bytes spreads banks
  __shared__ __attribute__((aligned(16))) T Ks[kChunk][KSTR];
  __shared__ __attribute__((aligned(16))) T Vs[kChunk][D];
  __shared__ __attribute__((aligned(16))) float qs[kMaxG][D];
  __shared__ float lg[kMaxG][kChunk];
  __shared__ float mls[kMaxG][2];

  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const long long lst = a.per_head ? (long long)b * a.Hkv + g : b;  // this KV head's list
  int n = a.n_idx[lst];
  n = n < 0 ? 0 : (n > a.max_idx ? a.max_idx : n);
  const int k0 = c * kChunk;
  if (k0 >= n) return;
  const int nk = min(kChunk, n - k0);
  const int G = a.G;

  // gather: every load of the chunk is issued before any is used
  const char* kb = reinterpret_cast<const char*>(a.kv.k) + (long long)g * ROWB;
  const char* vb = reinterpret_cast<const char*>(a.kv.v) + (long long)g * ROWB;
  const long long sb = (long long)a.Hkv * ROWB;
  uint4 kx[LOADS], vx[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int e = tid + 256 * i, key = e / CPR, col = e % CPR;
    long long s = -1;
    if (key < nk) s = a.kv.slot(b, a.idx[lst * a.idx_stride + k0 + key]);
    if (s < 0) s = 0;  // unused or unmapped entries read slot 0 and are masked below
    kx[i] = *reinterpret_cast<const uint4*>(kb + s * sb + col * 16);
    vx[i] = *reinterpret_cast<const uint4*>(vb + s * sb + col * 16);
  }
  for (int e = tid; e < G * D; e += 256) {
    const int j = e / D, d = e % D;
    qs[j][d] = (float)reinterpret_cast<const T*>(a.q)[((long long)b * a.Hq + g * G + j) * D + d];
  }
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int e = tid + 256 * i, key = e / CPR, col = e % CPR;
    *reinterpret_cast<uint4*>(&Ks[key][col * EPC]) = kx[i];
    *reinterpret_cast<uint4*>(&Vs[key][col * EPC]) = vx[i];
  }
  __syncthreads();

  // logits: one (head, key) pair per thread, 16-byte LDS reads
  for (int e = tid; e < G * kChunk; e += 256) {
    const int j = e / kChunk, key = e % kChunk;
    float acc = 0.f;
#pragma unroll
    for (int cc = 0; cc < CPR; ++cc) {
      const uint4 raw = *reinterpret_cast<const uint4*>(&Ks[key][cc * EPC]);
      const T* kt = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int u = 0; u < EPC; ++u) acc += qs[j][cc * EPC + u] * (float)kt[u];
    }
    lg[j][key] = key < nk ? acc * a.scale_log2 : kNegInf;
  }
  __syncthreads();

  // softmax statistics per head: one wave per head, one lane per key
  const int wave = tid >> 6, lane = tid & 63;
  for (int j = wave; j < G; j += 4) {
    const float x = lg[j][lane];
    const float mx = wave_max(x);
    const float p = x == kNegInf ? 0.f : fast_exp2(x - mx);
    const float ls = wave_sum(p);
    lg[j][lane] = p;
    if (lane == 0) {
      mls[j][0] = mx;
      mls[j][1] = ls;
    }
  }
  __syncthreads();

  // P V: one (head, column pair) per thread
  for (int e = tid; e < G * (D / 2); e += 256) {
    const int j = e / (D / 2), d = 2 * (e % (D / 2));
    float a0 = 0.f, a1 = 0.f;
#pragma unroll 8
    for (int key = 0; key < nk; ++key) {
      const float p = lg[j][key];
      a0 += p * (float)Vs[key][d];
      a1 += p * (float)Vs[key][d + 1];
    }
    const long long rec = ((long long)b * a.Hq + g * G + j) * a.n_chunks + c;
    *reinterpret_cast<f32x2*>(a.ws_o + rec * D + d) = f32x2{a0, a1};
    if (d == 0) a.ws_ml[rec] = f32x2{mls[j][0], mls[j][1]};
  }
}

// Chunk merge: one wave per (sequence, query head).  The pair's partials are
// contiguous ([chunk][D] floats), so the wave fetches up to 256 / (D / 4)
// chunks per round with one 16-byte load per lane per step, every load issued
// before any is used; lanes holding the same columns are then summed.
template <typename T, int D>
__global__ void __launch_bounds__(256) sparse_merge(const SparseArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + wave;
  if (bh >= a.B * a.Hq) return;
  const int b = bh / a.Hq;
  int n = a.n_idx[a.per_head ? (long long)b * a.Hkv + (bh % a.Hq) / a.G : b];
  n = n < 0 ? 0 : (n > a.max_idx ? a.max_idx : n);
  const int nc = (n + kChunk - 1) / kChunk;
  const long long rec0 = (long long)bh * a.n_chunks;
  float M = kNegInf;
  for (int c = lane; c < nc; c += 64) M = fmaxf(M, a.ws_ml[rec0 + c][0]);
  M = wave_max(M);
  constexpr int Q4 = D / 4;          // float4 column groups per row
  constexpr int CPL = 64 / Q4;       // chunks covered by one wave-wide load step
  constexpr int STEPS = 8;           // load steps in flight per round
  const int quad = lane % Q4, sub = lane / Q4;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
  for (int cb = 0; cb < nc; cb += CPL * STEPS) {
    f32x4 x[STEPS];
    float w[STEPS];
#pragma unroll
    for (int j = 0; j < STEPS; ++j) {
      const int c = cb + j * CPL + sub;
      x[j] = c < nc ? *reinterpret_cast<const f32x4*>(a.ws_o + (rec0 + c) * D + 4 * quad) : f32x4{0.f, 0.f, 0.f, 0.f};
      const f32x2 ml = c < nc ? a.ws_ml[rec0 + c] : f32x2{kNegInf, 0.f};
      w[j] = (M == kNegInf || c >= nc) ? 0.f : fast_exp2(ml[0] - M);
      if (quad == 0) lsum += w[j] * ml[1];
    }
#pragma unroll
    for (int j = 0; j < STEPS; ++j) acc += w[j] * x[j];
  }
  // lanes with the same quad (different sub) hold different chunks: sum them
#pragma unroll
  for (int o = Q4; o < 64; o <<= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], o);
  }
  lsum = wave_sum(lsum);
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
    uint4 kx[U], vx[U];
    long long dst[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = base + tid + 256 * u;
      const int r = e / a.row_pieces, c = e % a.row_pieces;
      long long sl = -1;
      if (e < total) sl = a.kv.slot(b, a.idx[(long long)b * a.idx_stride + j0 + r]);
      if (sl < 0) sl = 0;  // unmapped positions copy slot 0 (a caller-contract violation)
      dst[u] = e < total ? ((long long)b * a.cap + j0 + r) * row_bytes + c * 16 : -1;
      kx[u] = *reinterpret_cast<const uint4*>(kb + sl * row_bytes + c * 16);
      vx[u] = *reinterpret_cast<const uint4*>(vb + sl * row_bytes + c * 16);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (dst[u] >= 0) {
        *reinterpret_cast<uint4*>(a.ck + dst[u]) = kx[u];
        *reinterpret_cast<uint4*>(a.cv + dst[u]) = vx[u];
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
  p.KCH = kChunk;
  p.n_chunks = (max_idx + kChunk - 1) / kChunk;
  if (p.n_chunks < 1) p.n_chunks = 1;
  size_t off = 0;
  p.off_o = off; off = align_up(off + (size_t)B * Hq * p.n_chunks * D * 4);
  p.off_ml = off; off = align_up(off + (size_t)B * Hq * p.n_chunks * 8);
  p.bytes = off;
  return p;
}

template <typename T, int D>
static void launch_sparse_typed(const SparsePlan& p, const SparseArgs& a, hipStream_t st) {
  if (p.max_idx > 0)
    hipLaunchKernelGGL((sparse_partial<T, D>), dim3(p.n_chunks, p.Hkv, p.B), dim3(256), 0, st, a);
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
