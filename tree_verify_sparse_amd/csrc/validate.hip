// Device-side checks of the caller contract on device arrays (prefix
// lengths, tree parents, page tables, index lists).  The compute kernels are
// defensive (a position mapped outside the KV storage reads slot 0, a
// malformed parent makes a root), so a violated contract gives wrong results
// rather than a fault; these kernels find such violations on the caller's
// stream.  Each writes an error record {code, b, i, value} into a
// caller-owned int32[4]: all zero when every check passes, otherwise one of
// the violations (which one is not specified when there are several).
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

namespace {

__device__ __forceinline__ void report(int32_t* err, int code, int b, int i, int value) {
  if (atomicCAS(reinterpret_cast<int*>(err), 0, code) == 0) {
    err[1] = b;
    err[2] = i;
    err[3] = value;
  }
}

__global__ void clear_err(int32_t* err) {
  if (threadIdx.x < 4) err[threadIdx.x] = 0;
}

// One thread per (sequence, position in [0, P_max + N)): the prefix length is
// in [0, P_max], and every position below P_b + N maps to a slot of the
// storage (a mapped page for a paged cache).
__global__ void __launch_bounds__(256) check_kv_positions(KvView kv, const int32_t* prefix_len, int P_max, int N,
                                                          int32_t* err) {
  const int b = blockIdx.y;
  const int P = prefix_len[b];
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (P < 0 || P > P_max) {
    if (i == 0) report(err, kErrPrefixLen, b, 0, P);
    return;
  }
  if (i >= P + N) return;
  if (kv.slot(b, i) < 0) {
    int v = -1;
    if (kv.page_table) {
      const int pg = i / kv.page_size;
      v = pg < kv.max_pages ? kv.page_table[(long long)b * kv.max_pages + pg] : -1;
    }
    report(err, kErrUnmapped, b, i, v);
  }
}

// One thread per (sequence, node): parent[b][0] = -1 and 0 <= parent[b][i] < i.
__global__ void __launch_bounds__(256) check_parents(const int32_t* parent, int N, int32_t* err) {
  const int b = blockIdx.y, i = blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  const int p = parent[(long long)b * N + i];
  if (i == 0 ? p != -1 : (p < 0 || p >= i)) report(err, kErrParent, b, i, p);
}

// One thread per (list, entry): the count is in [0, max_idx], and each of
// the first count entries is a position >= 0 that maps to a slot.
__global__ void __launch_bounds__(256) check_index_lists(KvView kv, const int32_t* idx, int idx_stride,
                                                         const int32_t* n_idx, int max_idx, int lists_per_seq,
                                                         int32_t* err) {
  const int lst = blockIdx.y, b = lst / lists_per_seq;
  const int n = n_idx[lst];
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (n < 0 || n > max_idx) {
    if (j == 0) report(err, kErrCount, lst, 0, n);
    return;
  }
  if (j >= n) return;
  const int pos = idx[(long long)lst * idx_stride + j];
  if (pos < 0 || kv.slot(b, pos) < 0) report(err, kErrIndex, lst, j, pos);
}

KvView view(const KvArgs& kv) {
  return KvView{kv.k, kv.v, kv.page_table, kv.page_size, kv.max_pages, kv.seq_stride, kv.num_slots};
}

}  // namespace

int launch_validate_kv(int B, int N, const KvArgs& kv, const int32_t* prefix_len, int P_max, int32_t* err,
                       void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipLaunchKernelGGL(clear_err, dim3(1), dim3(64), 0, st, err);
  if (B > 0) {
    const long long L = (long long)P_max + N;
    hipLaunchKernelGGL(check_kv_positions, dim3((unsigned)((L + 255) / 256 > 0 ? (L + 255) / 256 : 1), B), dim3(256),
                       0, st, view(kv), prefix_len, P_max, N, err);
  }
  return (int)hipGetLastError();
}

int launch_validate_tree(int B, int N, const int32_t* parent, int32_t* err, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipLaunchKernelGGL(clear_err, dim3(1), dim3(64), 0, st, err);
  if (B > 0 && N > 0)
    hipLaunchKernelGGL(check_parents, dim3((N + 255) / 256, B), dim3(256), 0, st, parent, N, err);
  return (int)hipGetLastError();
}

int launch_validate_index(int n_lists, int lists_per_seq, const KvArgs& kv, const int32_t* idx, int idx_stride,
                          const int32_t* n_idx, int max_idx, int32_t* err, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipLaunchKernelGGL(clear_err, dim3(1), dim3(64), 0, st, err);
  if (n_lists > 0)
    hipLaunchKernelGGL(check_index_lists, dim3(max_idx > 0 ? (max_idx + 255) / 256 : 1, n_lists), dim3(256), 0, st,
                       view(kv), idx, idx_stride, n_idx, max_idx, lists_per_seq, err);
  return (int)hipGetLastError();
}

}  // namespace sv
