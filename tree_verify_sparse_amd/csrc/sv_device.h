// Device-side building blocks for gfx950 (CDNA4): vector types, MFMA wrappers,
// LDS transpose reads and small cross-lane helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// C/D layout of the 32x32 MFMAs (checked on gfx950): lane l holds column l % 32;
// element v holds row 8*(v/4) + 4*(l/32) + v%4.
__device__ __forceinline__ int mfma_row(int v, int half) { return 8 * (v >> 2) + 4 * half + (v & 3); }

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  // A: lane l holds row l%32, k = 8*(l/32) + [0,8); B: column l%32, same k.
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, const f32x16& c) {
  // A: lane l holds row l%32, k = l/32; B: column l%32, k = l/32.
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane 4e+c supplies the address of 4 consecutive 16-bit elements; lane j of
// the group receives, as its element e, element (j % 4) of lane 4e + j/4.
// With lane 4e+c pointing at row (base+e), columns [4c, 4c+4) of a row-major
// tile, lane j gets column j of rows base..base+3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const bf16* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)((__attribute__((address_space(3))) void*)p));
  bf16x4 out;
  __builtin_memcpy(&out, &r, sizeof(out));
  return out;
}

__device__ __forceinline__ float bf16_to_f32(bf16 x) { return (float)x; }

// Wave-wide reductions on DPP (row shifts by 1, 2, 4, 8 inside each row of
// 16 lanes, then the broadcasts of lane 15 into rows 1 and 3 and of lane 31
// into rows 2 and 3): lane 63 ends with the reduction of all 64 lanes, which
// is then broadcast.  No LDS round trips, unlike the shuffles.  Lanes a shift
// reads from outside the row contribute the identity `id`.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_f(float id, float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(id), __float_as_int(x), CTRL, ROWS, 0xf, false));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u(uint32_t id, uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, CTRL, ROWS, 0xf, false);
}
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T x, T id, Op op) {
  if constexpr (sizeof(T) == 4 && __is_same(T, float)) {
    x = op(x, dpp_f<0x111, 0xf>(id, x));
    x = op(x, dpp_f<0x112, 0xf>(id, x));
    x = op(x, dpp_f<0x114, 0xf>(id, x));
    x = op(x, dpp_f<0x118, 0xf>(id, x));
    x = op(x, dpp_f<0x142, 0xa>(id, x));
    x = op(x, dpp_f<0x143, 0xc>(id, x));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
  } else {
    x = op(x, dpp_u<0x111, 0xf>(id, x));
    x = op(x, dpp_u<0x112, 0xf>(id, x));
    x = op(x, dpp_u<0x114, 0xf>(id, x));
    x = op(x, dpp_u<0x118, 0xf>(id, x));
    x = op(x, dpp_u<0x142, 0xa>(id, x));
    x = op(x, dpp_u<0x143, 0xc>(id, x));
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
  }
}
__device__ __forceinline__ float wave_max(float x) {  // NaN lanes are skipped (fmaxf)
  return wave_reduce(x, -__builtin_inff(), [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float wave_min(float x) {  // NaN lanes are skipped (fminf)
  return wave_reduce(x, __builtin_inff(), [](float a, float b) { return fminf(a, b); });
}
__device__ __forceinline__ float wave_sum(float x) {
  return wave_reduce(x, 0.f, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  return wave_reduce(x, 0xffffffffu, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  return wave_reduce(x, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  return wave_reduce(x, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

// 2^x on the transcendental unit (2^-inf = 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wait until at most N vector-memory operations of this wave are outstanding
// and all its LDS operations are done (s_waitcnt vmcnt(N) lgkmcnt(0)).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0x0 << 8) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0): every LDS access of this wave has completed.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14)); }

// Workgroup barrier without the memory fence __syncthreads() implies (the
// fence would make the compiler drain every outstanding global->LDS copy).
// Callers order memory explicitly with wait_vm_lgkm0 first.
__device__ __forceinline__ void barrier_only() { __builtin_amdgcn_s_barrier(); }

// Copy 16 bytes per lane from global memory straight into LDS: lane l writes
// lds_base + 16*l (lds_base is wave-uniform).  Counted by vmcnt.  Issued as
// inline assembly on purpose: the compiler then does not know that LDS is
// written asynchronously and adds no vmcnt(0) drains before LDS reads that it
// cannot prove disjoint from the copy; callers order the copies themselves
// with wait_vm_lgkm0 + barrier_only (compiler-issued loads that are older
// than these copies stay correctly waited for, since completion is in order).
__device__ __forceinline__ void global_to_lds16(const void* src, void* lds_base) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(l), "v"(src) : "memory");  // streamed: non-temporal
}

// K/V storage addressing: logical position -> slot; out-of-range -> -1.
struct KvView {
  const void* k;
  const void* v;
  const int32_t* page_table;
  int page_size;
  int max_pages;
  long long seq_stride;
  long long num_slots;

  __device__ __forceinline__ long long slot(int b, int pos) const {
    long long s;
    if (page_table == nullptr) {
      s = (long long)b * seq_stride + pos;
    } else {
      bool in;
      s = slot_of_entry(pos, page_table[entry_index(b, pos, &in)], in);
    }
    return (s >= 0 && s < num_slots && pos >= 0) ? s : -1;
  }
  // Paged caches, in two steps, so that a caller can issue the page-table loads
  // of several positions before it uses any (one trip to memory for all of them,
  // not one each): the table entry of a position (clamped into the table; *in
  // says whether the page exists), then the slot from that entry.
  __device__ __forceinline__ long long entry_index(int b, int pos, bool* in) const {
    const int pg = pos / page_size;
    *in = pos >= 0 && pg < max_pages;
    return (long long)b * max_pages + (*in ? pg : 0);
  }
  __device__ __forceinline__ long long slot_of_entry(int pos, int entry, bool in) const {
    const long long s = (long long)entry * page_size + (pos - (pos / page_size) * page_size);
    return (in && entry >= 0 && s < num_slots) ? s : -1;
  }
};

}  // namespace sv
