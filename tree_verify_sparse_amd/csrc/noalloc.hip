// Verification attention without a caller workspace: the chunk partials,
// score partials and ancestor sets live in a library-owned static device
// array instead of caller memory, for callers that cannot allocate (code under
// graph capture, serving loops that forbid allocation).
//
// The array is `scratch` below.  Its host-side name is only a stand-in for the
// device symbol, so host code never passes it to a kernel: once per device, at
// that device's first call, its device address is fetched with
// hipGetSymbolAddress and kept, and every launch takes that address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sv.h"
#include "sv_internal.h"

namespace {

static __device__ __align__(256) char scratch[SV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::once_flag g_scratch_once[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices] = {};

// Device address of `scratch` on the current device (fetched once per device).
hipError_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (g_scratch_err[dev] == hipSuccess && p == nullptr) g_scratch_err[dev] = hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  });
  *out = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

}  // namespace

extern "C" sv_status sv_verify_attn_noalloc(const void* q, sv_dtype dtype, int B, int N, int Hq, int Hkv, int D,
                                            const sv_kv_cache* kv, const int32_t* prefix_len, int P_max,
                                            const int32_t* parent, const int32_t* score_rows_host,
                                            int n_score_rows, float softmax_scale, void* out, float* scores,
                                            sv_stream stream) {
  // Everything sv_verify_attn checks is checked by it; the scratch size is
  // checked first so that an oversized call launches nothing.
  size_t need = 0;
  if (B > 0 && N >= 1 && N <= sv::kMaxNodes && Hq > 0 && Hkv > 0 && Hq % Hkv == 0 && (D == 64 || D == 128) &&
      P_max >= 0 && n_score_rows >= 0 && kv != nullptr && (dtype == SV_F32 || dtype == SV_BF16)) {
    need = sv_verify_workspace_size(B, N, Hq, Hkv, D, P_max, dtype, parent != nullptr, n_score_rows,
                                    kv->page_table ? kv->page_size : 0);
    if (need > (size_t)SV_NOALLOC_SCRATCH_BYTES)
      return sv::set_error(SV_E_WORKSPACE,
                           "sv_verify_attn_noalloc: this call needs %zu bytes of scratch, more than the %zu "
                           "bytes of the library's static array (use sv_verify_attn with a workspace)",
                           need, (size_t)SV_NOALLOC_SCRATCH_BYTES);
  }
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = scratch_on_current_device(&ws);
    if (e != hipSuccess)
      return sv::set_error(SV_E_HIP, "sv_verify_attn_noalloc: no device address for the static scratch: %s",
                           hipGetErrorString(e));
  }
  return sv_verify_attn(q, dtype, B, N, Hq, Hkv, D, kv, prefix_len, P_max, parent, score_rows_host, n_score_rows,
                        softmax_scale, out, scores, ws, need, stream);
}
