// lla_decode_attn_noalloc: per-head decode attention (paper Sec. 3, Eq. 3
// and "RoPE and reconstruction") for callers that cannot allocate device
// memory.  It runs exactly the kernels of lla_decode_attn; the context-split
// partials (m, l, sum p c_v) that lla_decode_attn writes to the caller's
// workspace go to `scratch`, a static array of this file that every GPU the
// library runs on holds until the process ends.
//
// `scratch` is named only in the symbol lookup below: in host code its name
// is the host-side shadow, not a device address, so the kernels receive the
// address hipGetSymbolAddress returns for the current device.
#include <mutex>

#include "lla.h"
#include "lla_internal.h"

static __device__ __align__(256) unsigned char scratch[LLA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  std::once_flag once;
  hipError_t err = hipSuccess;
  void *ptr = nullptr;
};
DeviceScratch g_scratch[kMaxDevices];

// Device address of `scratch` on the current device, looked up on the
// device's first call (with that device current) and kept for the process.
lla_status_t current_scratch(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return LLA_E_HIP;
  if (dev >= kMaxDevices) return LLA_E_UNSUPPORTED;
  DeviceScratch &s = g_scratch[dev];
  std::call_once(s.once, [&s] {
    void *p = nullptr;
    s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (s.err == hipSuccess) s.ptr = p;
  });
  if (s.err != hipSuccess || s.ptr == nullptr) return LLA_E_HIP;
  *out = s.ptr;
  return LLA_OK;
}

}  // namespace

extern "C" lla_status_t lla_decode_attn_noalloc(const lla_store_t *store, int32_t layer,
                                                int32_t loop, const float *q,
                                                const void *w_up_k_t, const void *w_up_v_t,
                                                const float *mu_k_t, const float *mu_v_t,
                                                const int32_t *pos, const void *rope_table,
                                                float softmax_scale, float *out,
                                                int32_t n_splits, hipStream_t stream) {
  // Host-side checks first, so that an invalid or oversized call touches no
  // device state.
  lla_status_t e = lla_store_check(store);
  if (e != LLA_OK) return e;
  if (store->variant != LLA_PER_HEAD) return LLA_E_VARIANT;
  if (!store->data || !q || !w_up_k_t || !w_up_v_t || !mu_k_t || !mu_v_t || !pos ||
      !rope_table || !out)
    return LLA_E_NULL;
  if (n_splits < 0 || n_splits > store->max_ctx) return LLA_E_RANGE;
  const size_t need = lla_decode_workspace_bytes(store, n_splits);
  if (need == 0) return LLA_E_OVERFLOW;
  if (need > LLA_NOALLOC_SCRATCH_BYTES) return LLA_E_SCRATCH;
  void *ws = nullptr;
  e = current_scratch(&ws);
  if (e != LLA_OK) return e;
  e = lla_decode_attn(store, layer, loop, q, w_up_k_t, w_up_v_t, mu_k_t, mu_v_t, pos,
                      rope_table, softmax_scale, out, ws, LLA_NOALLOC_SCRATCH_BYTES, n_splits,
                      stream);
  // ws is non-null: a workspace error can only mean the scratch is too small
  // for the split count the call resolved to
  return e == LLA_E_WORKSPACE ? LLA_E_SCRATCH : e;
}
