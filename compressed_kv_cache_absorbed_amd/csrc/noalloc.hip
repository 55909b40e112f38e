// mla_decode_noalloc: mla_decode for callers that cannot allocate device
// memory (code under graph capture, tight serving loops, harnesses that
// forbid allocation). Its workspace is `scratch`, a file-scope device array
// of MLA_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until
// the process ends; the call itself allocates nothing.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is fetched once per device with hipGetSymbolAddress, with
// that device current, and only that address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mla_internal.hpp"

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[MLA_NOALLOC_SCRATCH_BYTES];

std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};

// The current device's address of scratch (fetched on the first call made
// with that device current).
mla_status scratch_on_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> g(g_mu);
  if (g_scratch[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return MLA_ERR_HIP;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MLA_OK;
}

}  // namespace

extern "C" mla_status mla_decode_noalloc(const mla_dims *dims, const mla_cache *cache, const mla_plan *plan,
                                         const void *q_nope, const void *q_rope, const int32_t *q_pos,
                                         const void *w_uk, const void *w_uv, mla_dtype q_w_dtype, void *o,
                                         mla_dtype o_dtype, int32_t *dev_status, void *stream) {
  // the arguments as mla_decode checks them, with the scratch array in the
  // workspace's place (any non-null, aligned address passes the check)
  alignas(256) static char placeholder;
  mla_status st = mla::decode_check_args(dims, cache, plan, q_nope, q_rope, w_uk, w_uv, q_w_dtype, o, o_dtype,
                                         &placeholder, ~static_cast<size_t>(0), 1);
  if (st != MLA_OK) return st;
  if (dev_status != nullptr && (reinterpret_cast<uintptr_t>(dev_status) & 3)) return MLA_ERR_INVALID_ARG;
  if (mla::decode_compact_bytes(*dims, *cache, *plan, q_w_dtype) > MLA_NOALLOC_SCRATCH_BYTES)
    return MLA_ERR_WORKSPACE;
  void *ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != MLA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = mla::decode_launch(dims, cache, plan, q_nope, q_rope, q_pos, w_uk, w_uv, q_w_dtype, o, o_dtype, ws, s, 1,
                          true, true);
  if (st != MLA_OK) return st;
  if (dev_status != nullptr && mla::launch_status_copy(s, static_cast<const int32_t *>(ws), dev_status) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}
