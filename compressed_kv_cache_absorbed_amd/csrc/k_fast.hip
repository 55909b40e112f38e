// Matrix-core (MFMA) fast path: selection and launchers.
#include "device_util.hpp"

namespace mla {

bool decode_fast_path(const mla_dims &, const mla_cache &, mla_dtype) { return false; }
bool append_fast_path(const mla_dims &, int32_t, mla_dtype) { return false; }

hipError_t launch_append_fast(hipStream_t, const mla_dims &, const mla_cache &, const void *, int32_t,
                              const void *, const void *, float *, int, int32_t *) {
  return hipErrorNotSupported;
}
hipError_t launch_absorb_fast(hipStream_t, const mla_dims &, int32_t, const void *, const void *,
                              const int32_t *, const void *, const SeqInfo *, uint16_t *) {
  return hipErrorNotSupported;
}
hipError_t launch_decode_fast(hipStream_t, const mla_dims &, const mla_cache &, int32_t, const WorkItem *,
                              const SeqInfo *, const uint16_t *, float *, float *, int32_t *) {
  return hipErrorNotSupported;
}
hipError_t launch_combine_fast(hipStream_t, const mla_dims &, const mla_cache &, const SeqInfo *,
                               const float *, const float *, const void *, void *, mla_dtype) {
  return hipErrorNotSupported;
}

}  // namespace mla
