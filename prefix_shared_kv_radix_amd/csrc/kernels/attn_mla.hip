// MLA decode (one latent KV head, 576-dim keys whose first 512 dims are the values).
#include <hip/hip_runtime.h>

#include "host/radix_host.hpp"
#include "radix_attn.h"

extern "C" radix_status radix_mla_decode_impl(const radix_attn_shape *, const radix_kv_buffers *,
                                              const void *, const int32_t *, int32_t,
                                              const int32_t *, const int32_t *, int32_t, int32_t,
                                              const radix_decode_plan *, int32_t, void *, float *,
                                              float *, float *, int32_t, hipStream_t) {
  radix::set_error("MLA decode not built yet");
  return RADIX_E_UNSUPPORTED;
}
