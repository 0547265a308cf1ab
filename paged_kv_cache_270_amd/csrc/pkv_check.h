// pkv_check.h — host-side argument checks shared by libpkv's kernel sources.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv.h"

namespace pkv_check {

inline bool aligned(const void* p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }

// Bytes per cached element, 0 for an unknown dtype.
inline int elem_bytes(int32_t dtype) {
  return dtype == PKV_F16 ? 2 : (dtype == PKV_FP8_E4M3FN ? 1 : 0);
}

// A layout the kernels support: 16-token blocks, head dim 128, fp16 or FP8.
inline pkv_status check_layout(const pkv_cache_layout* l) {
  if (!l) return PKV_ERR_INVALID_ARG;
  if (l->block_size != 16 || l->head_dim != 128 || elem_bytes(l->dtype) == 0)
    return PKV_ERR_UNSUPPORTED;
  if (l->num_blocks <= 0 || l->num_kv_heads <= 0 || l->num_kv_heads > 65535)
    return PKV_ERR_INVALID_ARG;
  return PKV_OK;
}

// Status of the launches since the last (void)hipGetLastError().
inline pkv_status launch_status() {
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace pkv_check
