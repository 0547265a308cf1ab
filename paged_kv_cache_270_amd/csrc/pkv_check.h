// pkv_check.h — host-side argument checks shared by libpkv's kernel sources.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

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

// The debug path of the table checks (pkv_set_debug_checks): copy the device
// block table and lengths to the host, waiting for `s`, and validate them.
// Without the switch nothing is copied.
inline pkv_status debug_check_tables(const int32_t* block_tables, int32_t max_blocks,
                                     const int32_t* context_lens, int32_t num_seqs,
                                     int32_t max_ctx, int32_t num_blocks, hipStream_t s) {
  if (num_seqs <= 0 || !pkv_get_debug_checks()) return PKV_OK;
  std::vector<int32_t> tables((size_t)num_seqs * (size_t)max_blocks), lens((size_t)num_seqs);
  if (hipMemcpyAsync(tables.data(), block_tables, tables.size() * sizeof(int32_t),
                     hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipMemcpyAsync(lens.data(), context_lens, lens.size() * sizeof(int32_t),
                     hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return PKV_ERR_HIP;
  return pkv_validate_tables(tables.data(), max_blocks, lens.data(), num_seqs, max_ctx,
                             num_blocks, nullptr);
}

}  // namespace pkv_check
