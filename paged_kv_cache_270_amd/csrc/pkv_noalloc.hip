// pkv_noalloc.hip — the decode step for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc): pkv_paged_attention_decode_append with its split-KV
// workspace taken from `scratch`, a fixed array this library holds on every
// device it runs on, instead of from the caller.
//
// The same kernels run as for the workspace entry point; the partials (max,
// sum, unnormalised output per sequence, query head and partition) are
// written by the partition kernel before the merge kernel reads them within
// the same call, so nothing in the array needs clearing between calls.
// Calls that overlap in time on one device share the array and race.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "pkv.h"

static_assert(PKV_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");

// One copy per device, kept until the process ends.  In host code `scratch`
// names a host-side stand-in, not the device array: its device address comes
// from hipGetSymbolAddress (scratch_base below).
static __device__ __align__(256) uint8_t scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up once per
// device; null if the lookup fails.
void* scratch_base() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  static std::mutex mu;
  static void* base[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (base[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return nullptr;
    base[dev] = p;
  }
  return base[dev];
}

}  // namespace

extern "C" pkv_status pkv_paged_attention_decode_append_noalloc(
    float* out, const void* q, const void* key, const void* value, void* k_pool, void* v_pool,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* shared_prefix_blocks, int32_t num_seqs, int32_t num_q_heads,
    int32_t max_context_len, const pkv_cache_layout* layout, float sm_scale, float k_scale,
    float v_scale, int32_t partition_size, void* stream) {
  if (!layout) return PKV_ERR_INVALID_ARG;
  // the workspace the shape needs (0: no merge, or arguments the decode call
  // below rejects itself)
  uint64_t need = 0;
  if (num_seqs > 0 && layout->num_kv_heads > 0)
    need = pkv_decode_workspace_bytes(num_seqs, num_q_heads, layout->num_kv_heads,
                                      max_context_len, layout->dtype, partition_size);
  if (need > PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_base();
    if (ws == nullptr) return PKV_ERR_HIP;
  }
  return pkv_paged_attention_decode_append(
      out, q, key, value, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens,
      shared_prefix_blocks, num_seqs, num_q_heads, max_context_len, layout, sm_scale, k_scale,
      v_scale, partition_size, ws, need > 0 ? PKV_NOALLOC_SCRATCH_BYTES : 0, stream);
}
