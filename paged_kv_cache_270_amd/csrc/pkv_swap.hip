// pkv_swap.hip — gfx950 kernel of libpkv's swap space: whole blocks copied
// between the device pools and pinned host memory, for page-granular
// eviction ([KV-SLOW] "KV Cache y PagedAttention: por qué se reduce la
// velocidad de tu servidor LLM", "Cómo PagedAttention soluciona esto": when
// memory runs out, single pages move to CPU memory instead of whole
// sequences).  The host pool decides which blocks move (pkv_seq_swap_out /
// pkv_seq_swap_in); this file only copies them.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <initializer_list>

#include "pkv.h"
#include "pkv_check.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One workgroup per pair: copy one block (every KV head, K and V) between a
// device pool and the host buffers the device addresses directly, in 16-byte
// accesses.  Pairs with an id out of range are skipped.
__global__ void __launch_bounds__(256)
swap_blocks_kernel(u32x4* __restrict__ k_pool, u32x4* __restrict__ v_pool,
                   u32x4* __restrict__ host_k, u32x4* __restrict__ host_v,
                   const int32_t* __restrict__ pairs, int64_t vecs_per_block, int num_blocks,
                   int num_host, int to_host) {
  const int i = blockIdx.x;
  const int a = pairs[2 * i], b = pairs[2 * i + 1];
  const int dev = to_host ? a : b, host = to_host ? b : a;
  if (dev < 0 || dev >= num_blocks || host < 0 || host >= num_host) return;
  u32x4* dk = k_pool + (int64_t)dev * vecs_per_block;
  u32x4* dv = v_pool + (int64_t)dev * vecs_per_block;
  u32x4* hk = host_k + (int64_t)host * vecs_per_block;
  u32x4* hv = host_v + (int64_t)host * vecs_per_block;
  if (to_host) {
    for (int64_t v = threadIdx.x; v < vecs_per_block; v += 256) {
      hk[v] = dk[v];
      hv[v] = dv[v];
    }
  } else {
    for (int64_t v = threadIdx.x; v < vecs_per_block; v += 256) {
      dk[v] = hk[v];
      dv[v] = hv[v];
    }
  }
}

using namespace pkv_check;

bool aligned16(const void* p) { return aligned(p, 16); }

}  // namespace

extern "C" pkv_status pkv_swap_blocks(void* k_pool, void* v_pool, void* host_k, void* host_v,
                                      int32_t num_host_blocks, const pkv_cache_layout* layout,
                                      const int32_t* pairs, int32_t num_pairs, int32_t to_host,
                                      void* stream) {
  const pkv_status st = check_layout(layout);
  if (st != PKV_OK) return st;
  if (num_pairs < 0 || num_host_blocks < 0 || (to_host != 0 && to_host != 1))
    return PKV_ERR_INVALID_ARG;
  if (num_pairs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !host_k || !host_v || !pairs || !aligned16(k_pool) ||
      !aligned16(v_pool) || !aligned16(host_k) || !aligned16(host_v) ||
      ((uintptr_t)pairs % 4) != 0)
    return PKV_ERR_INVALID_ARG;
  const int64_t bytes = (int64_t)layout->num_kv_heads * 16 * 128 * elem_bytes(layout->dtype);
  // the device's address of each host buffer; memory that is not pinned host
  // memory the device can reach is refused here rather than faulted on
  (void)hipGetLastError();
  for (void* h : {host_k, host_v}) {
    hipPointerAttribute_t attr{};
    if (hipPointerGetAttributes(&attr, h) != hipSuccess || attr.type != hipMemoryTypeHost) {
      (void)hipGetLastError();
      return PKV_ERR_INVALID_ARG;  // pageable or device memory
    }
  }
  void* dk = nullptr;
  void* dv = nullptr;
  if (hipHostGetDevicePointer(&dk, host_k, 0) != hipSuccess ||
      hipHostGetDevicePointer(&dv, host_v, 0) != hipSuccess || !dk || !dv ||
      !aligned16(dk) || !aligned16(dv)) {
    (void)hipGetLastError();
    return PKV_ERR_INVALID_ARG;
  }
  swap_blocks_kernel<<<dim3((unsigned)num_pairs), dim3(256), 0,
                       static_cast<hipStream_t>(stream)>>>(
      static_cast<u32x4*>(k_pool), static_cast<u32x4*>(v_pool), static_cast<u32x4*>(dk),
      static_cast<u32x4*>(dv), pairs, bytes / 16, layout->num_blocks, num_host_blocks, to_host);
  return launch_status();
}
