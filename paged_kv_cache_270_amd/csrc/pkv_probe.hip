// pkv_probe.hip — memory ceilings the decode kernel is measured against (gfx950).
//
// "LLM Primer VI, Capítulo 8 — Gestión de caché KV de nueva generación" §8.1
// compares a paged attention kernel with one that reads a contiguous slab:
// on a GPU whose L2 absorbs the scattered accesses the paged kernel comes
// within a few percent.  Two reads give the two sides of that comparison on
// this part, without any attention arithmetic:
//   * pkv_hbm_read_probe: a contiguous buffer streamed once, 16 bytes per
//     lane per load, non-temporal -- the streaming-read ceiling;
//   * pkv_hbm_mix_probe: one or two contiguous source planes streamed into a
//     destination, non-temporal both ways -- the ceiling for a write with the
//     cache write's mix of reads and writes (fp16 rows in, FP8 rows out: two
//     bytes read per byte written);
//   * pkv_tile_gather_probe: the decode kernel's own reads -- every K and V
//     tile of every sequence, gathered through the block table with the same
//     16-byte lane loads and cache policy, one workgroup of four waves per
//     256 blocks of a (sequence, KV head), two tiles in flight per wave.
// Both fold what they read into one word per lane and store it only when it
// equals a value the host passes and the data never produces in practice,
// so the loads cannot be dropped and nothing measurable is written.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "pkv.h"
#include "pkv_check.h"
#include "pkv_tile.h"

namespace {

using namespace pkv_dev;
using namespace pkv_check;

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;   // 16-byte loads in flight per lane
constexpr uint64_t kStepVecs = (uint64_t)kProbeThreads * kProbeUnroll;  // 32 KiB per step

// Workgroup i streams its own contiguous slab of the buffer in steps of
// 32 KiB: each wave instruction covers 1 KiB of consecutive bytes, and a lane
// keeps eight 16-byte loads in flight.
__global__ void __launch_bounds__(kProbeThreads)
stream_read_kernel(const u32x4* __restrict__ buf, uint64_t n_vec, uint64_t slab_vecs,
                   uint32_t* sink, uint32_t key) {
  const uint64_t begin = (uint64_t)blockIdx.x * slab_vecs;
  const uint64_t end = begin + slab_vecs < n_vec ? begin + slab_vecs : n_vec;
  uint32_t acc = 0;
  uint64_t i = begin;
  for (; i + kStepVecs <= end; i += kStepVecs) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u)
      v[u] = __builtin_nontemporal_load(buf + i + u * kProbeThreads + threadIdx.x);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (uint64_t j = i + threadIdx.x; j < end; j += kProbeThreads) {
    const u32x4 v = __builtin_nontemporal_load(buf + j);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == key) sink[0] = acc;
}

// Workgroup i streams its own slab of the destination in 32 KiB steps and
// the same slab of each of the kPlanes source planes (plane p starts n_vec
// vectors after plane p - 1): kPlanes bytes read per byte written, every load
// and store non-temporal, eight 16-byte vectors in flight per lane and plane.
template <int kPlanes>
__global__ void __launch_bounds__(kProbeThreads)
stream_mix_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, uint64_t n_vec,
                  uint64_t slab_vecs) {
  const uint64_t begin = (uint64_t)blockIdx.x * slab_vecs;
  const uint64_t end = begin + slab_vecs < n_vec ? begin + slab_vecs : n_vec;
  uint64_t i = begin;
  for (; i + kStepVecs <= end; i += kStepVecs) {
    u32x4 v[kPlanes][kProbeUnroll];
#pragma unroll
    for (int p = 0; p < kPlanes; ++p)
#pragma unroll
      for (int u = 0; u < kProbeUnroll; ++u)
        v[p][u] = __builtin_nontemporal_load(src + p * n_vec + i + u * kProbeThreads +
                                             threadIdx.x);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      u32x4 r = v[0][u];
#pragma unroll
      for (int p = 1; p < kPlanes; ++p) r ^= v[p][u];
      __builtin_nontemporal_store(r, dst + i + u * kProbeThreads + threadIdx.x);
    }
  }
  for (uint64_t j = i + threadIdx.x; j < end; j += kProbeThreads) {
    u32x4 r = __builtin_nontemporal_load(src + j);
#pragma unroll
    for (int p = 1; p < kPlanes; ++p) r ^= __builtin_nontemporal_load(src + p * n_vec + j);
    __builtin_nontemporal_store(r, dst + j);
  }
}

// Whole 32 KiB steps per slab, one slab per workgroup (0 = 2048 workgroups).
void stream_slabs(uint64_t n_vec, int32_t workgroups, uint64_t* wg_out, uint64_t* slab_out) {
  const uint64_t steps = (n_vec + kStepVecs - 1) / kStepVecs;
  uint64_t wg = workgroups > 0 ? (uint64_t)workgroups : 2048;
  if (wg > steps) wg = steps;
  const uint64_t slab = (steps + wg - 1) / wg * kStepVecs;
  *wg_out = (n_vec + slab - 1) / slab;
  *slab_out = slab;
}

struct GatherArgs {
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t max_blocks, num_blocks, hkv, max_ctx;
  uint32_t* sink;
  uint32_t key;
};

// Workgroup (c, kvh, b) reads blocks [256c, 256c + 256) of sequence b for KV
// head kvh; wave w takes blocks w, w + 4, ... of them.
constexpr int kGatherBlocks = 256;

template <bool kFP8>
__global__ void __launch_bounds__(4 * kWave) tile_gather_kernel(GatherArgs a) {
  constexpr int kPD = 2;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int kvh = blockIdx.y, b = blockIdx.z;
  int L = a.context_lens[b];
  const int cap = min(a.max_ctx, a.max_blocks * kBS);
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int blk0 = blockIdx.x * kGatherBlocks;
  const int nblk = min((L + kBS - 1) / kBS - blk0, kGatherBlocks);
  const int my_n = w < nblk ? (nblk - w + 3) / 4 : 0;
  const int32_t* trow = a.block_tables + (int64_t)b * a.max_blocks + blk0 + w;
  uint32_t acc = 0;
  for (int c0 = 0; c0 < my_n; c0 += kWave) {
    const int cnt = min(kWave, my_n - c0);
    const int tbl = load_table(trow + (int64_t)c0 * 4, cnt, 4, lane);
    // every tile slot issues its loads (zeros past the end), as the decode
    // kernels do, so a wait never covers the loads issued after it
    TileRegs<kFP8> buf[kPD];
#pragma unroll
    for (int r = 0; r < kPD; ++r)
      load_tile<kFP8, kLoadNT>(buf[r], a.k_pool, a.v_pool, a.num_blocks, a.hkv,
                               r < cnt ? __builtin_amdgcn_readlane(tbl, r) : -1, kvh, lane);
    for (int base = 0; base < cnt; base += kPD) {
#pragma unroll
      for (int r = 0; r < kPD; ++r) {
        const int ii = base + r;
#pragma unroll
        for (int v = 0; v < TileRegs<kFP8>::kVecs; ++v)
          acc ^= buf[r].k[v].x ^ buf[r].k[v].w ^ buf[r].v[v].y ^ buf[r].v[v].z;
        const int nx = ii + kPD;
        load_tile<kFP8, kLoadNT>(buf[r], a.k_pool, a.v_pool, a.num_blocks, a.hkv,
                                 nx < cnt ? __builtin_amdgcn_readlane(tbl, nx) : -1, kvh, lane);
      }
    }
  }
  if (acc == a.key) a.sink[0] = acc;
}

}  // namespace

extern "C" pkv_status pkv_hbm_read_probe(const void* buf, uint64_t bytes, int32_t workgroups,
                                         uint32_t* sink, uint32_t key, void* stream) {
  if (bytes == 0) return PKV_OK;
  if (!buf || !sink || !aligned(buf, 16) || bytes % 16 != 0 || workgroups < 0)
    return PKV_ERR_INVALID_ARG;
  const uint64_t n_vec = bytes / 16;
  uint64_t wg = 0, slab = 0;
  stream_slabs(n_vec, workgroups, &wg, &slab);
  (void)hipGetLastError();
  stream_read_kernel<<<(unsigned)wg, kProbeThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4*>(buf), n_vec, slab, sink, key);
  return launch_status();
}

extern "C" pkv_status pkv_hbm_mix_probe(const void* src, void* dst, uint64_t dst_bytes,
                                        int32_t reads_per_write, int32_t workgroups,
                                        void* stream) {
  if (dst_bytes == 0) return PKV_OK;
  if (!src || !dst || !aligned(src, 16) || !aligned(dst, 16) || dst_bytes % 16 != 0 ||
      workgroups < 0 || reads_per_write < 1 || reads_per_write > 2)
    return PKV_ERR_INVALID_ARG;
  const uint64_t n_vec = dst_bytes / 16;
  uint64_t wg = 0, slab = 0;
  stream_slabs(n_vec, workgroups, &wg, &slab);
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* d = static_cast<u32x4*>(dst);
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (reads_per_write == 1)
    stream_mix_kernel<1><<<(unsigned)wg, kProbeThreads, 0, st>>>(s, d, n_vec, slab);
  else
    stream_mix_kernel<2><<<(unsigned)wg, kProbeThreads, 0, st>>>(s, d, n_vec, slab);
  return launch_status();
}

extern "C" pkv_status pkv_tile_gather_probe(const void* k_pool, const void* v_pool,
                                            const int32_t* block_tables,
                                            int32_t max_blocks_per_seq,
                                            const int32_t* context_lens, int32_t num_seqs,
                                            int32_t max_context_len,
                                            const pkv_cache_layout* layout, uint32_t* sink,
                                            uint32_t key, void* stream) {
  pkv_status st = check_layout(layout);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || num_seqs > 65535 || max_context_len < 0) return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !block_tables || !context_lens || !sink ||
      max_blocks_per_seq <= 0 || !aligned(k_pool, 16) || !aligned(v_pool, 16))
    return PKV_ERR_INVALID_ARG;
  GatherArgs a;
  a.k_pool = static_cast<const uint8_t*>(k_pool);
  a.v_pool = static_cast<const uint8_t*>(v_pool);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = layout->num_blocks;
  a.hkv = layout->num_kv_heads;
  a.max_ctx = max_context_len;
  a.sink = sink;
  a.key = key;
  const int64_t max_nblk = ((int64_t)max_context_len + kBS - 1) / kBS;
  const int64_t chunks = std::max<int64_t>(1, (max_nblk + kGatherBlocks - 1) / kGatherBlocks);
  const dim3 grid((unsigned)chunks, (unsigned)a.hkv, (unsigned)num_seqs);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (layout->dtype == PKV_FP8_E4M3FN)
    tile_gather_kernel<true><<<grid, 4 * kWave, 0, s>>>(a);
  else
    tile_gather_kernel<false><<<grid, 4 * kWave, 0, s>>>(a);
  return launch_status();
}
