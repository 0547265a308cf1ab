// pkv_write.hip — gfx950 kernels that write the paged cache, and their part
// of libpkv's C ABI: reshape_and_cache (fp16, or FP8 E4M3 with a per-tensor
// scale), the same write with per-block dynamic FP8 scales, and the block
// copies behind copy-on-write.
//
// Pages the kernels follow (cited by title and section):
//   [FP8-128K] "Optimización de KV Cache con PagedAttention y Cuantización FP8
//              para Contextos Largos (128K)"
//   [PRIMER-8] "LLM Primer VI, Capítulo 8 — Gestión de caché KV de nueva
//              generación"
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "pkv.h"
#include "pkv_check.h"
#include "pkv_codec.h"
#include "pkv_tile.h"

namespace {

using namespace pkv_dev;
using namespace pkv_check;

// ------------------------------------------------------ reshape_and_cache

// Store channels 8c .. 8c+7 of one token's K and V rows (16 bytes of fp16
// each) at position t of tile `tile` (= block * hkv + head).
template <bool kFP8>
__device__ __forceinline__ void store_rows8(uint8_t* __restrict__ k_pool,
                                            uint8_t* __restrict__ v_pool, int64_t tile, int t,
                                            int c, u32x4 kin, u32x4 vin, float k_scale,
                                            float v_scale) {
  const int n = c >> 1;                   // 16-channel group of these channels
  const int j0 = (c & 1) * 8;             // channel within the group
  if constexpr (!kFP8) {
    uint16_t* kp = reinterpret_cast<uint16_t*>(k_pool) + tile * (kBS * kD);
    uint16_t* vp = reinterpret_cast<uint16_t*>(v_pool) + tile * (kBS * kD);
    // K, x = 8: (d/8)*128 + t*8 + d%8 -> the 8 channels are contiguous
    *reinterpret_cast<u32x4*>(kp + c * 128 + t * 8) = kin;
    // V, x = 8: (n/2)*512 + ((t/4)*16 + d%16)*8 + (n%2)*4 + t%4
    const uint16_t* vh = reinterpret_cast<const uint16_t*>(&vin);
    uint16_t* vb = vp + (n >> 1) * 512 + ((t >> 2) * 16 + j0) * 8 + (n & 1) * 4 + (t & 3);
#pragma unroll
    for (int i = 0; i < 8; ++i) vb[i * 8] = vh[i];
  } else {
    uint8_t* kp = k_pool + tile * (kBS * kD);
    uint8_t* vp = v_pool + tile * (kBS * kD);
    const _Float16* kh = reinterpret_cast<const _Float16*>(&kin);
    const _Float16* vh = reinterpret_cast<const _Float16*>(&vin);
    // x / scale rounded as fp32 division rounds it (one division per scale)
    const ScaleDiv kd = scale_div(k_scale), vd = scale_div(v_scale);
    uint32_t kc[8], vc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      kc[i] = e4m3_from_f32(div_by((float)kh[i], kd));
      vc[i] = e4m3_from_f32(div_by((float)vh[i], vd));
    }
    // K, x = 16: (d/16)*256 + t*16 + d%16 -> 8 contiguous bytes
    u32x2 kw;
    kw.x = kc[0] | (kc[1] << 8) | (kc[2] << 16) | (kc[3] << 24);
    kw.y = kc[4] | (kc[5] << 8) | (kc[6] << 16) | (kc[7] << 24);
    *reinterpret_cast<u32x2*>(kp + n * 256 + t * 16 + j0) = kw;
    // V, x = 16: (n/4)*1024 + ((t/4)*16 + d%16)*16 + (n%4)*4 + t%4
    uint8_t* vb = vp + (n >> 2) * 1024 + ((t >> 2) * 16 + j0) * 16 + (n & 3) * 4 + (t & 3);
#pragma unroll
    for (int i = 0; i < 8; ++i) vb[i * 16] = (uint8_t)vc[i];
  }
}

// One thread per (token, kv head, run of 8 channels): 16 bytes of fp16 in.
// For calls of few tokens (a decode step) -- the most parallel form.  The
// row loads do not depend on the slot, so all three loads are in flight at
// once (the call is latency-bound).
template <bool kFP8>
__global__ void __launch_bounds__(256)
reshape_rows_kernel(const u32x4* __restrict__ key, const u32x4* __restrict__ value,
                    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
                    const int64_t* __restrict__ slots, uint32_t total, uint32_t hkv,
                    int64_t num_slots, float k_scale, float v_scale) {
  const uint32_t gid = blockIdx.x * 256u + threadIdx.x;  // total < 2^31 (checked on the host)
  if (gid >= total) return;
  const int c = (int)(gid & 15);          // channels 8c .. 8c+7
  const uint32_t th = gid >> 4;           // token * hkv + head
  const uint32_t tok = th / hkv;
  const int h = (int)(th - tok * hkv);
  const u32x4 kin = key[th * 16 + c];
  const u32x4 vin = value[th * 16 + c];
  const int64_t slot = slots[tok];
  asm volatile("" ::"v"(kin), "v"(vin));  // keeps the row loads ahead of the slot test
  if (slot < 0 || slot >= num_slots) return;
  store_rows8<kFP8>(k_pool, v_pool, (slot >> 4) * hkv + h, (int)(slot & 15), c, kin, vin,
                    k_scale, v_scale);
}

// Calls of at most this many tokens use the row kernel; longer ones (bulk
// fills, prefill chunks) the tile-building kernel below.
constexpr int64_t kRowWriteMaxTokens = 512;

// Largest finite magnitude among 8 fp16 values, as fp16 bits (integer order
// of non-negative fp16 bit patterns is their numeric order).
__device__ __forceinline__ uint32_t max_abs_bits8(u32x4 x) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = x[i];
    const uint32_t lo = w & 0x7FFFu, hi = (w >> 16) & 0x7FFFu;
    if (lo < 0x7C00u) m = max(m, lo);
    if (hi < 0x7C00u) m = max(m, hi);
  }
  return m;
}

__device__ __forceinline__ float f16_bits_to_float(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// A block the call fills whole under per-block scales (the tile-building
// kernel's dynamic mode) is marked in the write's scratch (bit 31 of its
// written-offsets word): the MaxAbs and encode launches then leave it alone.
constexpr uint32_t kWholeBlock = 0x80000000u | 0xFFFFu;

// Lane (q, c) holds channels 8c .. 8c+7 of tokens 4q .. 4q+3 of a group in
// r[0..3]; afterwards it holds those of tokens 4q + d .. 4q + d + 3, the rows
// of tokens tf + 4q .. tf + 4q + 3 (tf: the group's first token + d).  Rows
// of the group pass through LDS; those past it are read from `src`.
__device__ __forceinline__ void shift_rows(u32x4 (&r)[4], const u32x4* __restrict__ src,
                                           uint8_t* lo, uint8_t* hi, int64_t tf, int hkv,
                                           int h, int q, int c, int d) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int t = 4 * q + k;
    *reinterpret_cast<u32x4*>((t < 8 ? lo : hi) + (t & 7) * 256 + c * 16) = r[k];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int t = 4 * q + k + d;  // token of the group (t >= 16: of the next group)
    if (t < kBS)
      r[k] = *reinterpret_cast<const u32x4*>((t < 8 ? lo : hi) + (t & 7) * 256 + c * 16);
    else
      r[k] = __builtin_nontemporal_load(src + ((tf + 4 * q + k) * hkv + h) * 16 + c);
  }
  // the reads before the next writes to the same LDS
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wave per (group of 16 consecutive tokens of the call, KV head).  Each
// cache block whose 16 slots the call writes in order, from 16 consecutive
// tokens, is written by the wave whose group holds the block's first token:
// it builds the (block, head) tiles in LDS from coalesced loads of the 16
// rows and stores each tile as one contiguous run (2 KiB FP8 / 4 KiB fp16),
// so the scattered layout costs no partial-line writes.  In a bulk fill the
// groups are the blocks; in a batched prefill whose sequences are not
// multiples of 16 long each block starts inside a group and takes rows from
// the next.  Tokens of blocks the call only partly writes (a sequence's
// first and last blocks, a decode step's one token per sequence) are stored
// row by row by the wave of their own group.
constexpr int kFillWaves = 4;  // independent waves per workgroup

// Per-block scales (kDyn): the tiles' scales and the write's written-offsets
// scratch, where whole blocks are marked.
struct DynTiles {
  float* k_bscale;
  float* v_bscale;
  uint32_t* written;
};

template <bool kFP8, bool kDyn = false>
__global__ void __launch_bounds__(kFillWaves * kWave) __attribute__((amdgpu_waves_per_eu(kFP8 ? 4 : 1)))
reshape_and_cache_kernel(const u32x4* __restrict__ key, const u32x4* __restrict__ value,
                         uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
                         const int64_t* __restrict__ slots, int64_t num_tokens, int hkv,
                         int64_t num_slots, float k_scale, float v_scale, uint32_t units,
                         DynTiles dt) {
  static_assert(kFP8 || !kDyn, "per-block scales are for FP8 pools");
  constexpr int kTileBytes = kBS * kD * (kFP8 ? 1 : 2);
  __shared__ __align__(16) uint8_t lk_all[kFillWaves][kTileBytes];
  __shared__ __align__(16) uint8_t lv_all[kFillWaves][kTileBytes];
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  uint8_t* lk = lk_all[w];
  uint8_t* lv = lv_all[w];
  // one (16-token group, KV head) unit per wave; the head varies fastest:
  // neighbouring waves read neighbouring 256-byte parts of the same rows
  const uint32_t unit = blockIdx.x * kFillWaves + w;
  if (unit >= units) return;  // whole waves
  const int h = (int)(unit % (unsigned)hkv);
  const int64_t t0 = (int64_t)(unit / (unsigned)hkv) * kBS;
  const int ntok = (int)min<int64_t>(kBS, num_tokens - t0);
  // FP8: the group's own 16 rows -- the rows of its block when the group is
  // one whole block, as in every group of a bulk fill -- are requested with
  // the slots (their addresses do not depend on the slots), so such a block
  // costs one round trip to memory; each row is read once, past the caches.
  // Lane l takes channels 8c .. 8c+7, c = l % 16, of the four tokens
  // 4q .. 4q+3, q = l / 16 (each load instruction reads four whole rows).
  // fp16 loads its rows once the slots are known.
  u32x4 kin[4], vin[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (kFP8) {
      const int t = 4 * (lane >> 4) + j, c = lane & 15;
      if (t < ntok) {
        const int64_t th = (t0 + t) * hkv + h;
        kin[j] = __builtin_nontemporal_load(key + th * 16 + c);
        vin[j] = __builtin_nontemporal_load(value + th * 16 + c);
      } else {
        kin[j] = vin[j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  // the slots of tokens t0 - 16 .. t0 + 47 (lane l: token t0 - 16 + l); -1
  // outside the call
  const int64_t tl = t0 - kBS + lane;
  const int64_t sl = tl >= 0 && tl < num_tokens ? slots[tl] : -1;
  const bool valid = sl >= 0 && sl < num_slots;
  const int64_t s_next = __shfl_down(sl, 1, kWave);
  // bit l: token l + 1's slot follows token l's
  const uint64_t follows = __ballot(valid && lane < kWave - 1 && s_next == sl + 1);
  // bit l: a block starts at token l and the next 15 tokens fill it in order
  // (its last slot is then inside the pool as well)
  const uint64_t starts =
      __ballot(valid && (sl & (kBS - 1)) == 0 && lane <= kWave - kBS &&
               ((follows >> lane) & 0x7FFFull) == 0x7FFFull);
  // the group's tokens (lanes 16 .. 16 + ntok - 1) that no such block holds
  const bool mine = lane >= kBS && lane < kBS + ntok;
  const uint64_t near = lane >= kBS - 1 ? starts >> (lane - (kBS - 1)) : 0;  // starts l-15 .. l
  const uint64_t rows = __ballot(mine && valid && (near & 0xFFFFull) == 0);
  // (with per-block scales the three-launch write takes these tokens)
  if (!kDyn && rows) {
    // row by row: 16 runs of 8 channels per token
    for (int i = lane; i < ntok * 16; i += kWave) {
      if (!((rows >> (kBS + (i >> 4))) & 1)) continue;
      const int64_t tok = t0 + (i >> 4);
      const int c = i & 15;
      const int64_t slot = slots[tok];
      const int64_t th = tok * hkv + h;
      store_rows8<kFP8>(k_pool, v_pool, (slot >> 4) * hkv + h, (int)(slot & 15), c,
                        key[th * 16 + c], value[th * 16 + c], k_scale, v_scale);
    }
  }
  const uint64_t block = starts & (0xFFFFull << kBS);  // at most one start in the group
  if (!block) return;
  const int f = (int)__builtin_ctzll(block);
  const int64_t tf = t0 - kBS + f;                     // the block's first token
  const int64_t s0 = __shfl(sl, f, kWave);
  // whole block: place every element at its tile position in LDS
  if constexpr (kFP8) {
    const int q = lane >> 4, c = lane & 15;  // tokens 4q .. 4q+3, channels 8c .. 8c+7
    if (f != kBS) {
      // The block starts inside the group, d tokens in: its rows are the
      // group's last 16 - d rows, already loaded, then the next group's
      // first d.  K, then V, goes through the wave's LDS (rows 0-7 in lk,
      // 8-15 in lv, 256 bytes each) to move each kept row to the lane that
      // needs it; only the next group's rows are read from memory.
      const int d = f - kBS;
      shift_rows(kin, key, lk, lv, tf, hkv, h, q, c, d);
      shift_rows(vin, value, lk, lv, tf, hkv, h, q, c, d);
    }
    const int n = c >> 1, j0 = (c & 1) * 8;
    Fp8Enc ke, ve;
    if constexpr (kDyn) {
      // [FP8-128K] §8: the block is fresh (the call writes its offset 0), so
      // each tile's scale is max(fp32(MaxAbs of its finite values / 448),
      // 2^-126), as the three-launch write computes it
      uint32_t km = 0, vm = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        km = max(km, max_abs_bits8(kin[k]));
        vm = max(vm, max_abs_bits8(vin[k]));
      }
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        km = max(km, (uint32_t)__shfl_xor((int)km, m, kWave));
        vm = max(vm, (uint32_t)__shfl_xor((int)vm, m, kWave));
      }
      const float sk = fmaxf(f16_bits_to_float(km) / 448.0f, 0x1p-126f);
      const float sv = fmaxf(f16_bits_to_float(vm) / 448.0f, 0x1p-126f);
      ke = fp8_enc(sk);
      ve = fp8_enc(sv);
      if (lane == 0) {
        const int64_t tile = (s0 >> 4) * hkv + h;
        dt.k_bscale[tile] = sk;
        dt.v_bscale[tile] = sv;
        dt.written[s0 >> 4] = kWholeBlock;  // every head's wave stores the same word
      }
    } else {
      ke = fp8_enc(k_scale);
      ve = fp8_enc(v_scale);
    }
    uint32_t vc[2][4];  // V codes of channels 8c + 4i .. 8c + 4i + 3 of token 4q + k
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      u32x2 kw;
      kw.x = e4m3x4_from_f16x4(kin[k].x, kin[k].y, ke);
      kw.y = e4m3x4_from_f16x4(kin[k].z, kin[k].w, ke);
      // K, x = 16: (d/16)*256 + t*16 + d%16 -> 8 contiguous bytes
      *reinterpret_cast<u32x2*>(lk + n * 256 + (4 * q + k) * 16 + j0) = kw;
      vc[0][k] = e4m3x4_from_f16x4(vin[k].x, vin[k].y, ve);
      vc[1][k] = e4m3x4_from_f16x4(vin[k].z, vin[k].w, ve);
    }
    // V, x = 16: (n/4)*1024 + ((t/4)*16 + d%16)*16 + (n%4)*4 + t%4 -> the
    // codes of channel d for the four tokens 4q .. 4q+3 are one aligned
    // 4-byte word: transpose each 4 x 4 block of bytes (token x channel)
    uint8_t* vb = lv + (n >> 2) * 1024 + (q * 16 + j0) * 16 + (n & 3) * 4;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t* x = vc[i];
      const uint32_t p01_lo = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u);
      const uint32_t p01_hi = __builtin_amdgcn_perm(x[1], x[0], 0x07030602u);
      const uint32_t p23_lo = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);
      const uint32_t p23_hi = __builtin_amdgcn_perm(x[3], x[2], 0x07030602u);
      uint32_t* vw = reinterpret_cast<uint32_t*>(vb + 4 * i * 16);
      vw[0] = __builtin_amdgcn_perm(p23_lo, p01_lo, 0x05040100u);   // channel 8c + 4i
      vw[4] = __builtin_amdgcn_perm(p23_lo, p01_lo, 0x07060302u);   // + 1
      vw[8] = __builtin_amdgcn_perm(p23_hi, p01_hi, 0x05040100u);   // + 2
      vw[12] = __builtin_amdgcn_perm(p23_hi, p01_hi, 0x07060302u);  // + 3
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = lane + kWave * j;  // (token, run of 8 channels)
      const int t = i >> 4, c = i & 15;
      const int n = c >> 1, j0 = (c & 1) * 8;
      const int64_t th = (tf + t) * hkv + h;
      kin[j] = key[th * 16 + c];
      vin[j] = value[th * 16 + c];
      *reinterpret_cast<u32x4*>(lk + (c * 128 + t * 8) * 2) = kin[j];  // K: 16 contiguous bytes
      // V, x = 8: (n/2)*512 + ((t/4)*16 + d%16)*8 + (n%2)*4 + t%4
      const uint16_t* vh = reinterpret_cast<const uint16_t*>(&vin[j]);
      uint16_t* vb = reinterpret_cast<uint16_t*>(lv) + (n >> 1) * 512 +
                     ((t >> 2) * 16 + j0) * 8 + (n & 1) * 4 + (t & 3);
#pragma unroll
      for (int e = 0; e < 8; ++e) vb[e * 8] = vh[e];
    }
  }
  // the wave's own tiles: order its LDS writes before its reads
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int64_t tile = (s0 >> 4) * hkv + h;
  u32x4* kt = reinterpret_cast<u32x4*>(k_pool + tile * kTileBytes);
  u32x4* vt = reinterpret_cast<u32x4*>(v_pool + tile * kTileBytes);
  const u32x4* sk = reinterpret_cast<const u32x4*>(lk);
  const u32x4* sv = reinterpret_cast<const u32x4*>(lv);
  // the tiles are not read again by this call: stored past the caches
#pragma unroll
  for (int j = 0; j < kTileBytes / 16 / kWave; ++j) {
    __builtin_nontemporal_store(sk[lane + kWave * j], kt + lane + kWave * j);
    __builtin_nontemporal_store(sv[lane + kWave * j], vt + lane + kWave * j);
  }
}

// ------------------------------------------ write with per-block FP8 scales
//
// [FP8-128K] §8, dynamic scaling: each (block, KV head) tile of K and of V
// carries its own fp32 scale, following the MaxAbs of the values written
// into it.  Per call and per tile, with W the block's offsets this call
// writes: the block is fresh when offset 0 is in W (its old scale and other
// slots are disregarded); s_new = max(s_old or 0 if fresh, fp32(MaxAbs of
// the new finite values / 448), 2^-126); if a non-fresh tile's scale grows,
// its slots outside W are re-encoded as E4M3(fp32(value * fp32(s_old /
// s_new))); new rows are E4M3(fp32(x / s_new)).
//
// Three launches (one for calls of at most 64 tokens, dyn_write_small_kernel
// below), because the new scale of a block depends on every token the call
// writes into it; calls of more than 512 tokens first write the blocks they
// fill whole in the tile-building pass, which marks them, and the row passes
// skip those:
//   1. clear the scratch entries of the touched blocks;
//   2. MaxAbs of each new row into the scratch (integer atomic max of the
//      non-negative float bits) and the written offsets (atomic or);
//   3. every row is encoded with its tile's new scale; the call's token with
//      the lowest offset in a block re-encodes the other slots and stores the
//      new scales.  Any thread may read a tile's scale while that token
//      replaces it: both values give the same s_new, since s_new is the max.

// Value of an E4M3FN code (not NaN) as fp32, from the format definition.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float v = e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -v : v;
}

__device__ __forceinline__ uint32_t requant_code(uint32_t c, float r) {
  if ((c & 0x7Fu) == 0x7Fu) return c;  // NaN stays NaN
  return e4m3_from_f32(e4m3_value(c) * r);
}

// One thread per token.  A block's scratch entries need clearing once, by
// any of the call's tokens in it; a token clears them where it starts a run
// of consecutive slots (offset 0, or the previous token's slot not the one
// before its own).  Following any token's run back leads to such a token in
// the same block, and a bulk fill clears each block once instead of 16 times.
__global__ void __launch_bounds__(256)
dyn_clear_kernel(const int64_t* __restrict__ slots, int64_t num_tokens, int per_block,
                 int64_t num_slots, uint32_t* __restrict__ amax, uint32_t* __restrict__ written) {
  const int64_t tok = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (tok >= num_tokens) return;
  const int64_t slot = slots[tok];
  if (slot < 0 || slot >= num_slots) return;
  if ((slot & 15) != 0 && tok > 0 && slots[tok - 1] == slot - 1) return;
  const int64_t blk = slot >> 4;
  for (int j = 0; j < per_block; ++j) amax[blk * per_block + j] = 0u;
  written[blk] = 0u;
}

// MaxAbs of one (token th / hkv, kv head h) row into the scratch: 16
// consecutive lanes, lane c a run of 8 channels, as the plain write.
__device__ __forceinline__ void amax_row(const u32x4* __restrict__ key,
                                         const u32x4* __restrict__ value, int64_t th, int h,
                                         int64_t slot, int c, int hkv, uint32_t* __restrict__ amax,
                                         uint32_t* __restrict__ written) {
  uint32_t km = max_abs_bits8(key[th * 16 + c]);
  uint32_t vm = max_abs_bits8(value[th * 16 + c]);
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) {
    km = max(km, (uint32_t)__shfl_xor((int)km, m, kWave));
    vm = max(vm, (uint32_t)__shfl_xor((int)vm, m, kWave));
  }
  if (c == 0) {
    const int64_t blk = slot >> 4;
    uint32_t* a = amax + (blk * hkv + h) * 2;
    atomicMax(a, __float_as_uint(f16_bits_to_float(km)));
    atomicMax(a + 1, __float_as_uint(f16_bits_to_float(vm)));
    if (h == 0) atomicOr(written + blk, 1u << (slot & 15));
  }
}

// Rows of calls of up to kDynManyRows rows: one 16-lane group per row.
// Larger calls (bulk fills, long prefill chunks) go through dyn_by_token
// below.
__global__ void __launch_bounds__(256)
dyn_amax_kernel(const u32x4* __restrict__ key, const u32x4* __restrict__ value,
                const int64_t* __restrict__ slots, int64_t total, int hkv, int64_t num_slots,
                uint32_t* __restrict__ amax, uint32_t* __restrict__ written) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total) return;                  // total is a multiple of 16: whole rows leave
  const int c = (int)(gid & 15);
  const int64_t th = gid >> 4;
  const int64_t tok = th / hkv;
  const int h = (int)(th - tok * hkv);
  const int64_t slot = slots[tok];
  if (slot < 0 || slot >= num_slots) return;  // the same for all 16 lanes of the row
  if (written[slot >> 4] & 0x80000000u) return;  // a whole block, already written
  amax_row(key, value, th, h, slot, c, hkv, amax, written);
}

// Re-encode channels 8c .. 8c+7 of every slot of one FP8 tile outside `keep`.
__device__ __forceinline__ void requant_k_rows(uint8_t* kp, int c, uint32_t keep, float r) {
  const int n = c >> 1, j0 = (c & 1) * 8;
  for (int t = 0; t < kBS; ++t) {
    if (keep & (1u << t)) continue;
    u32x2* p = reinterpret_cast<u32x2*>(kp + n * 256 + t * 16 + j0);  // K: 8 contiguous bytes
    u32x2 w = *p;
    uint32_t o[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t x = w[i];
      o[i] = requant_code(x & 0xFFu, r) | (requant_code((x >> 8) & 0xFFu, r) << 8) |
             (requant_code((x >> 16) & 0xFFu, r) << 16) | (requant_code(x >> 24, r) << 24);
    }
    w.x = o[0];
    w.y = o[1];
    *p = w;
  }
}

__device__ __forceinline__ void requant_v_rows(uint8_t* vp, int c, uint32_t keep, float r) {
  const int n = c >> 1, j0 = (c & 1) * 8;
  for (int t = 0; t < kBS; ++t) {
    if (keep & (1u << t)) continue;
    uint8_t* vb = vp + (n >> 2) * 1024 + ((t >> 2) * 16 + j0) * 16 + (n & 3) * 4 + (t & 3);
#pragma unroll
    for (int i = 0; i < 8; ++i) vb[i * 16] = (uint8_t)requant_code(vb[i * 16], r);
  }
}

// Encode one row with its tile's new scale; the call's token with the
// lowest offset in the block re-encodes the other slots and stores the new
// scales.  mask: the block's mark (bit t: offset t written by this call).
__device__ __forceinline__ void write_row(const u32x4* __restrict__ key,
                                          const u32x4* __restrict__ value,
                                          uint8_t* __restrict__ k_pool,
                                          uint8_t* __restrict__ v_pool,
                                          float* __restrict__ k_bscale,
                                          float* __restrict__ v_bscale, int64_t th, int h,
                                          int64_t slot, uint32_t mask, int c, int hkv,
                                          const uint32_t* __restrict__ amax) {
  const int64_t blk = slot >> 4;
  const int off = (int)(slot & 15);
  const int64_t tile = blk * hkv + h;
  const bool fresh = (mask & 1u) != 0;
  const float min_scale = 0x1p-126f;
  const float sk_old = fresh ? 0.0f : k_bscale[tile];
  const float sv_old = fresh ? 0.0f : v_bscale[tile];
  const float sk = fmaxf(fmaxf(sk_old, __uint_as_float(amax[tile * 2]) / 448.0f), min_scale);
  const float sv = fmaxf(fmaxf(sv_old, __uint_as_float(amax[tile * 2 + 1]) / 448.0f), min_scale);
  store_rows8<true>(k_pool, v_pool, tile, off, c, key[th * 16 + c], value[th * 16 + c], sk, sv);
  if (off != __builtin_ctz(mask)) return;    // not this block's lowest new offset
  uint8_t* kp = k_pool + tile * (kBS * kD);
  uint8_t* vp = v_pool + tile * (kBS * kD);
  if (!fresh && sk > sk_old) requant_k_rows(kp, c, mask, sk_old / sk);
  if (!fresh && sv > sv_old) requant_v_rows(vp, c, mask, sv_old / sv);
  if (c == 0) {
    k_bscale[tile] = sk;
    v_bscale[tile] = sv;
  }
}

__global__ void __launch_bounds__(256)
dyn_write_kernel(const u32x4* __restrict__ key, const u32x4* __restrict__ value,
                 uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
                 float* __restrict__ k_bscale, float* __restrict__ v_bscale,
                 const int64_t* __restrict__ slots, int64_t total, int hkv, int64_t num_slots,
                 const uint32_t* __restrict__ amax, const uint32_t* __restrict__ written) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= total) return;
  const int c = (int)(gid & 15);
  const int64_t th = gid >> 4;
  const int64_t tok = th / hkv;
  const int h = (int)(th - tok * hkv);
  const int64_t slot = slots[tok];
  if (slot < 0 || slot >= num_slots) return;
  const uint32_t mask = written[slot >> 4];
  if (mask & 0x80000000u) return;            // a whole block, already written
  write_row(key, value, k_pool, v_pool, k_bscale, v_bscale, th, h, slot, mask, c, hkv, amax);
}

// Both passes for calls of more than kDynManyRows rows.  There the
// tile-building pass has usually written nearly every block whole, and one
// 16-lane group per row spent the launch on waves that only found that out
// (110 us of dispatch and two dependent loads each for the 524,288-token
// fill).  Here a wave takes kDynWaveTokens consecutive tokens: one lane per
// token reads its slot and its block's mark, and the wave then works only
// on the tokens left, four rows (kv heads) at a time.
constexpr int kDynWaveTokens = 16;

template <bool kWrite>
__global__ void __launch_bounds__(256)
dyn_by_token_kernel(const u32x4* __restrict__ key, const u32x4* __restrict__ value,
                    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
                    float* __restrict__ k_bscale, float* __restrict__ v_bscale,
                    const int64_t* __restrict__ slots, int64_t num_tokens, int hkv,
                    int64_t num_slots, uint32_t* __restrict__ amax,
                    uint32_t* __restrict__ written) {
  const int lane = threadIdx.x & 63;
  const int64_t t0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kDynWaveTokens;
  int64_t my_slot = -1;
  if (lane < kDynWaveTokens && t0 + lane < num_tokens) my_slot = slots[t0 + lane];
  const bool valid = my_slot >= 0 && my_slot < num_slots;
  // the amax pass only reads the whole-block bit (it sets the others itself);
  // the write pass reads the final mark
  const uint32_t my_mark = valid ? written[my_slot >> 4] : 0x80000000u;
  uint64_t left = __ballot(!(my_mark & 0x80000000u));
  const int c = lane & 15, q = lane >> 4;
  while (left != 0) {                        // uniform over the wave
    const int i = __builtin_ctzll(left);
    left &= left - 1;
    const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)my_slot, i, kWave);
    const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)((uint64_t)my_slot >> 32), i, kWave);
    const int64_t slot = (int64_t)(((uint64_t)hi << 32) | lo);
    const uint32_t mark = (uint32_t)__shfl((int)my_mark, i, kWave);
    for (int h = q; h < hkv; h += 4) {       // the same for the 16 lanes of a row
      const int64_t th = (t0 + i) * hkv + h;
      if constexpr (kWrite)
        write_row(key, value, k_pool, v_pool, k_bscale, v_bscale, th, h, slot, mark, c, hkv,
                  amax);
      else
        amax_row(key, value, th, h, slot, c, hkv, amax, written);
    }
  }
}

// Calls of at most one wave of tokens (a decode step) in one launch: each row
// finds the call's tokens in its block by comparing the call's slots, which
// one wave holds (lane l: token l), and computes the block's MaxAbs and
// written offsets itself instead of through the scratch.  Then as
// dyn_write_kernel: the same scale, codes and re-encoding.  Thread mapping
// as the plain write: 16 lanes per (token, kv head) row, 4 rows per wave.
constexpr int kDynSmallTokens = kWave;
constexpr int64_t kDynManyRows = (int64_t)1 << 17;

__global__ void __launch_bounds__(256)
dyn_write_small_kernel(const u32x4* __restrict__ key, const u32x4* __restrict__ value,
                       uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
                       float* __restrict__ k_bscale, float* __restrict__ v_bscale,
                       const int64_t* __restrict__ slots, int num_tokens, int hkv,
                       int64_t num_slots) {
  const int lane = threadIdx.x & 63;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)num_tokens * hkv * 16;
  const bool active = gid < total;          // inactive lanes still take part in the ballots
  const int c = (int)(gid & 15);
  const int64_t th = gid >> 4;
  const int tok = active ? (int)(th / hkv) : 0;
  const int h = active ? (int)(th - (int64_t)tok * hkv) : 0;
  const int64_t my_slot = active ? slots[tok] : -1;
  const bool valid = my_slot >= 0 && my_slot < num_slots;
  const int blk = valid ? (int)(my_slot >> 4) : -1;   // block ids fit 31 bits
  // lane l holds token l's block (or -1)
  const int64_t sl = lane < num_tokens ? slots[lane] : -1;
  const int lblk = sl >= 0 && sl < num_slots ? (int)(sl >> 4) : -1;
  uint64_t same = 0;                        // the call's tokens in this row's block
#pragma unroll
  for (int g = 0; g < 4; ++g) {             // every lane takes part: no lane has left yet
    const int bg = __shfl(blk, g * 16, kWave);
    const uint64_t m = __ballot(lblk == bg && bg >= 0);
    if ((lane >> 4) == g) same = m;
  }
  if (!valid) return;                       // the same for all 16 lanes of the row
  uint32_t km = 0, vm = 0, mask = 0;
  for (uint64_t rest = same; rest != 0; rest &= rest - 1) {
    const int t = __builtin_ctzll(rest);
    const int64_t row = ((int64_t)t * hkv + h) * 16 + c;
    km = max(km, max_abs_bits8(key[row]));
    vm = max(vm, max_abs_bits8(value[row]));
    mask |= 1u << (slots[t] & 15);
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) {
    km = max(km, (uint32_t)__shfl_xor((int)km, m, kWave));
    vm = max(vm, (uint32_t)__shfl_xor((int)vm, m, kWave));
  }
  const int off = (int)(my_slot & 15);
  const int64_t tile = blk * hkv + h;
  const bool fresh = (mask & 1u) != 0;
  const float min_scale = 0x1p-126f;
  const float sk_old = fresh ? 0.0f : k_bscale[tile];
  const float sv_old = fresh ? 0.0f : v_bscale[tile];
  const float sk = fmaxf(fmaxf(sk_old, f16_bits_to_float(km) / 448.0f), min_scale);
  const float sv = fmaxf(fmaxf(sv_old, f16_bits_to_float(vm) / 448.0f), min_scale);
  store_rows8<true>(k_pool, v_pool, tile, off, c, key[th * 16 + c], value[th * 16 + c], sk, sv);
  if (off != __builtin_ctz(mask)) return;    // not this block's lowest new offset
  uint8_t* kp = k_pool + tile * (kBS * kD);
  uint8_t* vp = v_pool + tile * (kBS * kD);
  if (!fresh && sk > sk_old) requant_k_rows(kp, c, mask, sk_old / sk);
  if (!fresh && sv > sv_old) requant_v_rows(vp, c, mask, sv_old / sv);
  if (c == 0) {
    k_bscale[tile] = sk;
    v_bscale[tile] = sv;
  }
}

// ------------------------------------------------------------ copy_blocks

// One workgroup per (source, destination) pair; with per-block scales the
// destination's scale rows are copied too.
__global__ void __launch_bounds__(256)
copy_blocks_kernel(u32x4* __restrict__ k_pool, u32x4* __restrict__ v_pool,
                   float* __restrict__ k_bscale, float* __restrict__ v_bscale, int hkv,
                   const int32_t* __restrict__ pairs, int64_t vecs_per_block, int num_blocks) {
  const int i = blockIdx.x;
  const int src = pairs[2 * i], dst = pairs[2 * i + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const int64_t s0 = (int64_t)src * vecs_per_block, d0 = (int64_t)dst * vecs_per_block;
  for (int64_t v = threadIdx.x; v < vecs_per_block; v += 256) {
    k_pool[d0 + v] = k_pool[s0 + v];
    v_pool[d0 + v] = v_pool[s0 + v];
  }
  if (k_bscale != nullptr) {
    for (int h = threadIdx.x; h < hkv; h += 256) {
      k_bscale[(int64_t)dst * hkv + h] = k_bscale[(int64_t)src * hkv + h];
      v_bscale[(int64_t)dst * hkv + h] = v_bscale[(int64_t)src * hkv + h];
    }
  }
}

}  // namespace

// ------------------------------------------------------------------ C ABI

// The tile-building kernel over a call: one workgroup per (16-token group,
// KV head), in launches of at most 2^24 workgroups.  A block that straddles
// two launches is written row by row by both.
template <bool kFP8, bool kDyn>
static pkv_status launch_fill(const void* key, const void* value, void* k_pool, void* v_pool,
                              const int64_t* slot_mapping, int32_t num_tokens,
                              const pkv_cache_layout* layout, float k_scale, float v_scale,
                              DynTiles dt, hipStream_t s) {
  const int64_t groups = ((int64_t)num_tokens + kBS - 1) / kBS;
  const int64_t num_slots = (int64_t)layout->num_blocks * kBS;
  const int hkv = layout->num_kv_heads;
  const int64_t max_groups = std::max<int64_t>(1, ((int64_t)1 << 24) / hkv);
  for (int64_t g0 = 0; g0 < groups; g0 += max_groups) {
    const int64_t ng = std::min(max_groups, groups - g0);
    const int64_t tok0 = g0 * kBS;
    const int64_t ntok = std::min<int64_t>((int64_t)num_tokens - tok0, ng * kBS);
    const u32x4* kin = static_cast<const u32x4*>(key) + tok0 * hkv * 16;
    const u32x4* vin = static_cast<const u32x4*>(value) + tok0 * hkv * 16;
    const uint32_t units = (uint32_t)(ng * hkv);
    const dim3 grid((units + kFillWaves - 1) / kFillWaves);
    reshape_and_cache_kernel<kFP8, kDyn><<<grid, dim3(kFillWaves * kWave), 0, s>>>(
        kin, vin, static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool),
        slot_mapping + tok0, ntok, hkv, num_slots, k_scale, v_scale, units, dt);
    const pkv_status st = launch_status();
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}

extern "C" pkv_status pkv_reshape_and_cache(const void* key, const void* value, void* k_pool,
                                            void* v_pool, const int64_t* slot_mapping,
                                            int32_t num_tokens, const pkv_cache_layout* layout,
                                            float k_scale, float v_scale, void* stream) {
  pkv_status st = check_layout(layout);
  if (st != PKV_OK) return st;
  if (num_tokens < 0) return PKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !k_pool || !v_pool || !slot_mapping) return PKV_ERR_INVALID_ARG;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(slot_mapping, 8))
    return PKV_ERR_INVALID_ARG;
  const bool fp8 = layout->dtype == PKV_FP8_E4M3FN;
  if (fp8 && !(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) &&
               v_scale > 0.0f))
    return PKV_ERR_INVALID_ARG;
  const int64_t num_slots = (int64_t)layout->num_blocks * kBS;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int64_t total = (int64_t)num_tokens * layout->num_kv_heads * 16;
  if (num_tokens <= kRowWriteMaxTokens && total < ((int64_t)1 << 31)) {
    const unsigned blocks = (unsigned)((total + 255) / 256);
    if (fp8)
      reshape_rows_kernel<true><<<dim3(blocks), dim3(256), 0, s>>>(
          static_cast<const u32x4*>(key), static_cast<const u32x4*>(value),
          static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), slot_mapping,
          (uint32_t)total, (uint32_t)layout->num_kv_heads, num_slots, k_scale, v_scale);
    else
      reshape_rows_kernel<false><<<dim3(blocks), dim3(256), 0, s>>>(
          static_cast<const u32x4*>(key), static_cast<const u32x4*>(value),
          static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), slot_mapping,
          (uint32_t)total, (uint32_t)layout->num_kv_heads, num_slots, 1.0f, 1.0f);
    return launch_status();
  }
  if (fp8)
    return launch_fill<true, false>(key, value, k_pool, v_pool, slot_mapping, num_tokens,
                                    layout, k_scale, v_scale, DynTiles{}, s);
  return launch_fill<false, false>(key, value, k_pool, v_pool, slot_mapping, num_tokens,
                                   layout, 1.0f, 1.0f, DynTiles{}, s);
}

extern "C" pkv_status pkv_copy_blocks(void* k_pool, void* v_pool, const pkv_cache_layout* layout,
                                      const int32_t* src_dst_pairs, int32_t num_pairs,
                                      void* stream) {
  pkv_status st = check_layout(layout);
  if (st != PKV_OK) return st;
  if (num_pairs < 0) return PKV_ERR_INVALID_ARG;
  if (num_pairs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !src_dst_pairs || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(src_dst_pairs, 4))
    return PKV_ERR_INVALID_ARG;
  const int64_t bytes = (int64_t)layout->num_kv_heads * kBS * kD * elem_bytes(layout->dtype);
  (void)hipGetLastError();
  copy_blocks_kernel<<<dim3((unsigned)num_pairs), dim3(256), 0,
                       static_cast<hipStream_t>(stream)>>>(
      static_cast<u32x4*>(k_pool), static_cast<u32x4*>(v_pool), nullptr, nullptr,
      layout->num_kv_heads, src_dst_pairs, bytes / 16, layout->num_blocks);
  return launch_status();
}

extern "C" uint64_t pkv_reshape_dynamic_workspace_bytes(const pkv_cache_layout* layout) {
  if (check_layout(layout) != PKV_OK || layout->dtype != PKV_FP8_E4M3FN) return 0;
  const uint64_t words = (uint64_t)layout->num_blocks * (2 * (uint64_t)layout->num_kv_heads + 1);
  return (words * 4 + 255) / 256 * 256;
}

extern "C" pkv_status pkv_reshape_and_cache_dynamic(
    const void* key, const void* value, void* k_pool, void* v_pool, float* k_block_scales,
    float* v_block_scales, const int64_t* slot_mapping, int32_t num_tokens,
    const pkv_cache_layout* layout, void* workspace, uint64_t workspace_bytes, void* stream) {
  pkv_status st = check_layout(layout);
  if (st != PKV_OK) return st;
  if (layout->dtype != PKV_FP8_E4M3FN) return PKV_ERR_UNSUPPORTED;
  if (num_tokens < 0) return PKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !k_pool || !v_pool || !slot_mapping || !k_block_scales ||
      !v_block_scales)
    return PKV_ERR_INVALID_ARG;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(slot_mapping, 8) || !aligned(k_block_scales, 4) || !aligned(v_block_scales, 4))
    return PKV_ERR_INVALID_ARG;
  const uint64_t need = pkv_reshape_dynamic_workspace_bytes(layout);
  if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return PKV_ERR_INVALID_ARG;
  const int hkv = layout->num_kv_heads;
  const int64_t total = (int64_t)num_tokens * hkv * 16;
  const int64_t blocks = (total + 255) / 256;
  const int64_t clear_blocks = ((int64_t)num_tokens + 255) / 256;
  if (blocks > 0x7FFFFFFF) return PKV_ERR_INVALID_ARG;
  const int64_t num_slots = (int64_t)layout->num_blocks * kBS;
  uint32_t* amax = static_cast<uint32_t*>(workspace);
  uint32_t* written = amax + (int64_t)layout->num_blocks * 2 * hkv;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (num_tokens <= kDynSmallTokens) {  // a decode step: one launch, no scratch
    dyn_write_small_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
        static_cast<const u32x4*>(key), static_cast<const u32x4*>(value),
        static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), k_block_scales,
        v_block_scales, slot_mapping, num_tokens, hkv, num_slots);
    return launch_status();
  }
  dyn_clear_kernel<<<dim3((unsigned)clear_blocks), dim3(256), 0, s>>>(
      slot_mapping, (int64_t)num_tokens, 2 * hkv, num_slots, amax, written);
  // blocks the call fills whole: tiles, scales and marks in one pass
  if (num_tokens > kRowWriteMaxTokens) {
    st = launch_status();
    if (st != PKV_OK) return st;
    st = launch_fill<true, true>(key, value, k_pool, v_pool, slot_mapping, num_tokens, layout,
                                 1.0f, 1.0f, DynTiles{k_block_scales, v_block_scales, written},
                                 s);
    if (st != PKV_OK) return st;
  }
  if ((int64_t)num_tokens * hkv > kDynManyRows) {
    const int64_t waves = ((int64_t)num_tokens + kDynWaveTokens - 1) / kDynWaveTokens;
    const dim3 grid((unsigned)((waves + 3) / 4));
    dyn_by_token_kernel<false><<<grid, dim3(256), 0, s>>>(
        static_cast<const u32x4*>(key), static_cast<const u32x4*>(value), nullptr, nullptr,
        nullptr, nullptr, slot_mapping, num_tokens, hkv, num_slots, amax, written);
    dyn_by_token_kernel<true><<<grid, dim3(256), 0, s>>>(
        static_cast<const u32x4*>(key), static_cast<const u32x4*>(value),
        static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), k_block_scales,
        v_block_scales, slot_mapping, num_tokens, hkv, num_slots, amax, written);
  } else {
    dyn_amax_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
        static_cast<const u32x4*>(key), static_cast<const u32x4*>(value), slot_mapping, total,
        hkv, num_slots, amax, written);
    dyn_write_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(
        static_cast<const u32x4*>(key), static_cast<const u32x4*>(value),
        static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), k_block_scales,
        v_block_scales, slot_mapping, total, hkv, num_slots, amax, written);
  }
  return launch_status();
}

extern "C" pkv_status pkv_copy_blocks_dynamic(void* k_pool, void* v_pool, float* k_block_scales,
                                              float* v_block_scales,
                                              const pkv_cache_layout* layout,
                                              const int32_t* src_dst_pairs, int32_t num_pairs,
                                              void* stream) {
  pkv_status st = check_layout(layout);
  if (st != PKV_OK) return st;
  if (layout->dtype != PKV_FP8_E4M3FN) return PKV_ERR_UNSUPPORTED;
  if (num_pairs < 0) return PKV_ERR_INVALID_ARG;
  if (num_pairs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !src_dst_pairs || !k_block_scales || !v_block_scales ||
      !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(src_dst_pairs, 4) ||
      !aligned(k_block_scales, 4) || !aligned(v_block_scales, 4))
    return PKV_ERR_INVALID_ARG;
  const int64_t bytes = (int64_t)layout->num_kv_heads * kBS * kD;
  (void)hipGetLastError();
  copy_blocks_kernel<<<dim3((unsigned)num_pairs), dim3(256), 0,
                       static_cast<hipStream_t>(stream)>>>(
      static_cast<u32x4*>(k_pool), static_cast<u32x4*>(v_pool), k_block_scales, v_block_scales,
      layout->num_kv_heads, src_dst_pairs, bytes / 16, layout->num_blocks);
  return launch_status();
}
