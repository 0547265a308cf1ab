// pkv_tile.h — device building blocks shared by libpkv's gfx950 attention
// kernels (decode and chunked prefill): shapes, vector types, the load of one
// (block, KV head) tile into registers in MFMA operand order, FP8 -> fp16
// conversion and wave reductions.  Included by the .hip sources only.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pkv_dev {

constexpr int kBS = 16;      // tokens per block
constexpr int kD = 128;      // head dim
constexpr int kWave = 64;
constexpr int kMaxG = 16;    // MFMA N dimension: query heads per KV head

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Four E4M3 codes (one dword) -> four fp16 values equal to code_value / 256.
// fp16 bits s|0|eeee|mmm|0000000 read as binary16 are (1 + m/8) 2^(e-15)
// (or m/8 * 2^-14 for e = 0), i.e. exactly 2^-8 times the E4M3 value.
__device__ __forceinline__ f16x4 e4m3x4_to_f16_div256(uint32_t x) {
  const uint32_t hi = ((x >> 1) & 0x3F3F3F3Fu) | (x & 0x80808080u);  // s 0 e e e e m m
  const uint32_t lo = (x << 7) & 0x80808080u;                        // m0 0000000
  u32x2 r;
  r.x = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // lo0 hi0 lo1 hi1
  r.y = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // lo2 hi2 lo3 hi3
  return __builtin_bit_cast(f16x4, r);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

template <bool kFP8>
struct TileRegs {
  static constexpr int kVecs = kFP8 ? 2 : 4;  // 16-byte loads per lane per tile
  u32x4 k[kVecs];
  u32x4 v[kVecs];
};

// A raw buffer resource over `bytes` bytes at `base`.  A load through it
// that falls past `bytes` (every load when bytes is 0) returns zeros and
// touches no memory.  The decode loops use this to issue the same loads on
// every path: the compiler counts outstanding vector memory operations at
// each control-flow join as the fewest that any incoming path leaves, so a
// load issued on one path only (a prefetch past the last tile, a block id
// outside the pool) made every later wait also wait for the loads issued
// after the one it needed -- the next tile's, which defeated the prefetch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_range(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

constexpr int kLoadNT = 2;  // buffer load cache policy: non-temporal (stream past the caches)

// Load one (block, kv head) tile: each lane reads 16 bytes at i * 1 KiB +
// 16 * lane, with cache policy kAux: tiles only this sequence reads are
// streamed past the caches (kLoadNT); tiles of a shared prefix go through
// them (0), so the sibling sequences that read the same tile shortly after
// can hit.  The policy is a template argument because a branch between two
// policies is itself a path the compiler may count as issuing no load.  A
// phys outside [0, num_blocks) -- no tile, or a prefetch past the end --
// loads zeros, with the same instructions.  phys and kvh are wave-uniform.
template <bool kFP8, int kAux>
__device__ __forceinline__ void load_tile(TileRegs<kFP8>& r, const uint8_t* k_pool,
                                          const uint8_t* v_pool, int num_blocks, int hkv,
                                          int phys, int kvh, int lane) {
  constexpr int kTileBytes = kBS * kD * (kFP8 ? 1 : 2);
  // uniform by contract; said so, the resources stay scalar
  phys = __builtin_amdgcn_readfirstlane(phys);
  kvh = __builtin_amdgcn_readfirstlane(kvh);
  const bool ok = (unsigned)phys < (unsigned)num_blocks;
  const int64_t off = ok ? ((int64_t)phys * hkv + kvh) * kTileBytes : 0;
  const __amdgpu_buffer_rsrc_t kr = byte_range(k_pool + off, ok ? kTileBytes : 0);
  const __amdgpu_buffer_rsrc_t vr = byte_range(v_pool + off, ok ? kTileBytes : 0);
#pragma unroll
  for (int i = 0; i < TileRegs<kFP8>::kVecs; ++i) {
    r.k[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, (i * kWave + lane) * 16, 0, kAux);
    r.v[i] = __builtin_amdgcn_raw_buffer_load_b128(vr, (i * kWave + lane) * 16, 0, kAux);
  }
}

// Entries [first, first + n * stride) of a block-table row, lane i taking
// entry first + i * stride (i < n <= 64); lanes past n read 0.
__device__ __forceinline__ int load_table(const int32_t* first, int n, int stride, int lane) {
  const __amdgpu_buffer_rsrc_t tr = byte_range(first, n > 0 ? ((n - 1) * stride + 1) * 4 : 0);
  return (int)__builtin_amdgcn_raw_buffer_load_b32(tr, lane * stride * 4, 0, 0);
}

// FP8 dequantisation of four codes (one dword) to fp16.  Two exact ways:
//  * kHwCvt: the gfx950 conversion v_cvt_scalef32_pk_f16_fp8 (scale 1.0)
//    gives the code values themselves;
//  * otherwise integer bit operations give code_value / 256 (see
//    e4m3x4_to_f16_div256); the factor 256 is folded into the scales.
template <bool kHwCvt>
__device__ __forceinline__ f16x4 dequant4(uint32_t x) {
  if constexpr (kHwCvt) {
    typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
    const f16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)x, 1.0f, false);
    const f16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)x, 1.0f, true);
    return f16x4{lo[0], lo[1], hi[0], hi[1]};
  } else {
    return e4m3x4_to_f16_div256(x);
  }
}

// Logits may exceed the reference max by up to 2^8 before the max is
// re-reduced across the wave and the accumulators rescaled: p <= 256 stays
// exact enough in fp16 and far from fp32 overflow.  On random data the
// reference settles after a few tiles, so the steady state runs no
// cross-lane reduction and no rescaling.
constexpr float kLazyMaxSlack = 8.0f;

// Zero the value elements of tokens >= L in a sequence's last, partly filled
// tile.  Their probabilities are zero, but the slots may hold anything (a
// pool allocated without clearing, an earlier sequence's data): a NaN or
// infinity there would turn 0 * v into NaN inside the PV product.  Lane qg
// holds tokens 4qg .. 4qg+3 of each value register (the innermost index).
template <bool kFP8>
__device__ __forceinline__ void mask_tail_values(TileRegs<kFP8>& t, int tb, int qg, int L) {
  const int nv = min(max(L - (tb + qg * 4), 0), 4);  // valid tokens among this lane's four
  if constexpr (kFP8) {  // one byte per token
    const uint32_t m = nv >= 4 ? 0xFFFFFFFFu : ((1u << (8 * nv)) - 1u);
#pragma unroll
    for (int i = 0; i < TileRegs<kFP8>::kVecs; ++i) {
      t.v[i].x &= m;
      t.v[i].y &= m;
      t.v[i].z &= m;
      t.v[i].w &= m;
    }
  } else {  // two tokens per 32-bit word: x, z hold tokens 0-1, y, w tokens 2-3
    const uint32_t m01 = nv >= 2 ? 0xFFFFFFFFu : (nv == 1 ? 0xFFFFu : 0u);
    const uint32_t m23 = nv >= 4 ? 0xFFFFFFFFu : (nv == 3 ? 0xFFFFu : 0u);
#pragma unroll
    for (int i = 0; i < TileRegs<kFP8>::kVecs; ++i) {
      t.v[i].x &= m01;
      t.v[i].y &= m23;
      t.v[i].z &= m01;
      t.v[i].w &= m23;
    }
  }
}

}  // namespace pkv_dev
