// pkv_prefill.hip — gfx950 kernel for chunked prefill over the paged cache:
// the queries of a prompt chunk attend causally to every token of their
// sequence already in the cache ([FP8-128K] "Optimización de KV Cache con
// PagedAttention y Cuantización FP8 para Contextos Largos (128K)", §5:
// chunked prefill cuts a long prompt into packets of tokens).
//
// Sequence b's chunk is its last n_b tokens (their keys and values are in the
// cache), so chunk row i sits at position p = L_b - n_b + i and attends to
// tokens 0..p.
//
// Unlike decode this is a dense contraction: each K/V tile meets 16 query
// tokens x G heads, so the work is bound by the matrix cores, not by HBM.
// Design for CDNA4:
//   * a 16-row tile of chunk tokens and one KV head take ceil(G/2) waves,
//     two query heads each, so a K/V tile loaded once per wave (the waves of
//     a workgroup share it through L1) feeds 32 query rows per wave and
//     16 x G per row tile; a workgroup holds one row tile (FP8) or up to
//     8 waves' worth (fp16, whose pairs are not kept in flight);
//   * tiles go in pairs (32 tokens): S^T = K Q^T by four 16x16x32 fp16 MFMAs
//     per tile and head, and O^T += V^T P^T by eight 16x16x32 MFMAs per pair
//     and head -- the S^T accumulators of the two tiles, taken as fp16, are
//     exactly the B operand of the second product (contraction order: this
//     lane's four tokens of the first tile, then its four of the second);
//   * FP8 tiles are converted to fp16 in registers (exact), probabilities are
//     fp16 (the normaliser sums them in fp32 before rounding), accumulation
//     fp32; the online softmax keeps a lazy reference max per query row, as
//     the decode kernel does, tested on each lane's largest logit;
//   * only the pairs that reach past the row tile's first position apply
//     the causal mask; value slots past the sequence's end are zeroed;
//   * FP8 caches (per-tensor or per-block scales) run the pairs as a software
//     pipeline: one straight-line block takes pair i's exponentials, pair
//     i+1's QK^T products and pair i's PV products, so the compiler
//     interleaves vector and matrix work within each wave;
//   * the fp16 cache's loop takes one pair at a time and runs its matrix
//     bursts at raised priority (s_setprio), so the two waves of a SIMD tend
//     to alternate matrix and vector phases.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "pkv.h"
#include "pkv_check.h"
#include "pkv_tile.h"

namespace {

using namespace pkv_dev;
using namespace pkv_check;

constexpr int kQT = 16;       // chunk tokens per workgroup
constexpr int kHeadsPerWave = 2;

struct PrefillArgs {
  float* out;                   // [rows][Hq][D]
  const _Float16* q;            // [rows][Hq][D]
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const int32_t* block_tables;  // [B][max_blocks]
  const int32_t* context_lens;  // [B]
  const int32_t* query_start;   // [B + 1]
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t hq, hkv, g;
  int32_t max_ctx;
  int32_t wpt;                  // waves per 16-row tile: ceil(G / kHeadsPerWave)
  int32_t rt;                   // 16-row tiles per workgroup
  float qk_scale;               // sm_scale * k_scale * log2(e) (per-block scales: no k_scale)
  float out_scale;              // v_scale (per-block scales: unused)
  const float* k_bscale;        // [num_blocks][hkv] per-block K scales, or null
  const float* v_bscale;        // [num_blocks][hkv] per-block V scales, or null
};

struct RowState {
  float m_ref;   // reference max of the row (log2 units), equal on its 4 lanes
  float l;       // this lane's share of the normaliser
  f32x4 acc[8];  // O^T rows 16n + 4qg .. +3
};

// Two FP8 codes (the low or high half of a dword) -> two fp16 values, as the
// 32-bit word an MFMA operand register holds (exact).
template <bool kHi>
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t x) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  const f16x2_t h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)x, 1.0f, kHi);
  return __builtin_bit_cast(uint32_t, h);
}

template <bool kFP8>
__device__ __forceinline__ f16x8 k_operand(const TileRegs<kFP8>& t, int m) {
  if constexpr (kFP8) {
    const u32x4 raw = t.k[m >> 1];
    const uint32_t a = (m & 1) ? raw.z : raw.x, b = (m & 1) ? raw.w : raw.y;
    const u32x4 w = u32x4{fp8x2_to_f16x2<false>(a), fp8x2_to_f16x2<true>(a),
                          fp8x2_to_f16x2<false>(b), fp8x2_to_f16x2<true>(b)};
    return __builtin_bit_cast(f16x8, w);
  } else {
    return __builtin_bit_cast(f16x8, t.k[m]);
  }
}

// Channel 16n + (lane % 16), tokens 4qg..4qg+3 of tile a then of tile b: the
// A operand of the PV product for one pair.
template <bool kFP8>
__device__ __forceinline__ f16x8 v_operand(const TileRegs<kFP8>& ta, const TileRegs<kFP8>& tb,
                                           int n) {
  if constexpr (kFP8) {
    const uint32_t a = ta.v[n >> 2][n & 3], b = tb.v[n >> 2][n & 3];
    const u32x4 w = u32x4{fp8x2_to_f16x2<false>(a), fp8x2_to_f16x2<true>(a),
                          fp8x2_to_f16x2<false>(b), fp8x2_to_f16x2<true>(b)};
    return __builtin_bit_cast(f16x8, w);
  } else {
    const u32x4 ra = ta.v[n >> 1], rb = tb.v[n >> 1];
    const int o = (n & 1) * 2;
    return __builtin_bit_cast(f16x8, u32x4{ra[o], ra[o + 1], rb[o], rb[o + 1]});
  }
}

// One half (K or V) of both tiles of a pair, zeros for ids outside the pool
// (and for tile b when `zero_b`: the pair reaches past the last tile).
template <bool kFP8, bool kV>
__device__ __forceinline__ void load_pair_half(TileRegs<kFP8>& ta, TileRegs<kFP8>& tb,
                                               const PrefillArgs& a, int pa, int pb, int kvh,
                                               int lane, bool zero_b) {
  constexpr int kTileBytes = kBS * kD * (kFP8 ? 1 : 2);
  const bool oka = (unsigned)pa < (unsigned)a.num_blocks;
  const bool okb = (unsigned)pb < (unsigned)a.num_blocks && !zero_b;
  const uint8_t* pool = kV ? a.v_pool : a.k_pool;
  const u32x4* xa = reinterpret_cast<const u32x4*>(
                        pool + ((int64_t)(oka ? pa : 0) * a.hkv + kvh) * kTileBytes) + lane;
  const u32x4* xb = reinterpret_cast<const u32x4*>(
                        pool + ((int64_t)(okb ? pb : 0) * a.hkv + kvh) * kTileBytes) + lane;
  u32x4* da = kV ? ta.v : ta.k;
  u32x4* db = kV ? tb.v : tb.k;
#pragma unroll
  for (int i = 0; i < TileRegs<kFP8>::kVecs; ++i) {
    da[i] = xa[i * kWave];
    db[i] = xb[i * kWave];
  }
  if (!oka || !okb) {
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < TileRegs<kFP8>::kVecs; ++i) {
      if (!oka) da[i] = u32x4{0, 0, 0, 0};
      if (!okb) db[i] = u32x4{0, 0, 0, 0};
    }
  }
}

// fp16 tiles are twice the registers of FP8 ones: the V halves of a pair
// are loaded after its QK^T products (process_pair calls this there).
struct VLate {
  const PrefillArgs* a;
  int pa, pb, kvh, lane;
  bool zero_b;
  __device__ void operator()(TileRegs<false>& ta, TileRegs<false>& tb) const {
    load_pair_half<false, true>(ta, tb, *a, pa, pb, kvh, lane, zero_b);
  }
};

// One pair of fp16 tiles (tokens tb .. tb+31) for the wave's query heads.
// pos_j: position of this lane's query row.  masked: the pair reaches past
// the workgroup's first position, so tokens after pos_j are dropped.  qk is
// the logit scale; it is positive, so a row's largest logit is qk times its
// largest dot product.  fp16 tiles take twice the registers of FP8 ones: the
// pair's V halves are loaded (late_v) only after its QK^T products, into the
// registers K no longer needs, so those loads overlap the softmax.
__device__ __forceinline__ void process_pair(TileRegs<false>& ta, TileRegs<false>& tb_,
                                             const f16x8 (&qop)[kHeadsPerWave][4],
                                             RowState (&st)[kHeadsPerWave], int tb, int qg,
                                             int pos_j, int L, bool masked, float qk,
                                             const VLate& late_v) {
  f32x4 s[kHeadsPerWave][2];
  // matrix bursts run at raised priority, so the SIMD's other wave does its
  // vector work meanwhile instead of both reaching their softmax together
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int h = 0; h < kHeadsPerWave; ++h) s[h][0] = s[h][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const f16x8 ka = k_operand<false>(ta, m);
    const f16x8 kb = k_operand<false>(tb_, m);
#pragma unroll
    for (int h = 0; h < kHeadsPerWave; ++h) {
      s[h][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qop[h][m], s[h][0], 0, 0, 0);
      s[h][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb, qop[h][m], s[h][1], 0, 0, 0);
    }
  }
  __builtin_amdgcn_s_setprio(0);
  late_v(ta, tb_);
  if (masked) {  // wave-uniform; only the pairs that reach past the first position
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int tok = tb + (r >> 2) * kBS + qg * 4 + (r & 3);
      if (tok > pos_j) {
#pragma unroll
        for (int h = 0; h < kHeadsPerWave; ++h) s[h][r >> 2][r & 3] = -INFINITY;
      }
    }
  }
  f16x8 p[kHeadsPerWave];
#pragma unroll
  for (int h = 0; h < kHeadsPerWave; ++h) {
    // exponent of each weight relative to the reference max (log2 units)
    float y[8];
    const float neg_m = -st[h].m_ref;
#pragma unroll
    for (int r = 0; r < 8; ++r) y[r] = fmaf(s[h][r >> 2][r & 3], qk, neg_m);
    float ymax = y[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) ymax = fmaxf(ymax, y[r]);
    if (__any(ymax > kLazyMaxSlack)) {
      __asm__ volatile("" ::: "memory");  // rare: keep the rescale a branch
      // the row's new reference: its largest logit so far
      float top = -INFINITY;
#pragma unroll
      for (int r = 0; r < 8; ++r) top = fmaxf(top, s[h][r >> 2][r & 3] * qk);
      top = fmaxf(top, __shfl_xor(top, 16, kWave));
      top = fmaxf(top, __shfl_xor(top, 32, kWave));
      const float m_upd = fmaxf(st[h].m_ref, top);
      const float alpha = __builtin_amdgcn_exp2f(st[h].m_ref - m_upd);
      st[h].l *= alpha;
#pragma unroll
      for (int n = 0; n < 8; ++n) st[h].acc[n] *= alpha;
      st[h].m_ref = m_upd;
#pragma unroll
      for (int r = 0; r < 8; ++r) y[r] = fmaf(s[h][r >> 2][r & 3], qk, -m_upd);
    }
    float e[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) e[r] = __builtin_amdgcn_exp2f(y[r]);
    st[h].l += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
#pragma unroll
    for (int r = 0; r < 8; ++r) p[h][r] = (_Float16)e[r];
  }
  if (tb + 2 * kBS > L) {  // the sequence's last tiles: slots past L may hold anything
    __asm__ volatile("" ::: "memory");
    mask_tail_values<false>(ta, tb, qg, L);
    mask_tail_values<false>(tb_, tb + kBS, qg, L);
  }
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const f16x8 v = v_operand<false>(ta, tb_, n);
#pragma unroll
    for (int h = 0; h < kHeadsPerWave; ++h)
      st[h].acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v, p[h], st[h].acc[n], 0, 0, 0);
  }
  __builtin_amdgcn_s_setprio(0);
}

// ---- FP8 caches: pairs in a software pipeline ---------------------------
// Each iteration takes the softmax of pair i, the QK^T products of pair
// i + 1 and the PV products of pair i in one straight-line block, so the
// matrix cores work on pair i + 1 while the vector ALUs take pair i's
// exponentials.  K halves are loaded three pairs ahead and V halves two,
// through buffer resources (ids outside the pool: 0 bytes, zeros), so every
// path issues the same loads and each wait covers only the pair it needs.
// Nothing in this path may be an inline asm statement: the compiler takes
// one as a write to memory, and then loads the table entries through the
// vector memory path (whose waits also cover the tiles in flight) instead
// of the scalar one.  The rare branches stay branches without it.
template <bool kV>
__device__ __forceinline__ void load_half_pipe(TileRegs<true>& ta, TileRegs<true>& tb,
                                               const PrefillArgs& a, int pa, int pb, int kvh,
                                               int lane) {
  constexpr int kTileBytes = kBS * kD;
  pa = __builtin_amdgcn_readfirstlane(pa);
  pb = __builtin_amdgcn_readfirstlane(pb);
  kvh = __builtin_amdgcn_readfirstlane(kvh);
  const bool oka = (unsigned)pa < (unsigned)a.num_blocks;
  const bool okb = (unsigned)pb < (unsigned)a.num_blocks;
  const uint8_t* pool = kV ? a.v_pool : a.k_pool;
  // a resource of 0 bytes never touches memory, so its base may be anything:
  // no branch around the address arithmetic
  const __amdgpu_buffer_rsrc_t ra =
      byte_range(pool + ((int64_t)pa * a.hkv + kvh) * kTileBytes, oka ? kTileBytes : 0);
  const __amdgpu_buffer_rsrc_t rb =
      byte_range(pool + ((int64_t)pb * a.hkv + kvh) * kTileBytes, okb ? kTileBytes : 0);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const u32x4 xa = __builtin_amdgcn_raw_buffer_load_b128(ra, (i * kWave + lane) * 16, 0, 0);
    const u32x4 xb = __builtin_amdgcn_raw_buffer_load_b128(rb, (i * kWave + lane) * 16, 0, 0);
    if constexpr (kV) {
      ta.v[i] = xa;
      tb.v[i] = xb;
    } else {
      ta.k[i] = xa;
      tb.k[i] = xb;
    }
  }
}

// S^T of both tiles of a pair for the wave's heads: 16 MFMAs.
__device__ __forceinline__ void qk_pair(const TileRegs<true>& ta, const TileRegs<true>& tb,
                                        const f16x8 (&qop)[kHeadsPerWave][4],
                                        f32x4 (&s)[kHeadsPerWave][2]) {
#pragma unroll
  for (int h = 0; h < kHeadsPerWave; ++h) s[h][0] = s[h][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const f16x8 ka = k_operand<true>(ta, m);
    const f16x8 kb = k_operand<true>(tb, m);
#pragma unroll
    for (int h = 0; h < kHeadsPerWave; ++h) {
      s[h][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qop[h][m], s[h][0], 0, 0, 0);
      s[h][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb, qop[h][m], s[h][1], 0, 0, 0);
    }
  }
}

// Causal mask of a pair's logits (tokens after the lane's row position).
__device__ __forceinline__ void mask_pair(f32x4 (&s)[kHeadsPerWave][2], int tb, int qg,
                                          int pos_j) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int tok = tb + (r >> 2) * kBS + qg * 4 + (r & 3);
    if (tok > pos_j) {
#pragma unroll
      for (int h = 0; h < kHeadsPerWave; ++h) s[h][r >> 2][r & 3] = -INFINITY;
    }
  }
}

// Exponents of a pair's weights relative to each row's reference max (log2
// units), after rescaling a row whose logits overshoot it (rare: a branch).
__device__ __forceinline__ void check_pair(const f32x4 (&s)[kHeadsPerWave][2],
                                           RowState (&st)[kHeadsPerWave], const float (&qk)[2],
                                           float (&y)[kHeadsPerWave][8]) {
#pragma unroll
  for (int h = 0; h < kHeadsPerWave; ++h) {
    const float neg_m = -st[h].m_ref;
#pragma unroll
    for (int r = 0; r < 8; ++r) y[h][r] = fmaf(s[h][r >> 2][r & 3], qk[r >> 2], neg_m);
    float ymax = y[h][0];
#pragma unroll
    for (int r = 1; r < 8; ++r) ymax = fmaxf(ymax, y[h][r]);
    if (__any(ymax > kLazyMaxSlack)) {
      float top = -INFINITY;
#pragma unroll
      for (int r = 0; r < 8; ++r) top = fmaxf(top, s[h][r >> 2][r & 3] * qk[r >> 2]);
      top = fmaxf(top, __shfl_xor(top, 16, kWave));
      top = fmaxf(top, __shfl_xor(top, 32, kWave));
      const float m_upd = fmaxf(st[h].m_ref, top);
      const float alpha = __builtin_amdgcn_exp2f(st[h].m_ref - m_upd);
      st[h].l *= alpha;
#pragma unroll
      for (int n = 0; n < 8; ++n) st[h].acc[n] *= alpha;
      st[h].m_ref = m_upd;
#pragma unroll
      for (int r = 0; r < 8; ++r) y[h][r] = fmaf(s[h][r >> 2][r & 3], qk[r >> 2], -m_upd);
    }
  }
}

// Probabilities as fp16 (the PV product's B operand) and the normaliser.
// With per-block scales (kDyn) each tile's weights are multiplied by its V
// scale relative to the wave's reference (vm[t]).  kLo: the weights are taken
// as fp16 hi + lo, two PV products of about 22 bits together, for rows whose
// V values are large (see kHiOnlyVRef): there one fp16 rounding of P is too
// coarse against the absolute tolerance.  The normaliser sums the unscaled
// weights.
template <bool kDyn, bool kLo>
__device__ __forceinline__ void probs_pair(const float (&y)[kHeadsPerWave][8],
                                           RowState (&st)[kHeadsPerWave], const float (&vm)[2],
                                           f16x8 (&p)[kHeadsPerWave],
                                           f16x8 (&plo)[kHeadsPerWave]) {
  static_assert(kDyn || !kLo, "the lo halves are for per-block scales");
#pragma unroll
  for (int h = 0; h < kHeadsPerWave; ++h) {
    float e[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) e[r] = __builtin_amdgcn_exp2f(y[h][r]);
    st[h].l += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    if constexpr (kDyn) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float w = e[r] * vm[r >> 2];
        p[h][r] = (_Float16)w;
        if constexpr (kLo) plo[h][r] = (_Float16)(w - (float)p[h][r]);
      }
    } else {
      (void)vm;
#pragma unroll
      for (int r = 0; r < 8; ++r) p[h][r] = (_Float16)e[r];
    }
    (void)plo;
  }
}

// O^T += V^T P^T over a pair: 16 MFMAs (32 with the lo halves, kLo).
template <bool kLo>
__device__ __forceinline__ void pv_pair(const TileRegs<true>& ta, const TileRegs<true>& tb,
                                        const f16x8 (&p)[kHeadsPerWave],
                                        const f16x8 (&plo)[kHeadsPerWave],
                                        RowState (&st)[kHeadsPerWave]) {
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const f16x8 v = v_operand<true>(ta, tb, n);
#pragma unroll
    for (int h = 0; h < kHeadsPerWave; ++h) {
      st[h].acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v, p[h], st[h].acc[n], 0, 0, 0);
      if constexpr (kLo)
        st[h].acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v, plo[h], st[h].acc[n], 0, 0, 0);
    }
  }
  (void)plo;
}

// Per-block scales: while the largest V scale a wave has met (its reference)
// is at most this, every V value it has accumulated is at most 8 in
// magnitude, and rounding each weight once to fp16 (relative error at most
// 2^-11) moves an output by at most 2^-11 * 8 < 4e-3 (the FP8 tolerance is
// 1e-2; the per-tensor kernel has the same bound for its own scale).  The
// reference only grows, so from the first pair past it every pair takes the
// hi + lo products.
constexpr float kHiOnlyVRef = 8.0f / 448.0f;

// Grid (ceil(max chunk / (16 rt)), Hkv, B); rt 16-row tiles of ceil(G / 2)
// waves each per workgroup (a.wpt waves a tile).  Wave v takes heads 2 (v %
// wpt) and 2 (v % wpt) + 1 of tile qt = rt * blockIdx.x + v / wpt; lane (j =
// lane % 16, qg = lane / 16) serves chunk row 16 qt + j of them.  The waves
// of a workgroup share each K/V tile through L1.  kDyn: FP8 pool with
// per-block scales.
template <bool kFP8, bool kDyn = false>
__global__ void __launch_bounds__(512) prefill_kernel(PrefillArgs a) {
  static_assert(kFP8 || !kDyn, "per-block scales are for FP8 pools");
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int w = wv % a.wpt;  // the wave's pair of heads
  const int j = lane & 15, qg = lane >> 4;
  const int qt = blockIdx.x * a.rt + wv / a.wpt, kvh = blockIdx.y, b = blockIdx.z;
  const int q0 = a.query_start[b];
  const int n = a.query_start[b + 1] - q0;
  if (qt * kQT >= n) return;
  int L = a.context_lens[b];
  const int cap = min(a.max_ctx, a.max_blocks * kBS);
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int i = qt * kQT + j;             // this lane's chunk row
  const bool row_ok = i < n;
  const int pos = L - n + i;              // its position; < 0 sees nothing
  const int first = L - n + qt * kQT;     // the workgroup's first position
  const int last = L - n + min(qt * kQT + kQT - 1, n - 1);
  const int h0 = kvh * a.g + w * kHeadsPerWave;

  f16x8 qop[kHeadsPerWave][4];
#pragma unroll
  for (int h = 0; h < kHeadsPerWave; ++h) {
    const bool ok = row_ok && pos >= 0 && w * kHeadsPerWave + h < a.g;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int d0 = kFP8 ? (m >> 1) * 64 + qg * 16 + (m & 1) * 8 : m * 32 + qg * 8;
      qop[h][m] = ok ? *reinterpret_cast<const f16x8*>(
                           a.q + ((int64_t)(q0 + i) * a.hq + h0 + h) * kD + d0)
                     : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  RowState st[kHeadsPerWave];
#pragma unroll
  for (int h = 0; h < kHeadsPerWave; ++h) {
    st[h].m_ref = -INFINITY;
    st[h].l = 0.0f;
#pragma unroll
    for (int nn = 0; nn < 8; ++nn) st[h].acc[nn] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // rows before the sequence (a chunk longer than it) attend to nothing and
  // rows past the chunk are not written; every row computed sees token 0, so
  // its max is finite
  const int pos_c = pos < 0 ? 0 : (pos > L - 1 ? L - 1 : pos);
  const int ntiles = last >= 0 ? last / kBS + 1 : 0;
  float vref = 0.0f;  // per-block scales: the largest V scale seen so far
  float inv_vref = 0.0f;
  const int32_t* trow = a.block_tables + (int64_t)b * a.max_blocks;
  if constexpr (kFP8) {
    // pairs 0 .. np - 1, run two at a time (the buffers alternate); an odd
    // count adds one pair past the last tile, all of it masked
    const int np = (ntiles + 1) >> 1;
    // table entries by scalar loads, from a clamped index so the load is
    // unconditional (no branch splits the block the loads feed)
    auto tile_id = [&](int t) {
      const int v = trow[min(t, ntiles - 1)];
      return t < ntiles ? v : -1;
    };
    // per-block scales of a pair (kDyn), by unconditional scalar loads.  A
    // tile outside the pool (past the sequence's last tile, or an id out of
    // range) reads as zeros; its V scale is 0 and its K scale 1: the causal
    // mask sets such a tile's logits to -inf before the K scale multiplies
    // them, and -inf times 0 would be NaN.
    auto scales = [&](int i, float (&sk)[2], float (&sv)[2]) {
      if constexpr (kDyn) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int id = tile_id(2 * i + t);
          const bool ok = (unsigned)id < (unsigned)a.num_blocks;
          const int64_t o = (int64_t)(ok ? id : 0) * a.hkv + kvh;
          const float ks = a.k_bscale[o], vs = a.v_bscale[o];
          sk[t] = ok ? ks : 1.0f;
          sv[t] = ok ? vs : 0.0f;
        }
      }
    };
    if (np > 0) {
      TileRegs<true> kb[2][2], vb[2][2];
      float sk[2][2] = {{1.f, 1.f}, {1.f, 1.f}}, sv[2][2] = {{1.f, 1.f}, {1.f, 1.f}};
      load_half_pipe<false>(kb[0][0], kb[0][1], a, tile_id(0), tile_id(1), kvh, lane);
      load_half_pipe<true>(vb[0][0], vb[0][1], a, tile_id(0), tile_id(1), kvh, lane);
      load_half_pipe<false>(kb[1][0], kb[1][1], a, tile_id(2), tile_id(3), kvh, lane);
      load_half_pipe<true>(vb[1][0], vb[1][1], a, tile_id(2), tile_id(3), kvh, lane);
      scales(0, sk[0], sv[0]);
      scales(1, sk[1], sv[1]);
      f32x4 s[kHeadsPerWave][2];
      qk_pair(kb[0][0], kb[0][1], qop, s);
      load_half_pipe<false>(kb[0][0], kb[0][1], a, tile_id(4), tile_id(5), kvh, lane);
      if (31 > first) mask_pair(s, 0, qg, pos_c);
      // pair i: K of pair i + 1 in kb[(i + 1) % 2], V of pair i in vb[i % 2],
      // its scales in sk/sv[i % 2]
      // per-block scales: when a tile's V scale exceeds the reference,
      // rescale the accumulators (they hold sum p * (V scale / vref) * code)
      // to the new one
      auto raise_vref = [&](const float (&sa)[2], const float (&sb)[2]) {
        const float ref =
            fmaxf(fmaxf(vref, fmaxf(fmaxf(sa[0], sa[1]), fmaxf(sb[0], sb[1]))), 0x1p-126f);
        if (ref > vref) {  // wave-uniform, rare
          if (vref > 0.0f) {
            const float f = vref / ref;
#pragma unroll
            for (int h = 0; h < kHeadsPerWave; ++h)
#pragma unroll
              for (int nn = 0; nn < 8; ++nn) st[h].acc[nn] *= f;
          }
          vref = ref;
          inv_vref = 1.0f / ref;
        }
      };
      // lo: std::true_type for the hi + lo products (per-block scales with
      // large values), std::false_type otherwise; one straight-line block each
      auto step = [&](auto lo, int i, TileRegs<true> (&kn)[2], TileRegs<true> (&vc)[2],
                      float (&ski)[2], float (&svi)[2]) {
        constexpr bool kLo = decltype(lo)::value;
        const int tb = i * 2 * kBS;
        float qk[2] = {a.qk_scale, a.qk_scale}, vm[2] = {1.0f, 1.0f};
        if constexpr (kDyn) {
          qk[0] = a.qk_scale * ski[0];
          qk[1] = a.qk_scale * ski[1];
          vm[0] = svi[0] * inv_vref;
          vm[1] = svi[1] * inv_vref;
        }
        float y[kHeadsPerWave][8];
        check_pair(s, st, qk, y);
        if (tb + 2 * kBS > L) {  // the sequence's last tiles: slots past L may hold anything
          mask_tail_values<true>(vc[0], tb, qg, L);
          mask_tail_values<true>(vc[1], tb + kBS, qg, L);
        }
        f16x8 p[kHeadsPerWave], plo[kHeadsPerWave];
        probs_pair<kDyn, kLo>(y, st, vm, p, plo);
        qk_pair(kn[0], kn[1], qop, s);
        load_half_pipe<false>(kn[0], kn[1], a, tile_id(2 * i + 6), tile_id(2 * i + 7), kvh, lane);
        pv_pair<kLo>(vc[0], vc[1], p, plo, st);
        load_half_pipe<true>(vc[0], vc[1], a, tile_id(2 * i + 4), tile_id(2 * i + 5), kvh, lane);
        scales(i + 2, ski, svi);
        if (tb + 4 * kBS - 1 > first) {  // pair i + 1 reaches past the first position
          mask_pair(s, tb + 2 * kBS, qg, pos_c);
        }
      };
      // two pairs per iteration (the buffers alternate); with per-block
      // scales the reference is raised to both pairs' V scales first, and
      // the rows run one fp16 product per pair until it passes kHiOnlyVRef,
      // then hi + lo to the end (two loops: no branch inside a pair's block)
      int i = 0;
      if constexpr (kDyn) {
        for (; i < np; i += 2) {
          raise_vref(sv[0], sv[1]);
          if (vref > kHiOnlyVRef) break;  // wave-uniform
          step(std::false_type{}, i, kb[1], vb[0], sk[0], sv[0]);
          step(std::false_type{}, i + 1, kb[0], vb[1], sk[1], sv[1]);
        }
        for (; i < np; i += 2) {
          raise_vref(sv[0], sv[1]);
          step(std::true_type{}, i, kb[1], vb[0], sk[0], sv[0]);
          step(std::true_type{}, i + 1, kb[0], vb[1], sk[1], sv[1]);
        }
      } else {
        for (; i < np; i += 2) {
          step(std::false_type{}, i, kb[1], vb[0], sk[0], sv[0]);
          step(std::false_type{}, i + 1, kb[0], vb[1], sk[1], sv[1]);
        }
      }
    }
  } else {
    // fp16 tiles are twice the registers: one pair at a time, its V halves
    // loaded after its QK^T products
    for (int c0 = 0; c0 < ntiles; c0 += kWave) {
      const int cnt = min(kWave, ntiles - c0);
      const int tbl = lane < cnt ? trow[c0 + lane] : -1;  // lane i: tile c0 + i
      for (int t = 0; t < cnt; t += 2) {
        TileRegs<false> ta, tb;
        const int pa = __builtin_amdgcn_readlane(tbl, t);
        const int pb = t + 1 < cnt ? __builtin_amdgcn_readlane(tbl, t + 1) : pa;
        const bool past = t + 1 >= cnt;     // past the last tile: all masked below
        load_pair_half<false, false>(ta, tb, a, pa, pb, kvh, lane, past);
        const int tok0 = (c0 + t) * kBS;
        process_pair(ta, tb, qop, st, tok0, qg, pos_c, L, tok0 + 2 * kBS - 1 > first,
                     a.qk_scale, VLate{&a, pa, pb, kvh, lane, past});
      }
    }
  }

  if (!row_ok) return;
#pragma unroll
  for (int h = 0; h < kHeadsPerWave; ++h) {
    if (w * kHeadsPerWave + h >= a.g) break;
    float l = st[h].l;
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    const float f = pos < 0 ? 0.0f : (kDyn ? vref : a.out_scale) / l;
    float* o = a.out + ((int64_t)(q0 + i) * a.hq + h0 + h) * kD;
#pragma unroll
    for (int nn = 0; nn < 8; ++nn)
      *reinterpret_cast<f32x4*>(o + nn * 16 + qg * 4) = st[h].acc[nn] * f;
  }
}

// Argument checks and kernel arguments shared by both entry points; with
// per-block scales (k_bscale non-null) the per-tensor scales are not used.
pkv_status plan_prefill(float* out, const void* q, const void* k_pool, const void* v_pool,
                        const float* k_bscale, const float* v_bscale,
                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, const int32_t* query_start,
                        int32_t num_seqs, int32_t num_q_heads, int32_t max_query_len,
                        int32_t max_context_len, const pkv_cache_layout* layout, float sm_scale,
                        float k_scale, float v_scale, PrefillArgs& a, bool& empty) {
  empty = false;
  const pkv_status st = check_layout(layout);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || num_seqs > 65535 || num_q_heads <= 0 || max_query_len < 0 ||
      max_context_len < 0)
    return PKV_ERR_INVALID_ARG;
  if (num_q_heads % layout->num_kv_heads != 0) return PKV_ERR_INVALID_ARG;
  const int32_t G = num_q_heads / layout->num_kv_heads;
  if (G > kMaxG) return PKV_ERR_UNSUPPORTED;
  const bool fp8 = layout->dtype == PKV_FP8_E4M3FN;
  const bool dyn = k_bscale != nullptr;
  if (dyn && !fp8) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0 || max_query_len == 0) {
    empty = true;
    return PKV_OK;
  }
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || !query_start)
    return PKV_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
    return PKV_ERR_INVALID_ARG;
  if (dyn && (!v_bscale || !aligned(k_bscale, 4) || !aligned(v_bscale, 4)))
    return PKV_ERR_INVALID_ARG;
  if (max_blocks_per_seq <= 0 || !std::isfinite(sm_scale) || !(sm_scale > 0.0f))
    return PKV_ERR_INVALID_ARG;
  if (fp8 && !dyn &&
      !(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) && v_scale > 0.0f))
    return PKV_ERR_INVALID_ARG;
  a.out = out;
  a.q = static_cast<const _Float16*>(q);
  a.k_pool = static_cast<const uint8_t*>(k_pool);
  a.v_pool = static_cast<const uint8_t*>(v_pool);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = layout->num_blocks;
  a.hq = num_q_heads;
  a.hkv = layout->num_kv_heads;
  a.g = G;
  a.max_ctx = max_context_len;
  a.qk_scale = sm_scale * (fp8 && !dyn ? k_scale : 1.0f) * 1.4426950408889634f;
  a.out_scale = fp8 && !dyn ? v_scale : 1.0f;
  a.k_bscale = dyn ? k_bscale : nullptr;
  a.v_bscale = dyn ? v_bscale : nullptr;
  return PKV_OK;
}

template <bool kFP8, bool kDyn>
pkv_status launch_prefill(const PrefillArgs& a, int32_t max_query_len, int32_t num_seqs,
                          void* stream) {
  // fp16 tiles: several 16-row tiles per workgroup (up to 8 waves), so each
  // K/V tile is fetched from L2 once for them all: 800 against 770 TFLOP/s
  // on the 128K chunk.  FP8 measured slower that way (987-989 against
  // 1054-1059 TFLOP/s, with the loop that preceded its pipeline): its pairs
  // stay in flight and the loads are not what binds it.
  PrefillArgs c = a;
  c.wpt = (a.g + kHeadsPerWave - 1) / kHeadsPerWave;
  c.rt = kFP8 ? 1 : std::max(1, 8 / c.wpt);
  const int tiles = (max_query_len + kQT - 1) / kQT;
  const dim3 grid((unsigned)((tiles + c.rt - 1) / c.rt), (unsigned)a.hkv, (unsigned)num_seqs);
  (void)hipGetLastError();
  prefill_kernel<kFP8, kDyn>
      <<<grid, dim3(c.wpt * c.rt * kWave), 0, static_cast<hipStream_t>(stream)>>>(c);
  return launch_status();
}

}  // namespace

extern "C" pkv_status pkv_paged_prefill_attention(
    float* out, const void* q, const void* k_pool, const void* v_pool,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* query_start, int32_t num_seqs, int32_t num_q_heads, int32_t max_query_len,
    int32_t max_context_len, const pkv_cache_layout* layout, float sm_scale, float k_scale,
    float v_scale, void* stream) {
  PrefillArgs a;
  bool empty;
  const pkv_status st = plan_prefill(out, q, k_pool, v_pool, nullptr, nullptr, block_tables,
                                     max_blocks_per_seq, context_lens, query_start, num_seqs,
                                     num_q_heads, max_query_len, max_context_len, layout,
                                     sm_scale, k_scale, v_scale, a, empty);
  if (st != PKV_OK || empty) return st;
  const pkv_status chk =
      debug_check_tables(block_tables, max_blocks_per_seq, context_lens, num_seqs,
                         max_context_len, layout->num_blocks, static_cast<hipStream_t>(stream));
  if (chk != PKV_OK) return chk;
  return layout->dtype == PKV_FP8_E4M3FN
             ? launch_prefill<true, false>(a, max_query_len, num_seqs, stream)
             : launch_prefill<false, false>(a, max_query_len, num_seqs, stream);
}

extern "C" pkv_status pkv_paged_prefill_attention_dynamic(
    float* out, const void* q, const void* k_pool, const void* v_pool,
    const float* k_block_scales, const float* v_block_scales, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, const int32_t* query_start,
    int32_t num_seqs, int32_t num_q_heads, int32_t max_query_len, int32_t max_context_len,
    const pkv_cache_layout* layout, float sm_scale, void* stream) {
  if (!k_block_scales || !v_block_scales) return PKV_ERR_INVALID_ARG;
  PrefillArgs a;
  bool empty;
  const pkv_status st = plan_prefill(out, q, k_pool, v_pool, k_block_scales, v_block_scales,
                                     block_tables, max_blocks_per_seq, context_lens,
                                     query_start, num_seqs, num_q_heads, max_query_len,
                                     max_context_len, layout, sm_scale, 1.0f, 1.0f, a, empty);
  if (st != PKV_OK || empty) return st;
  const pkv_status chk =
      debug_check_tables(block_tables, max_blocks_per_seq, context_lens, num_seqs,
                         max_context_len, layout->num_blocks, static_cast<hipStream_t>(stream));
  if (chk != PKV_OK) return chk;
  return launch_prefill<true, true>(a, max_query_len, num_seqs, stream);
}
