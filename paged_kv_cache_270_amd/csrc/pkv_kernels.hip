// pkv_kernels.hip — gfx950 (MI355X) decode kernels and their part of libpkv's
// C ABI: split-KV decode PagedAttention (per-tensor or per-block FP8 scales)
// with its log-sum-exp merge.  The cache writes and block copies are in
// pkv_write.hip, chunked prefill in pkv_prefill.hip, swap in pkv_swap.hip.
//
// Pages the kernels follow (cited by title and section):
//   [FP8-128K] "Optimización de KV Cache con PagedAttention y Cuantización FP8
//              para Contextos Largos (128K)"
//   [PRIMER-8] "LLM Primer VI, Capítulo 8 — Gestión de caché KV de nueva
//              generación"
//
// Design for CDNA4, in short:
//   * one wavefront owns a (sequence, KV head) pair over a run of 16-token
//     blocks and serves all G <= 16 query heads of the group at once: the
//     group's queries form the B operand of a 16x16x32 fp16 MFMA, so each K/V
//     tile is read from HBM once and shared by the whole group in registers;
//   * tiles are stored in the order the MFMA operands consume them (see the
//     layout in pkv.h), so a wave reads a 2 KiB FP8 tile with two 16-byte
//     loads per lane, each instruction covering 1 KiB of contiguous memory;
//   * FP8 codes become fp16 exactly (every E4M3 value is an fp16 value) with
//     the gfx950 conversion instruction; per-tensor scales are folded into
//     the logit scale and the final output, per-block scales into the tile's
//     logits and probabilities, never applied per element;
//   * QK^T gives S^T (tokens x heads) in the accumulator layout that is
//     exactly the B operand of the PV MFMA, so the online softmax runs on
//     registers; its reference max is re-reduced only when a logit exceeds
//     it by a fixed slack;
//   * split-KV: up to eight waves per workgroup share a partition and merge
//     through LDS, or, for short partitions, each wave streams a chain of
//     consecutive partitions and stores each partial from registers;
//     partitions are merged by a second kernel with the log-sum-exp rule.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "pkv.h"
#include "pkv_check.h"
#include "pkv_codec.h"
#include "pkv_tile.h"

namespace {

using namespace pkv_dev;
using namespace pkv_check;

constexpr int kRW = 4;       // waves per merge workgroup

// ----------------------------------------------------------------- decode

struct DecodeArgs {
  float* out;                  // [B][Hq][D]
  const _Float16* q;           // [B][Hq][D]
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const int32_t* block_tables; // [B][max_blocks]
  const int32_t* context_lens; // [B]
  const int32_t* shared_prefix;// [B] or null: leading blocks shared with other sequences
  // Partials, one row per (sequence, KV head, partition, head of the group):
  // the G rows a workgroup or wave stores at a partition's end are adjacent.
  float* ws_ml;                // [B][Hkv][n_p_max][G][2]: running max (log2 units), sum
  float* ws_o;                 // [B][Hkv][n_p_max][G][D]: unnormalised output
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t hq, hkv, g;
  int32_t max_ctx;             // clamp for context lengths
  int32_t part_blocks;         // most blocks per partition (partition_size / 16)
  int32_t n_p_max;
  float qk_scale;              // sm_scale * k_scale * log2(e) [* 256 for FP8 bit dequant]
  float out_scale;             // v_scale [* 256 for FP8 bit dequant]
  const float* k_bscale;       // [num_blocks][hkv] per-block K scales, or null
  const float* v_bscale;       // [num_blocks][hkv] per-block V scales, or null
  // Each sequence's newest token, when the decode call also writes it into
  // the cache (null otherwise): rows [B][Hkv][D] fp16, stored at position
  // L - 1 through the same pools, FP8 as E4M3(x / scale).
  const _Float16* new_k;
  const _Float16* new_v;
  uint8_t* k_wr;
  uint8_t* v_wr;
  float k_enc_scale, v_enc_scale;
  // Cascade over shared prefixes (null casc_prefix otherwise): sequence b's
  // first casc_prefix[b] blocks are attended once for its whole group; the
  // grid's first casc_items z-slices are (group, chunk of casc_m members)
  // items over those blocks, the rest one slice per sequence for its tail.
  const int32_t* casc_prefix;  // [B] prefix blocks of each sequence, 0 = none
  const int32_t* casc_groups;  // [n_groups][casc_cap] member sequences, -1 = none
  int32_t casc_items;          // n_groups * casc_chunks
  int32_t casc_chunks;         // items per group: ceil(casc_cap / casc_mi)
  int32_t casc_cap;            // member slots per group
  int32_t casc_m;              // members per wave: 16 / G, one MFMA column each
  int32_t casc_mi;             // members per item: casc_m, or kNW * casc_m when
                               // the item's waves share its tiles (item_shared)
  int32_t casc_max;            // largest prefix (blocks) the workspace is sized for
  const int32_t* seq_order;    // [B] or null: the sequence of each tail z-slice
  int32_t nseq;                // B
  // Flat cascade grid (casc_flat != 0): one dimension, KV head fastest; the
  // first casc_items * casc_pp units are (item, prefix partition), the rest
  // the tails' partitions in seq_order, each sequence's together.
  int32_t casc_flat;
  int32_t casc_pp;             // prefix partitions per item (flat grid)
  // Flat grid only: the (batch index, tail partition) of each of the
  // casc_tail_count tail units, in schedule order, or null: each workgroup
  // then finds its tail unit by a scan over the lengths.
  const int2* casc_tail_map;
  int32_t casc_tail_count;
};

// Partials are stored write-through to memory (cache policy sc0 sc1, through
// a buffer resource over the G rows of one partition): at 512-token
// partitions this measured about 5% faster for the partition kernel than
// ordinary write-back stores.
constexpr int kWriteThrough = 1 | 16;  // sc0 | sc1

__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rows(float* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000);
}

// Row of the partial of query head g of KV head kvh's group, partition p.
__device__ __forceinline__ int64_t part_row(const DecodeArgs& a, int b, int kvh, int p, int g) {
  return (((int64_t)b * a.hkv + kvh) * a.n_p_max + p) * a.g + g;
}

__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int b) {
  int L = a.context_lens[b];
  const int cap = min(a.max_ctx, a.max_blocks * kBS);
  return L < 0 ? 0 : (L > cap ? cap : L);
}

// Split-KV plan of one sequence: its nblk blocks are cut into
// n_p = ceil(nblk / part_blocks) partitions of equal size (the first ones one
// block longer when it does not divide), so no partition is nearly empty.
struct SeqSplit {
  int nblk, n_p, per;
};

__device__ __forceinline__ SeqSplit seq_split(const DecodeArgs& a, int L) {
  SeqSplit s;
  s.nblk = (L + kBS - 1) / kBS;
  s.n_p = (s.nblk + a.part_blocks - 1) / a.part_blocks;
  s.per = s.n_p > 0 ? (s.nblk + s.n_p - 1) / s.n_p : 0;
  return s;
}

// Cascade: blocks of sequence b (length L) attended by its group's prefix
// items.  0 unless the sequence has a prefix within what the workspace was
// sized for and at least one token after it (so its newest token, and its
// own partition, are in the tail).
__device__ __forceinline__ int casc_blocks(const DecodeArgs& a, int b, int L) {
  if (a.casc_prefix == nullptr) return 0;
  const int S = a.casc_prefix[b];
  return (S > 0 && S <= a.casc_max && S * kBS < L) ? S : 0;
}

// Prefix partitions of a prefix of S blocks: ceil(S / part_blocks), cut
// into equal runs of whole blocks.
__device__ __forceinline__ SeqSplit prefix_split(const DecodeArgs& a, int S) {
  SeqSplit s;
  s.nblk = S;
  s.n_p = (S + a.part_blocks - 1) / a.part_blocks;
  s.per = s.n_p > 0 ? (S + s.n_p - 1) / s.n_p : 0;
  return s;
}

// Partitions whose partials the merge combines for sequence b: without the
// cascade, seq_split's; with it, the prefix's partitions first, then the
// tail's (the blocks after the prefix, split as seq_split splits a sequence).
__device__ __forceinline__ int seq_parts(const DecodeArgs& a, int b, int L) {
  const int S = casc_blocks(a, b, L);
  if (S == 0) return seq_split(a, L).n_p;
  const int tail = (L + kBS - 1) / kBS - S;
  return prefix_split(a, S).n_p + (tail + a.part_blocks - 1) / a.part_blocks;
}

// Flat cascade grid: the (sequence, tail partition) of tail unit j, or
// (-1, -1) past the last one, and in *total the number of tail units.
// Units run through the sequences in seq_order (batch order without one),
// each sequence's partitions together: one unit for an empty sequence (it
// writes zeros), none for an order entry outside the batch.  Every lane of
// the wave takes four sequences of a chunk of 256, counts their units, and a
// wave-wide scan of the counts locates j; the result is the same on every
// wave.
__device__ int2 casc_tail_unit(const DecodeArgs& a, int j, int lane, int* total_out) {
  int base = 0;
  int2 found = make_int2(-1, -1);
  for (int c0 = 0; c0 < a.nseq; c0 += 4 * kWave) {
    int cnt[4], sq[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = c0 + lane * 4 + e;
      int sid = -1;
      if (i < a.nseq) sid = a.seq_order != nullptr ? a.seq_order[i] : i;
      if ((unsigned)sid >= (unsigned)a.nseq) sid = -1;
      sq[e] = sid;
      cnt[e] = 0;
      if (sid >= 0) {
        const int L = clamp_len(a, sid);
        const int S = casc_blocks(a, sid, L);
        cnt[e] = max(seq_split(a, L - S * kBS).n_p, 1);
      }
    }
    const int local = (cnt[0] + cnt[1]) + (cnt[2] + cnt[3]);
    int incl = local;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int y = __shfl_up(incl, d, kWave);
      if (lane >= d) incl += y;
    }
    const int total = __shfl(incl, kWave - 1, kWave);
    const int jj = j - base;
    if (jj >= 0 && jj < total) {  // wave-uniform
      // the first lane whose running count passes jj holds the unit
      const int t = __builtin_ctzll((unsigned long long)__ballot(jj < incl));
      int rem = jj - (__shfl(incl, t, kWave) - __shfl(local, t, kWave));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ce = __shfl(cnt[e], t, kWave);
        const int se = __shfl(sq[e], t, kWave);
        if (rem >= 0 && rem < ce) found = make_int2(se, rem);
        rem -= ce;
      }
    }
    base += total;
  }
  *total_out = base;
  return found;
}

// ------------------------------------------- newest token, written in place
//
// A decode step first stores the new token's K and V rows in its slot
// ([FP8-128K] §4, the cache write) and then attends over the whole
// context, that token included.  The decode kernels do both in one launch.
// The wave that reads the sequence's last block
//   1. loads the token's rows (one dword of K and one of V per lane) with
//      its first block-table load, so they cost no wait of their own;
//   2. once its first tiles are in flight, encodes them (fp16 as they are,
//      FP8 as E4M3(x / scale): the arithmetic of the cache-write kernels)
//      into LDS, in the order its lanes hold tile bytes;
//   3. when the last tile arrives, patches the token's bytes into the tile
//      registers (whatever the load returned for that slot) and stores them
//      to the slot.
// So the attention never depends on when the store lands, the stream does
// not wait for the write, and no separate write launch is needed.
//
// Lane (j, qg) loads, of each tile, K bytes of token j only and V bytes of
// tokens 4qg .. 4qg+3 only (the MFMA operand orders of the tile layout), so
// the token at block offset `off` is K on the lanes j == off and V on the
// lanes qg == off / 4.  Kept bytes in LDS: K at [qg][32 | 64 bytes] (FP8 |
// fp16), V at 256 + [j][8 | 16 bytes].

constexpr int kKeepBytes = 512;  // LDS per workgroup for the kept bytes

// Step 1: lane l's K and V dwords of the new rows (channels 2l, 2l + 1).
__device__ __forceinline__ u32x2 append_load(const DecodeArgs& a, int b, int kvh, int lane) {
  const int64_t row = ((int64_t)b * a.hkv + kvh) * kD;
  u32x2 r;
  r.x = reinterpret_cast<const uint32_t*>(a.new_k + row)[lane];
  r.y = reinterpret_cast<const uint32_t*>(a.new_v + row)[lane];
  return r;
}

// Step 2: encode lane l's four values and place them where patch_tile reads.
template <bool kFP8>
__device__ __forceinline__ void append_keep(const DecodeArgs& a, u32x2 rows, int lane,
                                            uint8_t* keep) {
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int c = 2 * lane + e;                       // channel
    const uint32_t kh = (rows.x >> (16 * e)) & 0xFFFFu;
    const uint32_t vh = (rows.y >> (16 * e)) & 0xFFFFu;
    const int vpos = ((c & 15) * (kFP8 ? 8 : 16)) + (c >> 4) * (kFP8 ? 1 : 2);  // [j][n]
    if constexpr (kFP8) {
      const float kx = (float)__builtin_bit_cast(_Float16, (uint16_t)kh);
      const float vx = (float)__builtin_bit_cast(_Float16, (uint16_t)vh);
      // K channel c = 64i + 16qg + x -> [qg][i][x]
      keep[((c >> 4) & 3) * 32 + (c >> 6) * 16 + (c & 15)] =
          (uint8_t)e4m3_from_f32(kx / a.k_enc_scale);  // correctly rounded fp32 division
      keep[256 + vpos] = (uint8_t)e4m3_from_f32(vx / a.v_enc_scale);
    } else {
      // K channel c = 32m + 8qg + x -> [qg][m][x]
      *reinterpret_cast<uint16_t*>(keep + ((c >> 3) & 3) * 64 + (c >> 5) * 16 + (c & 7) * 2) =
          (uint16_t)kh;
      *reinterpret_cast<uint16_t*>(keep + 256 + vpos) = (uint16_t)vh;
    }
  }
  // other lanes of this wave read these bytes (patch_tile): keep the LDS
  // stores ahead of any later LDS access of the wave
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// Step 3: replace the newest token's bytes in the loaded tile registers by
// the bytes append_keep placed in LDS (whatever the load returned for that
// slot).
template <bool kFP8>
__device__ __forceinline__ void patch_tile(TileRegs<kFP8>& t, const uint8_t* keep, int lane,
                                           int off) {
  const int j = lane & 15, qg = lane >> 4;
  if (j == off) {
#pragma unroll
    for (int i = 0; i < TileRegs<kFP8>::kVecs; ++i)
      t.k[i] = *reinterpret_cast<const u32x4*>(keep + qg * (kFP8 ? 32 : 64) + i * 16);
  }
  if (qg == (off >> 2)) {
    if constexpr (kFP8) {  // byte off % 4 of the dword of channel 16n + j
      const u32x2 kept = *reinterpret_cast<const u32x2*>(keep + 256 + j * 8);
      const uint32_t sh = (off & 3) * 8;
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const uint32_t c = (kept[n >> 2] >> ((n & 3) * 8)) & 0xFFu;
        t.v[n >> 2][n & 3] = (t.v[n >> 2][n & 3] & ~(0xFFu << sh)) | (c << sh);
      }
    } else {  // half off % 4 of the 4 tokens of channel 16n + j (two dwords)
      const u32x4 kept = *reinterpret_cast<const u32x4*>(keep + 256 + j * 16);
      const uint32_t sh = (off & 1) * 16;
      const uint32_t m_lo = (off & 2) ? 0u : (0xFFFFu << sh);
      const uint32_t m_hi = (off & 2) ? (0xFFFFu << sh) : 0u;
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const uint32_t h = ((kept[n >> 1] >> ((n & 1) * 16)) & 0xFFFFu) << sh;
        t.v[n >> 1][(n & 1) * 2] = (t.v[n >> 1][(n & 1) * 2] & ~m_lo) | (h & m_lo);
        t.v[n >> 1][(n & 1) * 2 + 1] = (t.v[n >> 1][(n & 1) * 2 + 1] & ~m_hi) | (h & m_hi);
      }
    }
  }
}

// Step 3's store: the newest token's bytes, from tile registers patched by
// patch_tile, into tile `phys` (a block of the pool) of KV head kvh.
template <bool kFP8>
__device__ __forceinline__ void append_store(const DecodeArgs& a, const TileRegs<kFP8>& t,
                                             int phys, int kvh, int lane, int off) {
  constexpr int kTileBytes = kBS * kD * (kFP8 ? 1 : 2);
  const int j = lane & 15, qg = lane >> 4;
  const int64_t tile = ((int64_t)phys * a.hkv + kvh) * kTileBytes;
  if (j == off) {
#pragma unroll
    for (int i = 0; i < TileRegs<kFP8>::kVecs; ++i)
      *reinterpret_cast<u32x4*>(a.k_wr + tile + i * 1024 + 16 * lane) = t.k[i];
  }
  if (qg == (off >> 2)) {
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      if constexpr (kFP8) {
        a.v_wr[tile + (n >> 2) * 1024 + 16 * lane + (n & 3) * 4 + (off & 3)] =
            (uint8_t)(t.v[n >> 2][n & 3] >> ((off & 3) * 8));
      } else {
        const uint32_t w = (off & 2) ? t.v[n >> 1][(n & 1) * 2 + 1] : t.v[n >> 1][(n & 1) * 2];
        *reinterpret_cast<uint16_t*>(a.v_wr + tile + (n >> 1) * 1024 + 16 * lane +
                                     (n & 1) * 8 + (off & 3) * 2) =
            (uint16_t)(w >> ((off & 1) * 16));
      }
    }
  }
}

// Online-softmax state of one lane: head j, tokens 4qg .. 4qg+3 of each tile.
struct SoftmaxState {
  float m_ref;   // reference max of the head (log2 units), equal on the 4 rows
  float l;       // sum of this lane's probabilities, relative to m_ref
  f32x4 acc[8];  // O^T rows 16n + 4qg .. +3 for head j, relative to m_ref
                 // (and, with per-block scales, in units of vref)
  float vref;    // per-block scales: the largest V scale seen by the wave
};

// One tile: logits, online softmax, PV.  With per-block scales (kDyn) the
// tile's K scale multiplies its logits (k_mul) and its V scale, relative to
// the wave's reference vref, its probabilities (v_mul); the normaliser sums
// the unscaled probabilities.
template <bool kFP8, bool kHwCvt, bool kSplitP, bool kDyn = false>
__device__ __forceinline__ void process_tile(TileRegs<kFP8>& t, const f16x8 (&qop)[4],
                                             SoftmaxState& st, int tb, int qg, int L,
                                             float qk_scale, float k_mul = 1.0f,
                                             float v_mul = 1.0f) {
  if (tb + kBS > L) mask_tail_values<kFP8>(t, tb, qg, L);  // wave-uniform: last tile only
  // S^T[t][g] = sum_d K[t][d] Q[g][d]: 4 MFMAs over the 128 channels
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    f16x8 ka;
    if constexpr (kFP8) {
      const u32x4 raw = t.k[m >> 1];
      const f16x4 lo = dequant4<kHwCvt>((m & 1) ? raw.z : raw.x);
      const f16x4 hi = dequant4<kHwCvt>((m & 1) ? raw.w : raw.y);
      ka = f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      ka = __builtin_bit_cast(f16x8, t.k[m]);
    }
    s = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qop[m], s, 0, 0, 0);
  }
  float sv[4];
  bool over = false;
  const float qk = kDyn ? qk_scale * k_mul : qk_scale;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sv[r] = (tb + qg * 4 + r < L) ? s[r] * qk : -INFINITY;
    over |= sv[r] - st.m_ref > kLazyMaxSlack;
  }
  if (__any(over)) {  // wave-uniform: re-reduce the max and rescale
    float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    bm = fmaxf(bm, __shfl_xor(bm, 16, kWave));
    bm = fmaxf(bm, __shfl_xor(bm, 32, kWave));
    const float m_new = fmaxf(st.m_ref, bm);
    const float alpha = __builtin_amdgcn_exp2f(st.m_ref - m_new);
    st.l *= alpha;
#pragma unroll
    for (int n = 0; n < 8; ++n) st.acc[n] *= alpha;
    st.m_ref = m_new;
  }
  float pr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) pr[r] = __builtin_amdgcn_exp2f(sv[r] - st.m_ref);
  f16x4 ph, pl;
  if constexpr (kDyn) {
    static_assert(kSplitP, "per-block scales use the split probabilities");
    st.l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    float pw[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pw[r] = pr[r] * v_mul;
#pragma unroll
    for (int r = 0; r < 4; ++r) ph[r] = (_Float16)pw[r];
#pragma unroll
    for (int r = 0; r < 4; ++r) pl[r] = (_Float16)(pw[r] - (float)ph[r]);
  } else {
#pragma unroll
  for (int r = 0; r < 4; ++r) ph[r] = (_Float16)pr[r];
  if constexpr (kSplitP) {
    // probabilities as fp16 hi + lo: the PV product keeps about 22 bits
#pragma unroll
    for (int r = 0; r < 4; ++r) pl[r] = (_Float16)(pr[r] - (float)ph[r]);
    st.l += (pr[0] + pr[1]) + (pr[2] + pr[3]);
  } else {
    // the normaliser sums exactly the fp16 weights the PV product uses
    st.l += ((float)ph[0] + (float)ph[1]) + ((float)ph[2] + (float)ph[3]);
  }
  }
  // O^T[d][g] += sum_t V^T[d][t] P^T[t][g]: 8 MFMAs of 16 channels.  With
  // P split into hi + lo the contraction runs over K = 32 = 16 tokens x
  // (hi, lo): lane (j, qg) supplies k = 8qg .. 8qg+7 as its four tokens'
  // values twice (A) against their hi then their lo parts (B), so one
  // 16x16x32 MFMA does the work of two 16x16x16 ones.
  f16x8 pp;
  if constexpr (kSplitP) pp = f16x8{ph[0], ph[1], ph[2], ph[3], pl[0], pl[1], pl[2], pl[3]};
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    f16x4 va;
    if constexpr (kFP8) {
      va = dequant4<kHwCvt>(t.v[n >> 2][n & 3]);
    } else {
      const u32x4 raw = t.v[n >> 1];
      u32x2 two;
      two.x = raw[(n & 1) * 2];
      two.y = raw[(n & 1) * 2 + 1];
      va = __builtin_bit_cast(f16x4, two);
    }
    if constexpr (kSplitP) {
      const f16x8 vv = f16x8{va[0], va[1], va[2], va[3], va[0], va[1], va[2], va[3]};
      st.acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vv, pp, st.acc[n], 0, 0, 0);
    } else {
      st.acc[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, ph, st.acc[n], 0, 0, 0);
    }
  }
}

// A prefix item whose four waves share its tiles (FP8; per-tensor or per-block scales):
// every wave serves its own members (16 MFMA columns) over every tile of the
// item's prefix partition.  Each tile is loaded once per workgroup -- a
// 1 KiB quarter per wave: K bytes 0-1023, K 1024-2047, V 0-1023, V 1024-2047
// -- converted to fp16 and staged in LDS as the fp16 image of each lane's
// 16 bytes (32 bytes per lane), two buffers with one barrier per tile; every
// wave reads the whole tile back in the order the fp16 tile registers hold,
// so the fp16 arithmetic of process_tile applies unchanged.  Compared with an
// item per wave, a tile is loaded and converted once instead of four times.
// The quarters are requested kItemRing tiles ahead, but the loads are
// conditional, so the wait before a tile is staged covers all of them: an
// item advances about one memory round trip per tile.  Letting the ring
// really run ahead (unconditional loads, as in the tails' loop) made the
// cascade launch slower, 182 against 175.5 us on the shared-prefix batch:
// the items then take HBM bandwidth from the tails, whose longest streams
// set the launch's length; a ring of 1 or 2 tiles measured in between.
// The wave stores its members' partials from registers at the end.
constexpr int kItemWaves = 4;
constexpr int kItemRing = 4;
constexpr int kItemBuf = 8192;  // bytes of one staged fp16 tile

// Quarter w of tile `phys` (K bytes 0-1023, K 1024-2047, V 0-1023, V
// 1024-2047 for w = 0..3), through the caches; zeros, with the same load
// instruction and no memory access, when phys is not a pool block.
__device__ __forceinline__ u32x4 item_quarter(const DecodeArgs& a, int phys, int kvh, int w,
                                              int lane) {
  if ((unsigned)phys >= (unsigned)a.num_blocks) return u32x4{0u, 0u, 0u, 0u};
  const uint8_t* pool = w < 2 ? a.k_pool : a.v_pool;
  const u32x4* src = reinterpret_cast<const u32x4*>(
      pool + ((int64_t)phys * a.hkv + kvh) * (kBS * kD) + (w & 1) * 1024);
  return src[lane];  // through the caches: every item of the group reads it
}

__device__ __forceinline__ void item_stage(uint8_t* buf, u32x4 raw, int w, int lane) {
  const f16x4 h0 = dequant4<true>(raw.x), h1 = dequant4<true>(raw.y);
  const f16x4 h2 = dequant4<true>(raw.z), h3 = dequant4<true>(raw.w);
  u32x4* dst = reinterpret_cast<u32x4*>(buf + w * 2048 + 32 * lane);
  dst[0] = __builtin_bit_cast(u32x4, f16x8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]});
  dst[1] = __builtin_bit_cast(u32x4, f16x8{h2[0], h2[1], h2[2], h2[3], h3[0], h3[1], h3[2], h3[3]});
}

template <bool kDyn>
__device__ void item_shared(const DecodeArgs& a, const f16x8 (&qop)[4], SoftmaxState& st,
                            const int32_t* trow, int kvh, int nblk, int pidx, int member,
                            int lane, int w, uint8_t* lds) {
  const int j = lane & 15, qg = lane >> 4;
  // An item's waves share their SIMDs with tail waves, which mostly wait on
  // HBM; the item runs a tile-by-tile dependency chain from L2 in lock step.
  // Issuing it first keeps it from holding its slot for the whole launch.
  __builtin_amdgcn_s_setprio(2);
  int g = 0;  // tiles staged so far: the parity of the LDS buffer
  for (int c0 = 0; c0 < nblk; c0 += kWave) {
    const int cnt = min(kWave, nblk - c0);
    const int tbl = lane < cnt ? trow[c0 + lane] : 0;
    // per-block scales, as the tails take them: lane i holds tile c0 + i's K
    // scale and its V scale relative to the wave's reference
    float k_mul = 1.0f, v_mul = 1.0f;
    if constexpr (kDyn) {
      float ks = 0.0f, vs = 0.0f;
      if (lane < cnt && (unsigned)tbl < (unsigned)a.num_blocks) {
        ks = a.k_bscale[(int64_t)tbl * a.hkv + kvh];
        vs = a.v_bscale[(int64_t)tbl * a.hkv + kvh];
      }
      const float ref = fmaxf(fmaxf(st.vref, wave_max(vs)), 0x1p-126f);
      if (ref > st.vref && st.vref > 0.0f) {  // wave-uniform: rescale what is accumulated
        const float f = st.vref / ref;
#pragma unroll
        for (int n = 0; n < 8; ++n) st.acc[n] *= f;
      }
      st.vref = ref;
      k_mul = ks;
      v_mul = vs / ref;
    }
    u32x4 raw[kItemRing];
#pragma unroll
    for (int r = 0; r < kItemRing; ++r)
      if (r < cnt) raw[r] = item_quarter(a, __builtin_amdgcn_readlane(tbl, r), kvh, w, lane);
    item_stage(lds + (g & 1) * kItemBuf, raw[0], w, lane);
    if (kItemRing < cnt)
      raw[0] = item_quarter(a, __builtin_amdgcn_readlane(tbl, kItemRing), kvh, w, lane);
    for (int base = 0; base < cnt; base += kItemRing) {
#pragma unroll
      for (int r = 0; r < kItemRing; ++r) {
        const int ii = base + r;
        if (ii < cnt) {
          __syncthreads();  // tile ii staged; the other buffer is free
          const uint8_t* buf = lds + (g & 1) * kItemBuf;
          TileRegs<false> t;
#pragma unroll
          for (int m = 0; m < 4; ++m)
            t.k[m] = *reinterpret_cast<const u32x4*>(buf + (m >> 1) * 2048 + 32 * lane +
                                                     16 * (m & 1));
#pragma unroll
          for (int q = 0; q < 4; ++q)
            t.v[q] = *reinterpret_cast<const u32x4*>(buf + (2 + (q >> 1)) * 2048 + 32 * lane +
                                                     16 * (q & 1));
          // prefix tokens are all valid: L is the prefix length
          if constexpr (kDyn)
            process_tile<false, true, true, true>(
                t, qop, st, 0, qg, kBS, a.qk_scale,
                __int_as_float(__builtin_amdgcn_readlane(__float_as_int(k_mul), ii)),
                __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v_mul), ii)));
          else
            process_tile<false, true, true>(t, qop, st, 0, qg, kBS, a.qk_scale);
          ++g;
          if (ii + 1 < cnt) {
            const int kNext = (r + 1) % kItemRing;  // static once unrolled
            item_stage(lds + (g & 1) * kItemBuf, raw[kNext], w, lane);
            if (ii + 1 + kItemRing < cnt)
              raw[kNext] = item_quarter(a, __builtin_amdgcn_readlane(tbl, ii + 1 + kItemRing),
                                        kvh, w, lane);
          }
        }
      }
    }
  }
  __builtin_amdgcn_s_setprio(0);
  if constexpr (kDyn) {  // back from units of the wave's V reference
#pragma unroll
    for (int n = 0; n < 8; ++n) st.acc[n] *= st.vref;
  }
  // the members' partials, straight from registers
  float l_run = st.l;
  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);
  if (member >= 0) {
    const int64_t prow = part_row(a, member, kvh, pidx, j % a.g);
    float* dst = a.ws_o + prow * kD + qg * 4;
#pragma unroll
    for (int n = 0; n < 8; ++n) *reinterpret_cast<f32x4*>(dst + n * 16) = st.acc[n];
    if (qg == 0) {
      a.ws_ml[prow * 2] = st.m_ref;
      a.ws_ml[prow * 2 + 1] = l_run;
    }
  }
}

// One unit of the decode partition kernel: partition p of KV head kvh of
// z-slice b, kNW waves.  The unit covers tokens [p*P, min(L, (p+1)*P)) of
// sequence b for the G query heads of KV head kvh.  Wave w takes the
// partition's blocks w, w + kNW, ...  Lane (j = lane % 16, qg = lane / 16)
// serves query head kvh*G + j and, in each tile, tokens 4qg .. 4qg+3.  Each
// wave keeps kPD tiles in flight while it computes on another.
// kAppend: the unit also writes the sequence's newest token (steps 1-3
// above).  kCasc: the cascade over shared prefixes -- z-slices below
// casc_items are prefix items, the rest sequences, through seq_order unless
// `ordered` says b - casc_items is the sequence itself.  Every return below
// is uniform over the workgroup.
template <bool kFP8, bool kHwCvt, bool kSplitP, int kPD, int kNW, bool kDyn, bool kAppend,
          bool kCasc>
__device__ __forceinline__ void partition_unit(const DecodeArgs& a, float* smem, int p, int kvh,
                                               int b, bool ordered) {
  // [kNW][CS][D] outputs, then [kNW][16] max and sum, then (kAppend) the
  // newest token's kept bytes, then (kCasc) the item's member per column
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int j = lane & 15;
  const int qg = lane >> 4;
  const int G = a.g;
  const int CS = kCasc ? kMaxG : G;  // LDS merge: columns per wave
  int* memb = reinterpret_cast<int*>(smem + kNW * CS * kD + 2 * kNW * 16 + kKeepBytes / 4);

  int L, n_p, pidx, blk0, nblk, ncol = G, shared_blocks;
  bool item = false;
  int item_member = -1;  // a prefix item: the member of this lane's column
  // prefix items whose waves share the tiles (item_shared)
  constexpr bool kSharedItem = kCasc && kFP8 && kNW == kItemWaves;
  int qrow = -1;       // this lane's query row [B*Hq], -1 = column unused
  if constexpr (kCasc) {
    if (b < a.casc_items) {
      // A prefix item: up to casc_m members of one group, G columns each,
      // over partition p of the group's prefix blocks (whole blocks, every
      // token valid).  Members whose prefix differs are left out.
      item = true;
      const int gi = b / a.casc_chunks, ch = b - gi * a.casc_chunks;
      const int32_t* grp = a.casc_groups + (int64_t)gi * a.casc_cap;
      const int lead = grp[0];
      if ((unsigned)lead >= (unsigned)a.nseq) return;
      const int S = casc_blocks(a, lead, clamp_len(a, lead));
      if (S == 0) return;
      const SeqSplit ps = prefix_split(a, S);
      if (p >= ps.n_p) return;
      b = lead;
      L = S * kBS;
      n_p = 2;  // never the only partition: partials are always stored
      pidx = p;
      blk0 = p * ps.per;
      nblk = min(S, blk0 + ps.per) - blk0;
      ncol = a.casc_m * G;
      shared_blocks = S;  // every item of the group reads these tiles
      const int slot = ch * a.casc_mi + (kSharedItem ? w * a.casc_m : 0) + j / G;
      int m = -1;
      if (j < ncol && slot < a.casc_cap) {
        m = grp[slot];
        if ((unsigned)m >= (unsigned)a.nseq || casc_blocks(a, m, clamp_len(a, m)) != S) m = -1;
      }
      if (m >= 0) qrow = m * a.hq + kvh * G + (j - (j / G) * G);
      item_member = m;
      if (w == 0 && qg == 0) memb[j] = m;
    } else {
      b -= a.casc_items;
      if (a.seq_order != nullptr && !ordered) {  // tails in the caller's order (longest first)
        b = a.seq_order[b];
        if ((unsigned)b >= (unsigned)a.nseq) return;
      }
    }
  }
  if (!item) {
    L = clamp_len(a, b);
    int S = 0;
    if constexpr (kCasc) S = casc_blocks(a, b, L);
    // the blocks after the prefix (all of them without one), split evenly
    const SeqSplit sp = seq_split(a, L - S * kBS);
    const int n_pp = S > 0 ? prefix_split(a, S).n_p : 0;
    n_p = n_pp + sp.n_p;
    if (p >= sp.n_p) {
      if (p == 0) {  // empty sequence: attention over nothing is defined as zeros
        const int64_t head0 = (int64_t)b * a.hq + (int64_t)kvh * G;
        for (int i = threadIdx.x; i < G * kD; i += kNW * kWave) a.out[head0 * kD + i] = 0.0f;
      }
      return;
    }
    pidx = n_pp + p;
    blk0 = S + p * sp.per;
    nblk = min(S + sp.nblk, blk0 + sp.per) - blk0;
    shared_blocks = a.shared_prefix != nullptr ? a.shared_prefix[b] : 0;
    if (j < G) qrow = b * a.hq + kvh * G + j;
  }
  const int64_t head0 = (int64_t)b * a.hq + (int64_t)kvh * G;  // first query head of the group

  // Query heads of the group as the MFMA B operand, in the channel order the
  // K tile registers hold (FP8: runs of 16 channels; fp16: runs of 8).
  f16x8 qop[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (qrow >= 0) {
      const int d0 = kFP8 ? (m >> 1) * 64 + qg * 16 + (m & 1) * 8 : m * 32 + qg * 8;
      qop[m] = *reinterpret_cast<const f16x8*>(a.q + (int64_t)qrow * kD + d0);
    } else {
      qop[m] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  SoftmaxState st;
  st.m_ref = -INFINITY;
  st.l = 0.0f;
  st.vref = 0.0f;
#pragma unroll
  for (int n = 0; n < 8; ++n) st.acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  if constexpr (kSharedItem) {
    if (item) {  // workgroup-uniform
      item_shared<kDyn>(a, qop, st, a.block_tables + (int64_t)b * a.max_blocks + blk0, kvh,
                        nblk, pidx, item_member, lane, w, reinterpret_cast<uint8_t*>(smem));
      return;
    }
  }

  const int my_n = w < nblk ? (nblk - w + kNW - 1) / kNW : 0;
  const int32_t* trow = a.block_tables + (int64_t)b * a.max_blocks + blk0 + w;

  // The sequence's last block is the last tile of wave (nblk - 1) % kNW of
  // the last partition: that wave writes the newest token and patches it
  // into its tile my_n - 1.
  uint8_t* keep = reinterpret_cast<uint8_t*>(smem + kNW * CS * kD + 2 * kNW * 16);
  int patch_at = -1;
  if constexpr (kAppend) {
    if (!item && pidx == n_p - 1 && w == (nblk - 1) % kNW) patch_at = my_n - 1;
    patch_at = __builtin_amdgcn_readfirstlane(patch_at);
  }

  // Logical blocks below shared_blocks are read by other sequences or items
  // too (cache hint).  A chunk ends where this wave's shared tiles end, so
  // each chunk takes one cache policy.
  const int n_sh = min(my_n, max(0, shared_blocks - blk0 - w + kNW - 1) / kNW);
  int cnt = 0;
  for (int c0 = 0; c0 < my_n; c0 += cnt) {
    cnt = min(kWave, (c0 < n_sh ? n_sh : my_n) - c0);
    // the newest token's rows, issued ahead of the table load whose wait
    // then covers them too
    u32x2 rows = u32x2{0u, 0u};
    if constexpr (kAppend)
      if (c0 == 0 && patch_at >= 0) rows = append_load(a, b, kvh, lane);
    // lane i holds the physical id of this wave's block c0 + i
    const int tbl = load_table(trow + (int64_t)c0 * kNW, cnt, kNW, lane);
    const int lb0 = blk0 + w + c0 * kNW;  // logical block of this chunk's tile 0
    // per-block scales: lane i holds block i's K scale and its V scale
    // relative to the wave's reference (the largest V scale so far)
    float k_mul = 1.0f, v_mul = 1.0f;
    if constexpr (kDyn) {
      float ks = 0.0f, vs = 0.0f;
      if (lane < cnt && (unsigned)tbl < (unsigned)a.num_blocks) {
        ks = a.k_bscale[(int64_t)tbl * a.hkv + kvh];
        vs = a.v_bscale[(int64_t)tbl * a.hkv + kvh];
      }
      const float ref = fmaxf(fmaxf(st.vref, wave_max(vs)), 0x1p-126f);
      if (ref > st.vref && st.vref > 0.0f) {  // wave-uniform: rescale what is accumulated
        const float f = st.vref / ref;
#pragma unroll
        for (int n = 0; n < 8; ++n) st.acc[n] *= f;
      }
      st.vref = ref;
      k_mul = ks;
      v_mul = vs / ref;
    }
    // Every tile slot issues its loads, past the chunk's end too (a tile
    // that is not there loads zeros without touching memory), so the waits
    // for a tile never cover the prefetch issued after it.  The chunk's
    // tiles take one cache policy: through the caches when all of them are
    // shared (below shared_blocks), streamed otherwise.
    auto chunk = [&](auto policy) {
      constexpr int kAux = decltype(policy)::value;
      TileRegs<kFP8> buf[kPD + 1];
#pragma unroll
      for (int r = 0; r < kPD; ++r)
        load_tile<kFP8, kAux>(buf[r], a.k_pool, a.v_pool, a.num_blocks, a.hkv,
                              r < cnt ? __builtin_amdgcn_readlane(tbl, r) : -1, kvh, lane);
      if constexpr (kAppend)
        if (c0 == 0 && patch_at >= 0) append_keep<kFP8>(a, rows, lane, keep);
      for (int base = 0; base < cnt; base += kPD + 1) {
#pragma unroll
        for (int r = 0; r <= kPD; ++r) {
          const int ii = base + r;
          const int nx = ii + kPD;
          load_tile<kFP8, kAux>(buf[(r + kPD) % (kPD + 1)], a.k_pool, a.v_pool, a.num_blocks,
                                a.hkv, nx < cnt ? __builtin_amdgcn_readlane(tbl, nx) : -1, kvh,
                                lane);
          if (ii < cnt) {
            const int tb = (blk0 + w + (c0 + ii) * kNW) * kBS;  // first token of the tile
            if constexpr (kAppend)
              if (c0 + ii == patch_at) {
                const int phys = __builtin_amdgcn_readlane(tbl, ii);
                if ((unsigned)phys < (unsigned)a.num_blocks) {  // else nothing is written
                  patch_tile<kFP8>(buf[r], keep, lane, (L - 1) & 15);
                  append_store<kFP8>(a, buf[r], phys, kvh, lane, (L - 1) & 15);
                }
              }
            if constexpr (kDyn)
              process_tile<kFP8, kHwCvt, kSplitP, true>(
                  buf[r], qop, st, tb, qg, L, a.qk_scale,
                  __int_as_float(__builtin_amdgcn_readlane(__float_as_int(k_mul), ii)),
                  __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v_mul), ii)));
            else
              process_tile<kFP8, kHwCvt, kSplitP>(buf[r], qop, st, tb, qg, L, a.qk_scale);
          }
        }
      }
    };
    if constexpr (kSharedItem) {
      chunk(std::integral_constant<int, kLoadNT>{});  // a tail: the prefix is the items'
    } else {
      if (lb0 + (cnt - 1) * kNW < shared_blocks)
        chunk(std::integral_constant<int, 0>{});
      else
        chunk(std::integral_constant<int, kLoadNT>{});
    }
  }

  // each head's sum over its four token rows
  float l_run = st.l;
  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);

  if constexpr (kDyn) {  // back from units of the wave's V reference
#pragma unroll
    for (int n = 0; n < 8; ++n) st.acc[n] *= st.vref;
  }

  // merge the kNW waves through LDS
  float* so = smem;                        // [kNW][CS][D]
  float* sm = smem + kNW * CS * kD;        // [kNW][16]
  float* sl = sm + kNW * 16;               // [kNW][16]
  if (j < ncol) {
#pragma unroll
    for (int n = 0; n < 8; ++n)
      *reinterpret_cast<f32x4*>(so + (w * CS + j) * kD + n * 16 + qg * 4) = st.acc[n];
    if (qg == 0) {
      sm[w * 16 + j] = st.m_ref;
      sl[w * 16 + j] = l_run;
    }
  }
  __syncthreads();
  const bool single = n_p == 1;
  // the G rows of this partition's partial output (not used when single,
  // nor by a prefix item, whose columns belong to several sequences)
  const __amdgpu_buffer_rsrc_t orows = partial_rows(
      single || item ? nullptr : a.ws_o + part_row(a, b, kvh, pidx, 0) * kD, G * kD * 4);
  for (int i = threadIdx.x; i < ncol * kD; i += kNW * kWave) {
    const int gg = i / kD, d = i - gg * kD;
    float mx = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kNW; ++ww) mx = fmaxf(mx, sm[ww * 16 + gg]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kNW; ++ww) {
      const float f = __builtin_amdgcn_exp2f(sm[ww * 16 + gg] - mx);
      num += so[(ww * CS + gg) * kD + d] * f;
      den += sl[ww * 16 + gg] * f;
    }
    const int64_t hrow = head0 + gg;
    if constexpr (kCasc) {
      if (item) {  // column gg: head gg % G of member gg / G
        const int m = memb[gg];
        if (m >= 0) {
          const int64_t prow = part_row(a, m, kvh, pidx, gg % G);
          a.ws_o[prow * kD + d] = num;
          if (d == 0) {
            a.ws_ml[prow * 2] = mx;
            a.ws_ml[prow * 2 + 1] = den;
          }
        }
        continue;
      }
    }
    if (single) {
      a.out[hrow * kD + d] = num / den * a.out_scale;
    } else {
      const int64_t prow = part_row(a, b, kvh, pidx, gg);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(num), orows, i * 4, 0, kWriteThrough);
      if (d == 0) {
        a.ws_ml[prow * 2] = mx;
        a.ws_ml[prow * 2 + 1] = den;
      }
    }
  }
}

// With per-block scales, and for the FP8 cascade, the kernel is held to 168
// VGPRs (3 waves per SIMD).  The per-block-scale variant fits in about 150
// without spilling; held to 128 (4 waves), it spilled once the next tile's
// loads stayed in flight across the current tile's arithmetic.  The cascade's
// loop over units of the flat grid otherwise grows it past 168.  The FP8
// cascade with fewer than kItemWaves waves (short partitions; its items then
// do not share their tiles) needs more than 168 and is held to 256 (2 waves
// per SIMD) instead of spilling.
// Decode partition kernel: one unit per workgroup, grid (n_p_max, Hkv, B) or
// (n_p_max, Hkv, items + B) for the cascade; or, with the cascade's flat
// grid, Hkv * n workgroups, KV head fastest: workgroup i takes unit i / Hkv
// and then every n-th unit after it until none is left, so the grid may hold
// exactly the units there are (the host's count) or any other number.
template <bool kFP8, bool kHwCvt, bool kSplitP, int kPD, int kNW, bool kDyn = false,
          bool kAppend = false, bool kCasc = false>
__global__ void __launch_bounds__(kNW * kWave)
__attribute__((amdgpu_waves_per_eu((kCasc && kFP8 && kNW < kItemWaves)
                                       ? 2
                                       : (kDyn || (kCasc && kFP8) ? 3 : 1))))
decode_partition_kernel(DecodeArgs a) {
  extern __shared__ float smem[];
  if constexpr (kCasc) {
    if (a.casc_flat) {
      const int lane = threadIdx.x & 63;
      const int n_wg = gridDim.x / a.hkv;
      const int kvh = blockIdx.x % a.hkv;
      const int iu = a.casc_items * a.casc_pp;
      int tails = -1;  // tail units, once a scan has counted them
      for (int u = blockIdx.x / a.hkv;; u += n_wg) {
        int b, p;
        bool ordered = false;
        if (u < iu) {
          b = u / a.casc_pp;
          p = u - b * a.casc_pp;
        } else {
          if (tails >= 0 && u - iu >= tails) break;  // past the last unit (uniform)
          int2 unit;
          if (a.casc_tail_map != nullptr) {
            // the host's map: one load instead of the scan's two dependent
            // round trips (an entry outside the batch is skipped)
            tails = a.casc_tail_count;
            if (u - iu >= tails) break;
            unit = a.casc_tail_map[u - iu];
            if ((unsigned)unit.x >= (unsigned)a.nseq || unit.y < 0) unit = make_int2(-1, 0);
          } else {
            unit = casc_tail_unit(a, u - iu, lane, &tails);
          }
          // the same on every lane: say so, so that everything derived from
          // them stays in scalar registers
          unit.x = __builtin_amdgcn_readfirstlane(unit.x);
          unit.y = __builtin_amdgcn_readfirstlane(unit.y);
          tails = __builtin_amdgcn_readfirstlane(tails);
          if (unit.x < 0 && a.casc_tail_map == nullptr) break;  // the scan found no unit
          b = unit.x < 0 ? -1 : a.casc_items + unit.x;
          p = unit.y;
          ordered = true;
        }
        if (b >= 0)
          partition_unit<kFP8, kHwCvt, kSplitP, kPD, kNW, kDyn, kAppend, kCasc>(a, smem, p, kvh,
                                                                                b, ordered);
        // a launch that holds every unit needs no second pass
        if (tails >= 0 && u + n_wg - iu >= tails) break;
        __syncthreads();  // the next unit reuses the LDS
      }
      return;
    }
  }
  partition_unit<kFP8, kHwCvt, kSplitP, kPD, kNW, kDyn, kAppend, kCasc>(
      a, smem, blockIdx.x, blockIdx.y, blockIdx.z, false);
}

// The same partition unit with both contractions on the vector ALUs instead
// of the matrix cores -- kept to measure that choice (PKV_DECODE_MATH=valu).
// FP8, per-tensor scales, G <= 8 (groups of fewer heads compute eight, the
// missing ones on zero queries); grid (n_p_max, Hkv, B), kValuWaves waves,
// wave w taking the partition's blocks w, w + kValuWaves, ...  One tile in
// flight besides the one being computed, as in the default family.  One
// cache policy per launch (kAux): through the caches when the caller names
// shared prefixes, streamed otherwise -- a per-chunk choice, as the
// partition kernel makes it, cost this kernel 67 more VGPRs.
//  * QK^T: lane (cg, hg, tp) = lane / 16, lane / 8 % 2, lane % 8 takes
//    tokens tp and tp + 8, heads 4hg .. 4hg+3 and the 32 channels 16cg ..
//    16cg+15, 64 + 16cg .. 64 + 16cg + 15.  It loads those K bytes itself
//    (the two lanes of a (cg, tp) pair read the same bytes; each load
//    instruction covers whole 128-byte lines), converts them to fp16 and
//    takes 2-element dot products with fp32 sums against the same channels
//    of its four queries, which stay in registers (64 VGPRs).  A
//    reduce-scatter over cg then leaves it the full logits of token
//    tp + 8 (cg / 2), heads 4hg + 2 (cg % 2) and the next.
//  * Softmax: the partition kernel's reference-max scheme, per head.
//  * PV: lane (j, qg) = lane % 16, lane / 16 holds channels 16c + j
//    (c = 0..7), tokens 4qg .. +3 of the V tile (the tile load's layout).  It
//    reads its four tokens' probabilities of all eight heads from an LDS row
//    the lanes wrote, and accumulates 8 heads x 8 channels in fp32 fused
//    multiply-adds on the values converted to fp32 exactly.
constexpr int kValuG = 8;
constexpr int kValuWaves = 4;

struct ValuTile {
  u32x4 k[4];  // [i][token tp + 8tt]: channels 64i + 16cg .. +15
  u32x4 v[2];  // as TileRegs<true>::v
};

template <int kAux>
__device__ __forceinline__ void valu_load(ValuTile& r, const DecodeArgs& a, int phys, int kvh,
                                          int koff, int lane) {
  constexpr int kTileBytes = kBS * kD;
  phys = __builtin_amdgcn_readfirstlane(phys);
  kvh = __builtin_amdgcn_readfirstlane(kvh);
  const bool ok = (unsigned)phys < (unsigned)a.num_blocks;
  const int64_t off = ok ? ((int64_t)phys * a.hkv + kvh) * kTileBytes : 0;
  const __amdgpu_buffer_rsrc_t kr = byte_range(a.k_pool + off, ok ? kTileBytes : 0);
  const __amdgpu_buffer_rsrc_t vr = byte_range(a.v_pool + off, ok ? kTileBytes : 0);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
      r.k[2 * i + tt] =
          __builtin_amdgcn_raw_buffer_load_b128(kr, i * 1024 + koff + tt * 128, 0, kAux);
    r.v[i] = __builtin_amdgcn_raw_buffer_load_b128(vr, (i * kWave + lane) * 16, 0, kAux);
  }
}

template <int kAux>
__global__ void __launch_bounds__(kValuWaves * kWave) decode_valu_kernel(DecodeArgs a) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  constexpr int kNW = kValuWaves;
  extern __shared__ float smem[];                 // [kNW][G][D], [kNW][16] max, [kNW][16] sum
  __shared__ __align__(16) float pst[kNW][kBS * kValuG];  // per wave: p[token][head]
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // QK^T roles
  const int tp = lane & 7, hg = (lane >> 3) & 1, cg = lane >> 4;
  const int b0 = cg & 1, b1 = cg >> 1;
  const int hsel = 2 * hg + b0;  // this lane's logits: heads 2 hsel, 2 hsel + 1
  // PV roles
  const int j = lane & 15, qg = lane >> 4;
  const int p = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = a.g;
  const int L = clamp_len(a, b);
  const SeqSplit sp = seq_split(a, L);
  const int64_t head0 = (int64_t)b * a.hq + (int64_t)kvh * G;
  if (p >= sp.n_p) {
    if (p == 0)
      for (int i = threadIdx.x; i < G * kD; i += kNW * kWave) a.out[head0 * kD + i] = 0.0f;
    return;
  }
  const int n_p = sp.n_p;
  const int blk0 = p * sp.per;
  const int nblk = min(sp.nblk, blk0 + sp.per) - blk0;
  const int koff = cg * 256 + tp * 16;

  // queries 4hg .. 4hg+3: channels 64i + 16cg .. +15 as 8 fp16 pairs per i
  h2 q[4][16];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int g = 4 * hg + h;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        f16x8 v = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
        if (g < G)
          v = *reinterpret_cast<const f16x8*>(a.q + (head0 + g) * kD + 64 * i + 16 * cg + 8 * x);
#pragma unroll
        for (int e = 0; e < 4; ++e) q[h][i * 8 + x * 4 + e] = h2{v[2 * e], v[2 * e + 1]};
      }
    }
  }

  float acc[kValuG][8];  // head g, channel 16c + j, over this lane's tokens
#pragma unroll
  for (int g = 0; g < kValuG; ++g)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[g][c] = 0.0f;
  // heads 2hsel, 2hsel + 1: reference max (equal on the lanes of the head)
  // and the sum over this lane's tokens
  float m0 = -INFINITY, m1 = -INFINITY;
  float l0 = 0.0f, l1 = 0.0f;
  float* prow = &pst[w][0];

  auto tile = [&](ValuTile& t, int tb) {
    if (tb + kBS > L) {  // wave-uniform: zero the values of tokens >= L
      const int nv = min(max(L - (tb + qg * 4), 0), 4);
      const uint32_t mk = nv >= 4 ? 0xFFFFFFFFu : ((1u << (8 * nv)) - 1u);
#pragma unroll
      for (int i = 0; i < 2; ++i) t.v[i] &= u32x4{mk, mk, mk, mk};
    }
    float s[2][4];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int h = 0; h < 4; ++h) s[tt][h] = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int d = (int)t.k[2 * i + tt][c];
          const h2 k01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d, 1.0f, false);
          const h2 k23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d, 1.0f, true);
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            s[tt][h] = __builtin_amdgcn_fdot2(k01, q[h][8 * i + 2 * c], s[tt][h], false);
            s[tt][h] = __builtin_amdgcn_fdot2(k23, q[h][8 * i + 2 * c + 1], s[tt][h], false);
          }
        }
    // reduce-scatter over cg: across cg bit 1 (lanes 32 apart) keeping token
    // tp + 8b1, then across bit 0 keeping heads 4hg + 2b0, +1
    float r4[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float keep = b1 ? s[1][h] : s[0][h];
      const float give = b1 ? s[0][h] : s[1][h];
      r4[h] = keep + __shfl_xor(give, 32, kWave);
    }
    float r2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float keep = b0 ? r4[2 + e] : r4[e];
      const float give = b0 ? r4[e] : r4[2 + e];
      r2[e] = keep + __shfl_xor(give, 16, kWave);
    }
    const int tok = tp + 8 * b1;
    const bool valid = tb + tok < L;
    const float s0 = valid ? r2[0] * a.qk_scale : -INFINITY;
    const float s1 = valid ? r2[1] * a.qk_scale : -INFINITY;
    if (__any(s0 - m0 > kLazyMaxSlack || s1 - m1 > kLazyMaxSlack)) {  // wave-uniform
      // the lanes of one head pair differ in tp and b1
      float x0 = s0, x1 = s1;
#pragma unroll
      for (int x = 1; x <= 32; x <<= 1) {
        if (x == 8 || x == 16) continue;
        x0 = fmaxf(x0, __shfl_xor(x0, x, kWave));
        x1 = fmaxf(x1, __shfl_xor(x1, x, kWave));
      }
      const float n0 = fmaxf(m0, x0), n1 = fmaxf(m1, x1);
      const float f0 = __builtin_amdgcn_exp2f(m0 - n0), f1 = __builtin_amdgcn_exp2f(m1 - n1);
      l0 *= f0;
      l1 *= f1;
      m0 = n0;
      m1 = n1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {  // heads 2e, 2e + 1: hsel = e on lane 16 (e % 2) + 8 (e / 2)
        const int src = 16 * (e & 1) + 8 * (e >> 1);
        const float g0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f0), src));
        const float g1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f1), src));
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          acc[2 * e][c] *= g0;
          acc[2 * e + 1][c] *= g1;
        }
      }
    }
    const float p0 = __builtin_amdgcn_exp2f(s0 - m0);
    const float p1 = __builtin_amdgcn_exp2f(s1 - m1);
    l0 += p0;
    l1 += p1;
    // p[tok][2 hsel, 2 hsel + 1]; one wave writes and then reads its own row
    *reinterpret_cast<f2*>(prow + tok * kValuG + 2 * hsel) = f2{p0, p1};
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {  // tokens 4qg + 2rr, +1
      float pp[2][kValuG];
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const f32x4 v4 =
              *reinterpret_cast<const f32x4*>(prow + (4 * qg + 2 * rr + r) * kValuG + 4 * x);
#pragma unroll
          for (int e = 0; e < 4; ++e) pp[r][4 * x + e] = v4[e];
        }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int d = (int)t.v[c >> 2][c & 3];
        const f2 v = rr ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d, 1.0f, true)
                        : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d, 1.0f, false);
#pragma unroll
        for (int g = 0; g < kValuG; ++g) {
          acc[g][c] = __builtin_fmaf(pp[0][g], v[0], acc[g][c]);
          acc[g][c] = __builtin_fmaf(pp[1][g], v[1], acc[g][c]);
        }
      }
    }
    // the next tile's writes come after every lane's reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  const int my_n = w < nblk ? (nblk - w + kNW - 1) / kNW : 0;
  const int32_t* trow = a.block_tables + (int64_t)b * a.max_blocks + blk0 + w;
  for (int c0 = 0; c0 < my_n; c0 += kWave) {
    const int cnt = min(kWave, my_n - c0);
    const int tbl = load_table(trow + (int64_t)c0 * kNW, cnt, kNW, lane);
    const int lb0 = blk0 + w + c0 * kNW;
    ValuTile buf[2];
    valu_load<kAux>(buf[0], a, __builtin_amdgcn_readlane(tbl, 0), kvh, koff, lane);
    for (int base = 0; base < cnt; base += 2) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int ii = base + r;
        valu_load<kAux>(buf[r ^ 1], a, ii + 1 < cnt ? __builtin_amdgcn_readlane(tbl, ii + 1) : -1,
                        kvh, koff, lane);
        if (ii < cnt) tile(buf[r], (lb0 + ii * kNW) * kBS);
      }
    }
  }

  // sums over the lanes of each head pair (tp, b1); outputs over qg by the
  // reduce-scatter of the logits (lane (j, qg) keeps heads 2qg, 2qg + 1)
#pragma unroll
  for (int x = 1; x <= 32; x <<= 1) {
    if (x == 8 || x == 16) continue;
    l0 += __shfl_xor(l0, x, kWave);
    l1 += __shfl_xor(l1, x, kWave);
  }
  const int hi = qg >> 1, lo = qg & 1;
  float o4[4][8], o2[2][8];
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float keep = hi ? acc[4 + e][c] : acc[e][c];
      const float give = hi ? acc[e][c] : acc[4 + e][c];
      o4[e][c] = keep + __shfl_xor(give, 32, kWave);
    }
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float keep = lo ? o4[2 + e][c] : o4[e][c];
      const float give = lo ? o4[e][c] : o4[2 + e][c];
      o2[e][c] = keep + __shfl_xor(give, 16, kWave);
    }

  // merge the waves through LDS, as the partition kernel does
  float* so = smem;                  // [kNW][G][D]
  float* sm = smem + kNW * G * kD;   // [kNW][16]
  float* sl = sm + kNW * 16;         // [kNW][16]
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    if (2 * qg + e < G) {
#pragma unroll
      for (int c = 0; c < 8; ++c) so[(w * G + 2 * qg + e) * kD + 16 * c + j] = o2[e][c];
    }
    // lane 16 b0 + 8 hg (tp = b1 = 0) holds heads 2 hsel, 2 hsel + 1
    if (tp == 0 && b1 == 0 && 2 * hsel + e < G) {
      sm[w * 16 + 2 * hsel + e] = e ? m1 : m0;
      sl[w * 16 + 2 * hsel + e] = e ? l1 : l0;
    }
  }
  __syncthreads();
  const bool single = n_p == 1;
  for (int i = threadIdx.x; i < G * kD; i += kNW * kWave) {
    const int gg = i / kD, d = i - gg * kD;
    float mx = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kNW; ++ww) mx = fmaxf(mx, sm[ww * 16 + gg]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kNW; ++ww) {
      const float f = __builtin_amdgcn_exp2f(sm[ww * 16 + gg] - mx);
      num += so[(ww * G + gg) * kD + d] * f;
      den += sl[ww * 16 + gg] * f;
    }
    if (single) {
      a.out[(head0 + gg) * kD + d] = num / den * a.out_scale;
    } else {
      const int64_t prow2 = part_row(a, b, kvh, p, gg);
      a.ws_o[prow2 * kD + d] = num;
      if (d == 0) {
        a.ws_ml[prow2 * 2] = mx;
        a.ws_ml[prow2 * 2 + 1] = den;
      }
    }
  }
}

// Short partitions (an explicit split-KV length of a few hundred tokens):
// launching one workgroup per partition leaves each wave a stream of a few
// tiles, and the stream drains at every partition end.  Here each wave owns
// `chain` consecutive partitions of one (sequence, KV head) instead -- a
// contiguous run of logical blocks -- and streams them back to back.  At the
// end of each partition it puts that partition's (max, sum, unnormalised
// output) into its own LDS staging area, and when the run ends it stores the
// run's partials together: they are adjacent rows of the workspace, so the
// wave writes one contiguous span.  Storing each partial when its partition
// ends cost the 128K-context batch at 512-token partitions 184 against 170
// us: a wave's vector memory operations complete in order for its wait
// counts, so the wait for the next tile, whose loads were issued after the
// stores, waited for the stores too.  The partials, and the merge kernel
// that combines them, are the same as with one workgroup per partition.
// Per-tensor scales only: with per-block scales the extra registers spill
// and one workgroup per partition is faster.  Grid (ceil(n_p_max /
// (kChainWaves * chain)), Hkv, B); kChainWaves waves per workgroup, each
// independent of the others; chain_lds_bytes of dynamic LDS.  kAppend: the
// kernel also writes each sequence's newest token (steps 1-3 above).
constexpr int kChainWaves = 2;
constexpr size_t kChainLdsMax = 65536;

// LDS staging of the chained kernel: [kChainWaves][chain][G][kD] outputs,
// then [kChainWaves][chain][G] (max, sum) pairs.
static inline size_t chain_lds_bytes(int chain, int g) {
  return (size_t)kChainWaves * chain * g * (kD + 2) * sizeof(float);
}

template <bool kFP8, bool kAppend = false>
__global__ void __launch_bounds__(kChainWaves * kWave) decode_chain_kernel(DecodeArgs a,
                                                                           int chain) {
  constexpr int kPD = 1;
  __shared__ __align__(16) uint8_t keep[kAppend ? kKeepBytes : 16];
  extern __shared__ __align__(16) float stage[];  // chain_lds_bytes(chain, G)
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int j = lane & 15;
  const int qg = lane >> 4;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int G = a.g;
  float2* ml_stage = reinterpret_cast<float2*>(stage + kChainWaves * chain * G * kD);

  const int L = clamp_len(a, b);
  const SeqSplit sp = seq_split(a, L);
  const int64_t head0 = (int64_t)b * a.hq + (int64_t)kvh * G;
  const int p_first = (blockIdx.x * kChainWaves + w) * chain;
  if (p_first >= sp.n_p) {
    if (p_first == 0) {  // empty sequence: attention over nothing is defined as zeros
      for (int i = lane; i < G * kD; i += kWave) a.out[head0 * kD + i] = 0.0f;
    }
    return;
  }
  const int blk_begin = p_first * sp.per;
  const int my_n = min(sp.nblk, (p_first + chain) * sp.per) - blk_begin;

  // the wave whose run ends with the sequence's last block writes the
  // newest token and patches it into its last tile (one such wave per
  // sequence and KV head, so the workgroup's kept bytes are its own)
  int patch_at = -1;
  if constexpr (kAppend) {
    if (blk_begin + my_n == sp.nblk) patch_at = my_n - 1;
    patch_at = __builtin_amdgcn_readfirstlane(patch_at);
  }

  f16x8 qop[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (j < G) {
      const int d0 = kFP8 ? (m >> 1) * 64 + qg * 16 + (m & 1) * 8 : m * 32 + qg * 8;
      qop[m] = *reinterpret_cast<const f16x8*>(a.q + (head0 + j) * kD + d0);
    } else {
      qop[m] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  SoftmaxState st;
  st.m_ref = -INFINITY;
  st.l = 0.0f;
#pragma unroll
  for (int n = 0; n < 8; ++n) st.acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bool single = sp.n_p == 1;
  int part = p_first;                                   // partition being accumulated
  int part_end = min(sp.nblk, (part + 1) * sp.per);     // its first block past the end
  const int32_t* trow = a.block_tables + (int64_t)b * a.max_blocks + blk_begin;
  const int shared_blocks = a.shared_prefix != nullptr ? a.shared_prefix[b] : 0;
  // chunks end where the shared tiles end, as in partition_unit
  const int n_sh = min(my_n, max(0, shared_blocks - blk_begin));
  int cnt = 0;
  for (int c0 = 0; c0 < my_n; c0 += cnt) {
    cnt = min(kWave, (c0 < n_sh ? n_sh : my_n) - c0);
    u32x2 rows = u32x2{0u, 0u};  // the newest token's rows, ahead of the table load
    if constexpr (kAppend)
      if (c0 == 0 && patch_at >= 0) rows = append_load(a, b, kvh, lane);
    const int tbl = load_table(trow + c0, cnt, 1, lane);
    const int lb0 = blk_begin + c0;
    // unconditional loads and one cache policy per chunk, as in partition_unit
    auto chunk = [&](auto policy) {
      constexpr int kAux = decltype(policy)::value;
      TileRegs<kFP8> buf[kPD + 1];
#pragma unroll
      for (int r = 0; r < kPD; ++r)
        load_tile<kFP8, kAux>(buf[r], a.k_pool, a.v_pool, a.num_blocks, a.hkv,
                              r < cnt ? __builtin_amdgcn_readlane(tbl, r) : -1, kvh, lane);
      if constexpr (kAppend)
        if (c0 == 0 && patch_at >= 0) append_keep<kFP8>(a, rows, lane, keep);
      for (int base = 0; base < cnt; base += kPD + 1) {
#pragma unroll
        for (int r = 0; r <= kPD; ++r) {
          const int ii = base + r;
          const int nx = ii + kPD;
          load_tile<kFP8, kAux>(buf[(r + kPD) % (kPD + 1)], a.k_pool, a.v_pool, a.num_blocks,
                                a.hkv, nx < cnt ? __builtin_amdgcn_readlane(tbl, nx) : -1, kvh,
                                lane);
          if (ii < cnt) {
            if constexpr (kAppend)
              if (c0 + ii == patch_at) {
                const int phys = __builtin_amdgcn_readlane(tbl, ii);
                if ((unsigned)phys < (unsigned)a.num_blocks) {  // else nothing is written
                  patch_tile<kFP8>(buf[r], keep, lane, (L - 1) & 15);
                  append_store<kFP8>(a, buf[r], phys, kvh, lane, (L - 1) & 15);
                }
              }
            process_tile<kFP8, true, true>(buf[r], qop, st, (lb0 + ii) * kBS, qg, L, a.qk_scale);
            if (lb0 + ii + 1 == part_end) {  // wave-uniform: partition `part` is complete
              float l_run = st.l;
              l_run += __shfl_xor(l_run, 16, kWave);
              l_run += __shfl_xor(l_run, 32, kWave);
              const int64_t hrow = head0 + j;
              if (j < G) {
                if (single) {
                  float* dst = a.out + hrow * kD + qg * 4;
#pragma unroll
                  for (int n = 0; n < 8; ++n) {
                    f32x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = st.acc[n][e] / l_run * a.out_scale;
                    *reinterpret_cast<f32x4*>(dst + n * 16) = o;
                  }
                } else {
                  const int k = (w * chain + part - p_first) * G + j;  // staged row
#pragma unroll
                  for (int n = 0; n < 8; ++n)
                    *reinterpret_cast<f32x4*>(stage + k * kD + n * 16 + qg * 4) = st.acc[n];
                  if (qg == 0) ml_stage[k] = make_float2(st.m_ref, l_run);
                }
              }
              st.m_ref = -INFINITY;
              st.l = 0.0f;
#pragma unroll
              for (int n = 0; n < 8; ++n) st.acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
              ++part;
              part_end = min(sp.nblk, part_end + sp.per);
            }
          }
        }
      }
    };
    if (lb0 + cnt - 1 < shared_blocks)
      chunk(std::integral_constant<int, 0>{});
    else
      chunk(std::integral_constant<int, kLoadNT>{});
  }
  if (!single) {
    // the run's partials: rows part_row(b, kvh, p_first, 0) onward, adjacent
    // in the workspace; lanes read rows other lanes staged (one wave)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int rows = __builtin_amdgcn_readfirstlane((part - p_first) * G);
    const int64_t row0 = part_row(a, b, kvh, p_first, 0);
    const __amdgpu_buffer_rsrc_t run = partial_rows(a.ws_o + row0 * kD, rows * kD * 4);
    const float* src = stage + w * chain * G * kD;
    for (int i = lane * 4; i < rows * kD; i += kWave * 4)
      __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(src + i), run, i * 4,
                                             0, kWriteThrough);
    for (int i = lane; i < rows; i += kWave)
      reinterpret_cast<float2*>(a.ws_ml)[row0 + i] = ml_stage[w * chain * G + i];
  }
}

// Merge kernel: for each (sequence, query head) whose sequence spans n_p > 1
// partitions, M = max_p m_p and
//   out = out_scale * sum_p o_p 2^(m_p - M) / sum_p l_p 2^(m_p - M).
// Half a wave (32 lanes x 16 bytes) reads one partition's 128-float output
// row, so one wave instruction covers two partitions.  Every load is issued
// at once -- the rows of all n_p_max partitions the workspace holds, with the
// sequence's length -- and rows past the sequence's own n_p are dropped by
// selection afterwards (never multiplied: a stale row may hold anything), so
// a merge costs one round trip to memory.
//   kMany = false: one wave per (b, h); its two halves take the even and the
//     odd partitions, n_p_max <= kFewPartitions.
//   kMany = true: four waves per (b, h); half-wave hw (0..7) takes
//     partitions hw, hw + 8, ... (up to kManyPartitions), the maximum and the
//     partition weights go through LDS, and the eight half-sums combine
//     through LDS.
// The summation order is fixed, so results do not depend on timing.
constexpr int kFewPartitions = 16;
constexpr int kManyPartitions = 8 * 32;  // 32 rows per lane of the kMany kernel

template <bool kMany>
__global__ void __launch_bounds__(kRW * kWave) decode_reduce_kernel(DecodeArgs a, int64_t rows) {
  __shared__ float wgt_s[kMany ? kManyPartitions : 1];  // partition weights (kMany)
  __shared__ f32x4 half_s[kMany ? 2 * kRW : 1][32];      // half-wave sums (kMany)
  __shared__ float red_s[kMany ? kRW : 1];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int half = lane >> 5, c4 = lane & 31;        // channels 4 c4 .. 4 c4 + 3
  const int64_t bh = kMany ? (int64_t)blockIdx.x : (int64_t)blockIdx.x * kRW + w;
  if (bh >= rows) return;                    // only when !kMany: whole waves leave
  const int b = (int)(bh / a.hq);
  const int h = (int)(bh - (int64_t)b * a.hq);
  const int64_t row0 = part_row(a, b, h / a.g, 0, h % a.g);
  const int64_t pst = a.g;                   // rows from one partition to the next
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml);
  const f32x4* orow = reinterpret_cast<const f32x4*>(a.ws_o + row0 * kD) + c4;
  const int64_t ost = pst * (kD / 4);        // f32x4 steps from one partition to the next
  const int npm = a.n_p_max;               // >= 2: the merge runs only then

  if constexpr (!kMany) {
    // the first two partitions' rows (every merged row has them) with the
    // ml pairs and the length; the others once the length says they exist
    const float2 mine = lane < npm ? ml[row0 + lane * pst] : make_float2(-INFINITY, 0.0f);
    f32x4 o[kFewPartitions / 2];
    o[0] = orow[half * ost];
    const int n_p = seq_parts(a, b, clamp_len(a, b));
    if (n_p <= 1) return;                    // written by the partition kernel
#pragma unroll
    for (int k = 1; k < kFewPartitions / 2; ++k) {
      const int pp = 2 * k + half;
      o[k] = pp < n_p ? orow[pp * ost] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const bool valid = lane < n_p;
    const float mx = wave_max(valid ? mine.x : -INFINITY);
    const float wgt = valid ? __builtin_amdgcn_exp2f(mine.x - mx) : 0.0f;
    const float den = wave_sum(valid ? mine.y * wgt : 0.0f);
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kFewPartitions / 2; ++k) {
      const int pp = 2 * k + half;
      // weight of partition 2k (lower half) or 2k + 1 (upper half)
      const float g0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), 2 * k));
      const float g1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), 2 * k + 1));
      if (pp < n_p) acc += o[k] * (half ? g1 : g0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], 32, kWave);
    if (half == 0)
      reinterpret_cast<f32x4*>(a.out + bh * kD)[c4] = acc * (a.out_scale / den);
    return;
  } else {
    const int tid = threadIdx.x;
    const int hw = w * 2 + half;             // half-wave 0..7
    constexpr int kPer = kManyPartitions / 8;
    // every row at once: thread tid's ml pair, this half-wave's output rows
    const float2 mine = tid < npm ? ml[row0 + tid * pst] : make_float2(-INFINITY, 0.0f);
    f32x4 o[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int pp = hw + 8 * u;
      o[u] = pp < npm ? orow[(int64_t)pp * ost] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int n_p = seq_parts(a, b, clamp_len(a, b));
    if (n_p <= 1) return;                    // written by the partition kernel (uniform)
    const bool valid = tid < n_p;
    float mx = wave_max(valid ? mine.x : -INFINITY);
    if (lane == 0) red_s[w] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red_s[0], red_s[1]), fmaxf(red_s[2], red_s[3]));
    const float g = valid ? __builtin_amdgcn_exp2f(mine.x - mx) : 0.0f;
    wgt_s[tid] = g;
    const float den_part = wave_sum(valid ? mine.y * g : 0.0f);
    __syncthreads();                         // weights in LDS; red_s read by all
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int pp = hw + 8 * u;
      if (pp < n_p) acc += o[u] * wgt_s[pp];
    }
    half_s[hw][c4] = acc;
    if (lane == 0) red_s[w] = den_part;
    __syncthreads();
    if (w == 0 && half == 0) {
      f32x4 t = half_s[0][c4];
#pragma unroll
      for (int k = 1; k < 2 * kRW; ++k) t += half_s[k][c4];
      const float dd = (red_s[0] + red_s[1]) + (red_s[2] + red_s[3]);
      reinterpret_cast<f32x4*>(a.out + bh * kD)[c4] = t * (a.out_scale / dd);
    }
  }
}

// Merge of up to kFewPartitions partitions, one wave per (sequence, KV
// head): the G query heads of a group share the sequence's partition count,
// and their partial rows are adjacent in the workspace (partition p's G
// rows, then partition p + 1's).  Lane l serves head g = l / kLH of the
// group and, in each of its rows, the 16-byte pieces sub, sub + kLH, ...
// (kLH lanes a head: 64 / G rounded up to a power of two, at most 32).  The
// sequence's length, the (max, sum) pairs of every partition the workspace
// holds and the first kChunk partitions' rows are requested at once, so a
// sequence of at most kChunk partitions costs one round trip to memory;
// rows past the sequence's own partition count are dropped by selection
// (never multiplied: a stale row may hold anything).  Partitions are summed
// in order, so results do not depend on timing.  One wave per row (the
// decode_reduce_kernel<false> layout) leaves 16,384 short waves for a
// 256-sequence batch, 13 us under the profiler, most of it waves waiting for
// a slot.
// The group merge is used from this many (sequence, KV head) groups on: at
// 128 groups (one GPU's share of a 4-way tensor-parallel 70B step) its 128
// waves took longer than the per-row kernel's 1,024 (step 49.4-49.6 against
// 48.7-49.2 us); at 2,048 (the 256-sequence batch) it saved 1.5 us.
constexpr int64_t kGroupMergeMin = 1024;

template <int kV>  // 16-byte pieces a lane takes of each row: 32 / kLH
__global__ void __launch_bounds__(kRW * kWave) decode_reduce_group_kernel(DecodeArgs a,
                                                                          int64_t groups) {
  constexpr int kLH = 32 / kV;
  constexpr int kChunk = kFewPartitions / kV;  // partitions whose rows are in flight at once
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t bk = (int64_t)blockIdx.x * kRW + w;  // (sequence, KV head)
  if (bk >= groups) return;                          // whole waves leave
  const int b = (int)(bk / a.hkv);
  const int kvh = (int)(bk - (int64_t)b * a.hkv);
  const int G = a.g;
  const int g = lane / kLH, sub = lane - g * kLH;
  const bool head = g < G;
  const int npm = a.n_p_max;  // >= 2: the merge runs only then
  const int64_t row0 = part_row(a, b, kvh, 0, 0) + g;
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml) + row0;
  const f32x4* orow = reinterpret_cast<const f32x4*>(a.ws_o + row0 * kD) + sub;
  const int64_t pst = (int64_t)G * (kD / 4);  // f32x4 steps from one partition to the next

  float2 mlp[kFewPartitions];
#pragma unroll
  for (int p = 0; p < kFewPartitions; ++p)
    mlp[p] = head && p < npm ? ml[p * G] : make_float2(-INFINITY, 0.0f);
  f32x4 o[kChunk][kV];
#pragma unroll
  for (int p = 0; p < kChunk; ++p)
#pragma unroll
    for (int v = 0; v < kV; ++v)
      o[p][v] = head && p < npm ? orow[p * pst + v * kLH] : f32x4{0.f, 0.f, 0.f, 0.f};
  const int n_p = seq_parts(a, b, clamp_len(a, b));
  if (n_p <= 1) return;  // written by the partition kernel (uniform)

  float mx = -INFINITY;
#pragma unroll
  for (int p = 0; p < kFewPartitions; ++p)
    if (p < n_p) mx = fmaxf(mx, mlp[p].x);
  float wgt[kFewPartitions];
  float den = 0.0f;
#pragma unroll
  for (int p = 0; p < kFewPartitions; ++p) {
    wgt[p] = p < n_p ? __builtin_amdgcn_exp2f(mlp[p].x - mx) : 0.0f;
    if (p < n_p) den += mlp[p].y * wgt[p];
  }
  f32x4 acc[kV];
#pragma unroll
  for (int v = 0; v < kV; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < kFewPartitions; c += kChunk) {
    if (c >= n_p) break;  // uniform
    if (c > 0) {          // a further chunk: one more round trip
#pragma unroll
      for (int p = 0; p < kChunk; ++p)
#pragma unroll
        for (int v = 0; v < kV; ++v)
          o[p][v] = head && c + p < n_p ? orow[(c + p) * pst + v * kLH]
                                        : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int p = 0; p < kChunk; ++p)
      if (c + p < n_p)
#pragma unroll
        for (int v = 0; v < kV; ++v) acc[v] += o[p][v] * wgt[c + p];
  }
  if (head) {
    f32x4* dst = reinterpret_cast<f32x4*>(a.out + ((int64_t)b * a.hq + kvh * G + g) * kD) + sub;
#pragma unroll
    for (int v = 0; v < kV; ++v) dst[v * kLH] = acc[v] * (a.out_scale / den);
  }
}

// Merge of sequences with more partitions than one launch of the kMany
// kernel takes (n_p_max > kManyPartitions): one workgroup of four waves per
// (b, h), chunks of kManyPartitions partitions, the same arithmetic in the
// same fixed order.
__global__ void __launch_bounds__(kRW * kWave) decode_reduce_long_kernel(DecodeArgs a,
                                                                          int64_t rows) {
  __shared__ float wgt_s[kManyPartitions];
  __shared__ f32x4 half_s[2 * kRW][32];
  __shared__ float red_s[kRW];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, tid = threadIdx.x;
  const int half = lane >> 5, c4 = lane & 31, hw = w * 2 + half;
  const int64_t bh = blockIdx.x;
  if (bh >= rows) return;
  const int b = (int)(bh / a.hq);
  const int n_p = seq_parts(a, b, clamp_len(a, b));
  if (n_p <= 1) return;
  const int h = (int)(bh - (int64_t)b * a.hq);
  const int64_t row0 = part_row(a, b, h / a.g, 0, h % a.g);
  const int64_t pst = a.g;
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml);
  const f32x4* orow = reinterpret_cast<const f32x4*>(a.ws_o + row0 * kD) + c4;
  const int64_t ost = pst * (kD / 4);
  float mx = -INFINITY;
  for (int pp = tid; pp < n_p; pp += kRW * kWave) mx = fmaxf(mx, ml[row0 + pp * pst].x);
  mx = wave_max(mx);
  if (lane == 0) red_s[w] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red_s[0], red_s[1]), fmaxf(red_s[2], red_s[3]));
  __syncthreads();
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float den = 0.0f;
  for (int c = 0; c < n_p; c += kManyPartitions) {
    const int cn = min(kManyPartitions, n_p - c);
    for (int pp = tid; pp < cn; pp += kRW * kWave) {
      const float2 v = ml[row0 + (int64_t)(c + pp) * pst];
      const float g = __builtin_amdgcn_exp2f(v.x - mx);
      wgt_s[pp] = g;
      den += v.y * g;
    }
    __syncthreads();
    for (int pp = hw; pp < cn; pp += 8) acc += orow[(int64_t)(c + pp) * ost] * wgt_s[pp];
    __syncthreads();
  }
  den = wave_sum(den);
  half_s[hw][c4] = acc;
  if (lane == 0) red_s[w] = den;
  __syncthreads();
  if (w == 0 && half == 0) {
    f32x4 t = half_s[0][c4];
#pragma unroll
    for (int k = 1; k < 2 * kRW; ++k) t += half_s[k][c4];
    const float dd = (red_s[0] + red_s[1]) + (red_s[2] + red_s[3]);
    reinterpret_cast<f32x4*>(a.out + bh * kD)[c4] = t * (a.out_scale / dd);
  }
}

// ------------------------------------------------------------- host side

// Automatic partition length (measured on MI355X at the five reference
// shapes): fewer, longer partitions are faster as long as enough tiles are in
// flight to cover HBM latency -- about 2048 waves of FP8 tiles (4 KiB per
// block and head) or 1024 waves of fp16 tiles (8 KiB).  So: the fewest
// partitions per sequence that give that many waves (4 per workgroup), cut
// into equal runs of whole blocks, at least 8 blocks each.  Batches with 1024
// or more (sequence, KV head) pairs -- where lengths may be ragged and
// prefixes shared -- cap a partition at 256 blocks (4096 tokens) so that long
// sequences leave no tail; otherwise the cap is 1024 blocks.
int32_t resolve_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_ctx,
                          int32_t dtype, int32_t requested) {
  if (requested < 0 || requested % kBS != 0) return -1;
  if (requested > 0) return requested;
  const int64_t nblk = max_ctx > 0 ? ((int64_t)max_ctx + kBS - 1) / kBS : 1;
  const int64_t pairs = std::max<int64_t>(1, (int64_t)num_seqs * std::max(1, num_kv_heads));
  const int64_t target_waves = dtype == PKV_F16 ? 1024 : 2048;
  int64_t n_p = (target_waves + 4 * pairs - 1) / (4 * pairs);
  n_p = std::max<int64_t>(1, std::min<int64_t>(n_p, nblk / 8));
  int64_t per = (nblk + n_p - 1) / n_p;
  per = std::min<int64_t>(per, pairs >= 1024 ? 256 : 1024);
  return (int32_t)(per * kBS);
}

struct WsLayout {
  uint64_t ml_bytes, o_bytes, total;
  int32_t n_p_max;
};

WsLayout ws_layout(int32_t num_seqs, int32_t num_q_heads, int32_t max_ctx, int32_t part) {
  WsLayout w{0, 0, 0, 0};
  // partitions of the longest sequence: ceil(blocks / (part / 16))
  const int64_t nblk = ((int64_t)std::max(max_ctx, 0) + kBS - 1) / kBS;
  const int64_t pb = part / kBS;
  w.n_p_max = nblk == 0 ? 1 : (int32_t)((nblk + pb - 1) / pb);
  if (w.n_p_max <= 1) return w;
  const uint64_t rows = (uint64_t)num_seqs * (uint64_t)num_q_heads * (uint64_t)w.n_p_max;
  w.ml_bytes = (rows * 2 * sizeof(float) + 255) / 256 * 256;
  w.o_bytes = rows * kD * sizeof(float);
  w.total = w.ml_bytes + w.o_bytes;
  return w;
}

// Cascade workspace: every sequence may have a prefix of up to max_prefix
// blocks (each split into ceil(S / (part / 16)) partitions) before its tail
// partitions.  Also gives the grid's partition dimension (x_dim).
struct CascLayout {
  WsLayout ws;
  int32_t s_max, x_dim;
  int32_t n_pp, n_pt;  // most prefix partitions, most tail partitions
};

CascLayout casc_layout(int32_t num_seqs, int32_t num_q_heads, int32_t max_ctx, int32_t part,
                       int32_t max_prefix) {
  CascLayout c{};
  const int64_t nblk = ((int64_t)std::max(max_ctx, 0) + kBS - 1) / kBS;
  const int64_t pb = part / kBS;
  // a prefix leaves at least one token to the tail
  c.s_max = (int32_t)std::max<int64_t>(
      0, std::min<int64_t>(max_prefix, ((int64_t)std::max(max_ctx, 1) - 1) / kBS));
  const int64_t n_pp = (c.s_max + pb - 1) / pb;
  const int64_t n_pt = nblk == 0 ? 1 : (nblk + pb - 1) / pb;
  c.x_dim = (int32_t)std::max(n_pp, n_pt);
  c.n_pp = (int32_t)n_pp;
  c.n_pt = (int32_t)n_pt;
  c.ws.n_p_max = (int32_t)(n_pp + n_pt);
  if (c.ws.n_p_max <= 1) return c;
  const uint64_t rows = (uint64_t)num_seqs * (uint64_t)num_q_heads * (uint64_t)c.ws.n_p_max;
  c.ws.ml_bytes = (rows * 2 * sizeof(float) + 255) / 256 * 256;
  c.ws.o_bytes = rows * kD * sizeof(float);
  c.ws.total = c.ws.ml_bytes + c.ws.o_bytes;
  return c;
}

// Kernel variants, chosen once per process.  Environment overrides exist for
// measurement (A/B runs of the same build); the defaults are the measured
// best.
//   PKV_FP8_DEQUANT = hw | bits   FP8 -> fp16 by the gfx950 conversion or by
//                                 integer bit operations
//   PKV_FP8_SPLIT_P = 0 | 1       probabilities as one fp16 or fp16 hi + lo
//                                 (fp16 caches always use hi + lo)
//   PKV_DECODE_PREFETCH = 1 | 2   tiles in flight per wave besides the one
//                                 being computed
//   PKV_DECODE_WAVES = 1|2|4|8    waves per partition workgroup (default:
//                                 from the partition length)
//   PKV_DECODE_CHAIN = 0 | n      partitions per wave for short partitions:
//                                 0 = one workgroup per partition, n = fixed
//                                 (default: from the shape)
//   PKV_DECODE_MATH = mfma | valu the contractions on the matrix cores or on
//                                 the vector ALUs (decode_valu_kernel: FP8,
//                                 per-tensor scales, G <= 8; other shapes and
//                                 the cascade keep the matrix cores)
struct KernelConfig {
  bool hw_cvt;
  bool split_p_fp8;
  int prefetch;
  int waves;
  int chain;  // -1 = automatic
  bool valu;
};

KernelConfig kernel_config() {
  static const KernelConfig cfg = [] {
    KernelConfig k{true, true, 1, 0, -1, false};
    if (const char* e = std::getenv("PKV_FP8_DEQUANT")) k.hw_cvt = std::strcmp(e, "hw") == 0;
    if (const char* e = std::getenv("PKV_FP8_SPLIT_P")) k.split_p_fp8 = std::atoi(e) != 0;
    if (const char* e = std::getenv("PKV_DECODE_PREFETCH")) {
      const int v = std::atoi(e);
      if (v >= 1 && v <= 2) k.prefetch = v;
    }
    if (const char* e = std::getenv("PKV_DECODE_CHAIN")) {
      const int v = std::atoi(e);
      if (v >= 0 && v <= 1024) k.chain = v;
    }
    if (const char* e = std::getenv("PKV_DECODE_WAVES")) {
      const int v = std::atoi(e);
      if (v == 1 || v == 2 || v == 4 || v == 8) k.waves = v;
    }
    if (const char* e = std::getenv("PKV_DECODE_MATH")) {
      k.valu = std::strcmp(e, "valu") == 0;
      if (k.valu) k.hw_cvt = true;  // the vector kernel converts to code values
    }
    return k;
  }();
  return cfg;
}

struct DecodePlan {
  DecodeArgs a;
  bool fp8;
  bool dyn;  // per-block scales
  bool need_reduce;
  KernelConfig cfg;
};

pkv_status plan_decode(float* out, const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, const int32_t* shared_prefix_blocks,
                       int32_t num_seqs, int32_t num_q_heads,
                       int32_t max_context_len, const pkv_cache_layout* layout, float sm_scale,
                       float k_scale, float v_scale, const float* k_bscale,
                       const float* v_bscale, int32_t partition_size, void* workspace,
                       uint64_t workspace_bytes, bool need_pools, DecodePlan* plan,
                       hipStream_t stream) {
  pkv_status st = check_layout(layout);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || num_seqs > 65535 || max_context_len < 0 || num_q_heads <= 0)
    return PKV_ERR_INVALID_ARG;
  if (num_q_heads % layout->num_kv_heads != 0) return PKV_ERR_INVALID_ARG;
  const int32_t G = num_q_heads / layout->num_kv_heads;
  if (G > kMaxG) return PKV_ERR_UNSUPPORTED;
  plan->cfg = kernel_config();
  plan->fp8 = layout->dtype == PKV_FP8_E4M3FN;
  plan->dyn = k_bscale != nullptr || v_bscale != nullptr;
  plan->need_reduce = false;
  if (plan->dyn && !plan->fp8) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;  // nothing to compute; no pointer is touched
  if (!out || !context_lens || !aligned(out, 16)) return PKV_ERR_INVALID_ARG;
  if (need_pools) {
    if (!q || !k_pool || !v_pool || !block_tables) return PKV_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
      return PKV_ERR_INVALID_ARG;
    if (max_blocks_per_seq <= 0) return PKV_ERR_INVALID_ARG;
    if (!std::isfinite(sm_scale)) return PKV_ERR_INVALID_ARG;
    if (plan->dyn && (!k_bscale || !v_bscale || !aligned(k_bscale, 4) || !aligned(v_bscale, 4)))
      return PKV_ERR_INVALID_ARG;
    st = debug_check_tables(block_tables, max_blocks_per_seq, context_lens, num_seqs,
                            max_context_len, layout->num_blocks, stream);
    if (st != PKV_OK) return st;
  } else if (max_blocks_per_seq <= 0) {
    return PKV_ERR_INVALID_ARG;
  }
  const bool fp8 = layout->dtype == PKV_FP8_E4M3FN;
  if (fp8 && !(std::isfinite(k_scale) && k_scale > 0.0f && std::isfinite(v_scale) &&
               v_scale > 0.0f))
    return PKV_ERR_INVALID_ARG;
  const int32_t part = resolve_partition(num_seqs, layout->num_kv_heads, max_context_len,
                                         layout->dtype, partition_size);
  if (part <= 0) return PKV_ERR_INVALID_ARG;
  const WsLayout wl = ws_layout(num_seqs, num_q_heads, max_context_len, part);
  if (wl.total > 0) {
    if (!workspace || workspace_bytes < wl.total) return PKV_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return PKV_ERR_INVALID_ARG;
  }
  DecodeArgs& a = plan->a;
  a.out = out;
  a.q = static_cast<const _Float16*>(q);
  a.k_pool = static_cast<const uint8_t*>(k_pool);
  a.v_pool = static_cast<const uint8_t*>(v_pool);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.shared_prefix = shared_prefix_blocks;
  a.ws_ml = wl.total ? static_cast<float*>(workspace) : nullptr;
  a.ws_o = wl.total ? reinterpret_cast<float*>(static_cast<char*>(workspace) + wl.ml_bytes)
                    : nullptr;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = layout->num_blocks;
  a.hq = num_q_heads;
  a.hkv = layout->num_kv_heads;
  a.g = G;
  a.max_ctx = max_context_len;
  a.part_blocks = part / kBS;
  a.n_p_max = wl.n_p_max;
  a.k_bscale = plan->dyn ? k_bscale : nullptr;
  a.v_bscale = plan->dyn ? v_bscale : nullptr;
  a.new_k = a.new_v = nullptr;
  a.k_wr = a.v_wr = nullptr;
  a.casc_prefix = nullptr;
  a.casc_groups = nullptr;
  a.casc_items = a.casc_chunks = a.casc_cap = a.casc_m = a.casc_mi = a.casc_max = 0;
  a.seq_order = nullptr;
  a.nseq = num_seqs;
  a.casc_flat = 0;
  a.casc_pp = 1;
  a.casc_tail_map = nullptr;
  a.casc_tail_count = 0;
  a.k_enc_scale = k_scale;
  a.v_enc_scale = v_scale;
  // FP8 tiles decoded by bit operations hold code / 256: fold the 256 back
  // in (per-block scales always use the hardware conversion)
  const float deq = (fp8 && !plan->cfg.hw_cvt && !plan->dyn) ? 256.0f : 1.0f;
  const float log2e = 1.4426950408889634f;
  a.qk_scale = sm_scale * (fp8 ? k_scale * deq : 1.0f) * log2e;
  a.out_scale = fp8 ? v_scale * deq : 1.0f;
  plan->fp8 = fp8;
  plan->need_reduce = wl.n_p_max > 1;
  return PKV_OK;
}

}  // namespace

// ------------------------------------------------------------------ C ABI

extern "C" int32_t pkv_decode_partition_size(int32_t num_seqs, int32_t num_kv_heads,
                                             int32_t max_context_len, int32_t dtype,
                                             int32_t requested) {
  if (dtype != PKV_F16 && dtype != PKV_FP8_E4M3FN) return -1;
  return resolve_partition(num_seqs, num_kv_heads, max_context_len, dtype, requested);
}

extern "C" uint64_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                               int32_t num_kv_heads, int32_t max_context_len,
                                               int32_t dtype, int32_t partition_size) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0) return 0;
  if (dtype != PKV_F16 && dtype != PKV_FP8_E4M3FN) return 0;
  const int32_t part =
      resolve_partition(num_seqs, num_kv_heads, max_context_len, dtype, partition_size);
  if (part <= 0) return 0;
  return ws_layout(num_seqs, num_q_heads, max_context_len, part).total;
}


// LDS of a partition workgroup: the wave merge for `cols` columns per wave,
// the kept bytes of the newest token, the prefix item's member per column.
static size_t partition_lds(int nw, int cols, bool append, bool casc) {
  return (size_t)(nw * cols * kD + 2 * nw * 16) * sizeof(float) +
         (append || casc ? kKeepBytes : 0) + (casc ? kMaxG * sizeof(int) : 0);
}

template <bool kFP8, bool kHw, bool kSplit, int kPD, int kNW, bool kDyn = false,
          bool kAppend = false, bool kCasc = false>
static void launch_partition_v(dim3 grid, hipStream_t s, const DecodeArgs& a) {
  const size_t lds = partition_lds(kNW, kCasc ? kMaxG : a.g, kAppend, kCasc);
  decode_partition_kernel<kFP8, kHw, kSplit, kPD, kNW, kDyn, kAppend, kCasc>
      <<<grid, dim3(kNW * kWave), lds, s>>>(a);
}

// Cascade over shared prefixes: the default family (FP8: hardware convert,
// split probabilities; one tile in flight), with or without the newest
// token's write.
template <bool kFP8, bool kAppend>
static void launch_partition_casc(int nw, dim3 grid, hipStream_t s, const DecodeArgs& a) {
  switch (nw) {
    case 1: return launch_partition_v<kFP8, kFP8, true, 1, 1, false, kAppend, true>(grid, s, a);
    case 2: return launch_partition_v<kFP8, kFP8, true, 1, 2, false, kAppend, true>(grid, s, a);
    default: return launch_partition_v<kFP8, kFP8, true, 1, 4, false, kAppend, true>(grid, s, a);
  }
}

// Cascade over per-block scales (FP8, decode only).
static void launch_partition_casc_dyn(int nw, dim3 grid, hipStream_t s, const DecodeArgs& a) {
  switch (nw) {
    case 1: return launch_partition_v<true, true, true, 1, 1, true, false, true>(grid, s, a);
    case 2: return launch_partition_v<true, true, true, 1, 2, true, false, true>(grid, s, a);
    default: return launch_partition_v<true, true, true, 1, 4, true, false, true>(grid, s, a);
  }
}

// Writing the newest token too: the default family (FP8: hardware convert,
// split probabilities; one tile in flight) at every wave count.
template <bool kFP8>
static void launch_partition_append(int nw, dim3 grid, hipStream_t s, const DecodeArgs& a) {
  switch (nw) {
    case 1: return launch_partition_v<kFP8, kFP8, true, 1, 1, false, true>(grid, s, a);
    case 2: return launch_partition_v<kFP8, kFP8, true, 1, 2, false, true>(grid, s, a);
    case 8: return launch_partition_v<kFP8, kFP8, true, 1, 8, false, true>(grid, s, a);
    default: return launch_partition_v<kFP8, kFP8, true, 1, 4, false, true>(grid, s, a);
  }
}

// Per-block scales: the default family (hardware convert, split P, one tile
// in flight besides the current one) at every wave count.
static void launch_partition_dyn(int nw, dim3 grid, hipStream_t s, const DecodeArgs& a) {
  switch (nw) {
    case 1: return launch_partition_v<true, true, true, 1, 1, true>(grid, s, a);
    case 2: return launch_partition_v<true, true, true, 1, 2, true>(grid, s, a);
    case 8: return launch_partition_v<true, true, true, 1, 8, true>(grid, s, a);
    default: return launch_partition_v<true, true, true, 1, 4, true>(grid, s, a);
  }
}

// The measured default family (hardware convert, split P) exists for every
// prefetch depth and wave count; the A/B variants only at the default shape.
template <bool kFP8, bool kHw, bool kSplit>
static void launch_partition(int pd, int nw, dim3 grid, hipStream_t s, const DecodeArgs& a) {
  constexpr bool kFull = !kFP8 || (kHw && kSplit);
  if constexpr (kFull) {
    if (pd == 2) {
      switch (nw) {
        case 1: return launch_partition_v<kFP8, kHw, kSplit, 2, 1>(grid, s, a);
        case 2: return launch_partition_v<kFP8, kHw, kSplit, 2, 2>(grid, s, a);
        case 8: return launch_partition_v<kFP8, kHw, kSplit, 2, 8>(grid, s, a);
        default: return launch_partition_v<kFP8, kHw, kSplit, 2, 4>(grid, s, a);
      }
    }
    switch (nw) {
      case 1: return launch_partition_v<kFP8, kHw, kSplit, 1, 1>(grid, s, a);
      case 2: return launch_partition_v<kFP8, kHw, kSplit, 1, 2>(grid, s, a);
      case 8: return launch_partition_v<kFP8, kHw, kSplit, 1, 8>(grid, s, a);
      default: return launch_partition_v<kFP8, kHw, kSplit, 1, 4>(grid, s, a);
    }
  } else {
    (void)pd;
    (void)nw;
    launch_partition_v<kFP8, kHw, kSplit, 1, 4>(grid, s, a);
  }
}

// Waves per partition workgroup: each wave should stream at least 16 tiles,
// so short partitions get fewer waves (and skip most of the LDS merge).
static int waves_for(const DecodePlan& pl, size_t extra_lds = 0) {
  int nw = pl.cfg.waves;
  if (nw <= 0) {
    const int per_wave_tiles = 16;
    const int want = pl.a.part_blocks / per_wave_tiles;
    nw = want >= 4 ? 4 : (want >= 2 ? 2 : 1);
  }
  // the LDS merge buffer must fit one workgroup's 64 KiB
  while (nw > 1 &&
         (size_t)(nw * pl.a.g * kD + 2 * nw * 16) * sizeof(float) + extra_lds > 65536)
    nw /= 2;
  return nw;
}

// Partitions per wave for the chained kernel, or 0 for one workgroup per
// partition.  Chaining applies to short partitions (at most 64 blocks) of the
// default kernel family with per-tensor scales: each wave gets about 128
// tiles, as with the automatic partition length, while the grid keeps about
// 2048 waves.  Not for batches of 1024 or more (sequence, KV head) pairs,
// where lengths may be ragged: there the longest sequence's chains would be
// the tail (measured: 256 ragged sequences at 1024-token partitions, 286 us
// chained against 234 us with a workgroup per partition).
static int chain_for(const DecodePlan& pl, int32_t num_seqs) {
  const KernelConfig& c = pl.cfg;
  if (c.chain == 0 || pl.a.n_p_max <= 1 || pl.dyn) return 0;
  if (pl.fp8 && !(c.hw_cvt && c.split_p_fp8)) return 0;
  if (c.chain > 0) {  // explicit, down to what the LDS staging holds
    int chain = c.chain;
    while (chain > 1 && chain_lds_bytes(chain, pl.a.g) > kChainLdsMax) chain /= 2;
    return chain;
  }
  const int64_t pairs = (int64_t)num_seqs * pl.a.hkv;
  if (c.prefetch != 1 || c.waves != 0 || pl.a.part_blocks > 64 || pairs >= 1024) return 0;
  int chain = std::max(1, 128 / pl.a.part_blocks);
  while (chain > 1 && (pairs * ((pl.a.n_p_max + chain - 1) / chain) < 2048 ||
                       chain_lds_bytes(chain, pl.a.g) > kChainLdsMax))
    chain /= 2;
  // one partition per wave is fewer waves than a workgroup per partition
  // gives (measured: 64 x 2 KV heads x 8193 tokens at 1024-token partitions,
  // 59.6 us against 53.8 us)
  return chain >= 2 ? chain : 0;
}

template <bool kFP8, bool kAppend = false>
static void launch_chain(int chain, int32_t num_seqs, hipStream_t s, const DecodeArgs& a) {
  const int per_wg = kChainWaves * chain;
  const dim3 grid((unsigned)((a.n_p_max + per_wg - 1) / per_wg), (unsigned)a.hkv,
                  (unsigned)num_seqs);
  decode_chain_kernel<kFP8, kAppend>
      <<<grid, dim3(kChainWaves * kWave), chain_lds_bytes(chain, a.g), s>>>(a, chain);
}

// The newest token alone, one wave per (KV head, sequence), for the kernel
// variants that do not write it themselves (the A/B variants of
// kernel_config); launched before them on the same stream.
template <bool kFP8>
__global__ void __launch_bounds__(kWave) append_kernel(DecodeArgs a) {
  __shared__ __align__(16) uint8_t keep[kKeepBytes];
  const int kvh = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int L = clamp_len(a, b);
  if (L <= 0) return;
  const int phys = a.block_tables[(int64_t)b * a.max_blocks + ((L - 1) >> 4)];
  if ((unsigned)phys >= (unsigned)a.num_blocks) return;  // nothing is written
  append_keep<kFP8>(a, append_load(a, b, kvh, lane), lane, keep);
  TileRegs<kFP8> t;  // only the token's bytes are patched in and stored
#pragma unroll
  for (int i = 0; i < TileRegs<kFP8>::kVecs; ++i) {
    t.k[i] = u32x4{0u, 0u, 0u, 0u};
    t.v[i] = u32x4{0u, 0u, 0u, 0u};
  }
  patch_tile<kFP8>(t, keep, lane, (L - 1) & 15);
  append_store<kFP8>(a, t, phys, kvh, lane, (L - 1) & 15);
}

// The vector-ALU measurement variant covers FP8 per-tensor decode of groups
// of at most eight query heads.
static bool use_valu(const DecodePlan& pl) {
  return pl.cfg.valu && pl.fp8 && !pl.dyn && pl.a.g <= kValuG;
}

static pkv_status run_partitions(const DecodePlan& pl, int32_t num_seqs, hipStream_t s) {
  if (num_seqs == 0) return PKV_OK;
  const dim3 grid((unsigned)pl.a.n_p_max, (unsigned)pl.a.hkv, (unsigned)num_seqs);
  (void)hipGetLastError();
  const KernelConfig& c = pl.cfg;
  const int nw = waves_for(pl);
  if (use_valu(pl)) {
    const size_t lds = partition_lds(kValuWaves, pl.a.g, false, false);
    if (pl.a.shared_prefix != nullptr)
      decode_valu_kernel<0><<<grid, dim3(kValuWaves * kWave), lds, s>>>(pl.a);
    else
      decode_valu_kernel<kLoadNT><<<grid, dim3(kValuWaves * kWave), lds, s>>>(pl.a);
  } else if (const int chain = chain_for(pl, num_seqs)) {
    if (pl.fp8)
      launch_chain<true>(chain, num_seqs, s, pl.a);
    else
      launch_chain<false>(chain, num_seqs, s, pl.a);
  } else if (pl.dyn)
    launch_partition_dyn(nw, grid, s, pl.a);
  else if (!pl.fp8)
    launch_partition<false, false, true>(c.prefetch, nw, grid, s, pl.a);
  else if (c.hw_cvt)
    c.split_p_fp8 ? launch_partition<true, true, true>(c.prefetch, nw, grid, s, pl.a)
                  : launch_partition<true, true, false>(c.prefetch, nw, grid, s, pl.a);
  else
    c.split_p_fp8 ? launch_partition<true, false, true>(c.prefetch, nw, grid, s, pl.a)
                  : launch_partition<true, false, false>(c.prefetch, nw, grid, s, pl.a);
  return launch_status();
}

// The partition kernels that also write each sequence's newest token: the
// chained kernel or the default family of the partition kernel; otherwise
// append_kernel, then the partition kernels as without the write.
static pkv_status run_partitions_append(const DecodePlan& pl, int32_t num_seqs,
                                        hipStream_t s) {
  if (num_seqs == 0) return PKV_OK;
  (void)hipGetLastError();
  const KernelConfig& c = pl.cfg;
  if (const int chain = use_valu(pl) ? 0 : chain_for(pl, num_seqs)) {
    if (pl.fp8)
      launch_chain<true, true>(chain, num_seqs, s, pl.a);
    else
      launch_chain<false, true>(chain, num_seqs, s, pl.a);
    return launch_status();
  }
  const bool default_family =
      !use_valu(pl) && c.prefetch == 1 && (!pl.fp8 || (c.hw_cvt && c.split_p_fp8));
  if (!default_family) {
    const dim3 grid((unsigned)pl.a.hkv, (unsigned)num_seqs);
    if (pl.fp8)
      append_kernel<true><<<grid, dim3(kWave), 0, s>>>(pl.a);
    else
      append_kernel<false><<<grid, dim3(kWave), 0, s>>>(pl.a);
    const pkv_status st = launch_status();
    if (st != PKV_OK) return st;
    return run_partitions(pl, num_seqs, s);
  }
  const dim3 grid((unsigned)pl.a.n_p_max, (unsigned)pl.a.hkv, (unsigned)num_seqs);
  const int nw = waves_for(pl, kKeepBytes);
  if (pl.fp8)
    launch_partition_append<true>(nw, grid, s, pl.a);
  else
    launch_partition_append<false>(nw, grid, s, pl.a);
  return launch_status();
}

static pkv_status run_reduce(const DecodePlan& pl, int32_t num_seqs, hipStream_t s) {
  if (num_seqs == 0 || !pl.need_reduce) return PKV_OK;
  (void)hipGetLastError();
  const int64_t rows = (int64_t)num_seqs * pl.a.hq;
  if (pl.a.n_p_max > kManyPartitions) {
    decode_reduce_long_kernel<<<dim3((unsigned)rows), dim3(kRW * kWave), 0, s>>>(pl.a, rows);
  } else if (pl.a.n_p_max > kFewPartitions) {
    decode_reduce_kernel<true><<<dim3((unsigned)rows), dim3(kRW * kWave), 0, s>>>(pl.a, rows);
  } else if ((int64_t)num_seqs * pl.a.hkv < kGroupMergeMin) {
    // few groups: a wave per (sequence, query head) keeps more waves busy
    const int64_t grid = (rows + kRW - 1) / kRW;
    decode_reduce_kernel<false><<<dim3((unsigned)grid), dim3(256), 0, s>>>(pl.a, rows);
  } else {
    // one wave per (sequence, KV head); lanes a head: 64 / G rounded up to
    // a power of two, at most 32
    const int64_t groups = (int64_t)num_seqs * pl.a.hkv;
    const dim3 grid((unsigned)((groups + kRW - 1) / kRW));
    const int g = pl.a.g;
    if (g <= 2)
      decode_reduce_group_kernel<1><<<grid, dim3(kRW * kWave), 0, s>>>(pl.a, groups);
    else if (g <= 4)
      decode_reduce_group_kernel<2><<<grid, dim3(kRW * kWave), 0, s>>>(pl.a, groups);
    else if (g <= 8)
      decode_reduce_group_kernel<4><<<grid, dim3(kRW * kWave), 0, s>>>(pl.a, groups);
    else
      decode_reduce_group_kernel<8><<<grid, dim3(kRW * kWave), 0, s>>>(pl.a, groups);
  }
  return launch_status();
}

extern "C" pkv_status pkv_decode_partitions(float* out, const void* q, const void* k_pool,
                                            const void* v_pool, const int32_t* block_tables,
                                            int32_t max_blocks_per_seq,
                                            const int32_t* context_lens,
                                            const int32_t* shared_prefix_blocks, int32_t num_seqs,
                                            int32_t num_q_heads, int32_t max_context_len,
                                            const pkv_cache_layout* layout, float sm_scale,
                                            float k_scale, float v_scale,
                                            int32_t partition_size, void* workspace,
                                            uint64_t workspace_bytes, void* stream) {
  DecodePlan pl;
  pkv_status st = plan_decode(out, q, k_pool, v_pool, block_tables, max_blocks_per_seq,
                              context_lens, shared_prefix_blocks, num_seqs, num_q_heads,
                              max_context_len, layout, sm_scale, k_scale, v_scale, nullptr,
                              nullptr, partition_size, workspace, workspace_bytes, true, &pl,
                              static_cast<hipStream_t>(stream));
  if (st != PKV_OK) return st;
  return run_partitions(pl, num_seqs, static_cast<hipStream_t>(stream));
}

extern "C" pkv_status pkv_decode_reduce(float* out, const int32_t* context_lens,
                                        int32_t num_seqs, int32_t num_q_heads,
                                        int32_t max_context_len, int32_t max_blocks_per_seq,
                                        const pkv_cache_layout* layout, float v_scale,
                                        int32_t partition_size, void* workspace,
                                        uint64_t workspace_bytes, void* stream) {
  DecodePlan pl;
  pkv_status st = plan_decode(out, nullptr, nullptr, nullptr, nullptr, max_blocks_per_seq,
                              context_lens, nullptr, num_seqs, num_q_heads, max_context_len,
                              layout, 1.0f, 1.0f, v_scale, nullptr, nullptr, partition_size,
                              workspace, workspace_bytes, false, &pl,
                              static_cast<hipStream_t>(stream));
  if (st != PKV_OK) return st;
  return run_reduce(pl, num_seqs, static_cast<hipStream_t>(stream));
}

extern "C" pkv_status pkv_paged_attention_decode(
    float* out, const void* q, const void* k_pool, const void* v_pool,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* shared_prefix_blocks, int32_t num_seqs, int32_t num_q_heads,
    int32_t max_context_len,
    const pkv_cache_layout* layout, float sm_scale, float k_scale, float v_scale,
    int32_t partition_size, void* workspace, uint64_t workspace_bytes, void* stream) {
  DecodePlan pl;
  pkv_status st = plan_decode(out, q, k_pool, v_pool, block_tables, max_blocks_per_seq,
                              context_lens, shared_prefix_blocks, num_seqs, num_q_heads,
                              max_context_len, layout, sm_scale, k_scale, v_scale, nullptr,
                              nullptr, partition_size, workspace, workspace_bytes, true, &pl,
                              static_cast<hipStream_t>(stream));
  if (st != PKV_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = run_partitions(pl, num_seqs, s);
  if (st != PKV_OK) return st;
  return run_reduce(pl, num_seqs, s);
}

// The newest-token arguments of the *_append entry points.
static pkv_status set_append(DecodePlan* pl, int32_t num_seqs, const void* key,
                             const void* value, void* k_pool, void* v_pool) {
  if (num_seqs == 0) return PKV_OK;
  if (!key || !value || !aligned(key, 16) || !aligned(value, 16)) return PKV_ERR_INVALID_ARG;
  pl->a.new_k = static_cast<const _Float16*>(key);
  pl->a.new_v = static_cast<const _Float16*>(value);
  pl->a.k_wr = static_cast<uint8_t*>(k_pool);
  pl->a.v_wr = static_cast<uint8_t*>(v_pool);
  return PKV_OK;
}

extern "C" pkv_status pkv_decode_partitions_append(
    float* out, const void* q, const void* key, const void* value, void* k_pool, void* v_pool,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* shared_prefix_blocks, int32_t num_seqs, int32_t num_q_heads,
    int32_t max_context_len, const pkv_cache_layout* layout, float sm_scale, float k_scale,
    float v_scale, int32_t partition_size, void* workspace, uint64_t workspace_bytes,
    void* stream) {
  DecodePlan pl;
  pkv_status st = plan_decode(out, q, k_pool, v_pool, block_tables, max_blocks_per_seq,
                              context_lens, shared_prefix_blocks, num_seqs, num_q_heads,
                              max_context_len, layout, sm_scale, k_scale, v_scale, nullptr,
                              nullptr, partition_size, workspace, workspace_bytes, true, &pl,
                              static_cast<hipStream_t>(stream));
  if (st != PKV_OK) return st;
  st = set_append(&pl, num_seqs, key, value, k_pool, v_pool);
  if (st != PKV_OK) return st;
  return run_partitions_append(pl, num_seqs, static_cast<hipStream_t>(stream));
}

extern "C" pkv_status pkv_paged_attention_decode_append(
    float* out, const void* q, const void* key, const void* value, void* k_pool, void* v_pool,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* shared_prefix_blocks, int32_t num_seqs, int32_t num_q_heads,
    int32_t max_context_len, const pkv_cache_layout* layout, float sm_scale, float k_scale,
    float v_scale, int32_t partition_size, void* workspace, uint64_t workspace_bytes,
    void* stream) {
  DecodePlan pl;
  pkv_status st = plan_decode(out, q, k_pool, v_pool, block_tables, max_blocks_per_seq,
                              context_lens, shared_prefix_blocks, num_seqs, num_q_heads,
                              max_context_len, layout, sm_scale, k_scale, v_scale, nullptr,
                              nullptr, partition_size, workspace, workspace_bytes, true, &pl,
                              static_cast<hipStream_t>(stream));
  if (st != PKV_OK) return st;
  st = set_append(&pl, num_seqs, key, value, k_pool, v_pool);
  if (st != PKV_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = run_partitions_append(pl, num_seqs, s);
  if (st != PKV_OK) return st;
  return run_reduce(pl, num_seqs, s);
}

extern "C" uint64_t pkv_decode_cascade_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                                       int32_t num_kv_heads,
                                                       int32_t max_context_len,
                                                       int32_t max_prefix_blocks, int32_t dtype,
                                                       int32_t partition_size) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0 ||
      max_prefix_blocks < 0)
    return 0;
  if (dtype != PKV_F16 && dtype != PKV_FP8_E4M3FN) return 0;
  const int32_t part =
      resolve_partition(num_seqs, num_kv_heads, max_context_len, dtype, partition_size);
  if (part <= 0) return 0;
  return casc_layout(num_seqs, num_q_heads, max_context_len, part, max_prefix_blocks).ws.total;
}

// Largest batch for the flat cascade grid: each workgroup scans the batch
// (four sequences per lane per pass) to find its unit.
constexpr int32_t kFlatCascadeSeqs = 2048;

// The cascade after plan_decode: its workspace layout, the prefix items,
// the partition kernel (per-tensor scales: with or without the newest
// token's write; per-block scales: decode only), then the merge.
static pkv_status run_cascade(DecodePlan& pl, const int32_t* prefix_blocks,
                              const int32_t* prefix_groups, int32_t num_groups,
                              int32_t group_cap, int32_t max_prefix_blocks,
                              const int32_t* seq_order, int32_t tail_units,
                              const int32_t* tail_map, int32_t num_seqs, int32_t num_q_heads,
                              int32_t max_context_len, void* workspace,
                              uint64_t workspace_bytes, hipStream_t s) {
  DecodeArgs& a = pl.a;
  const bool append = a.new_k != nullptr;
  const int32_t part = a.part_blocks * kBS;
  const CascLayout cl = casc_layout(num_seqs, num_q_heads, max_context_len, part,
                                    num_groups > 0 ? max_prefix_blocks : 0);
  if (cl.ws.total > 0) {
    if (!workspace || workspace_bytes < cl.ws.total) return PKV_ERR_WORKSPACE;
    // the output rows start ml_bytes (a multiple of 256) past the base
    if (!aligned(workspace, 256)) return PKV_ERR_INVALID_ARG;
    a.ws_ml = static_cast<float*>(workspace);
    a.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + cl.ws.ml_bytes);
  }
  a.n_p_max = cl.ws.n_p_max;
  a.seq_order = seq_order;
  pl.need_reduce = cl.ws.n_p_max > 1;
  const int members = kMaxG / a.g;  // MFMA columns of one wave, G per member
  // waves per workgroup as for the plain kernel, within 64 KiB of LDS at 16
  // columns per wave
  int nw = waves_for(pl);
  while (nw > 1 && partition_lds(nw, kMaxG, append, true) > 65536) nw /= 2;
  // FP8 items with four waves share their tiles: each wave takes its own
  // members
  const bool shared_items = pl.fp8 && nw == kItemWaves;
  const int per_item = shared_items ? nw * members : members;
  const int64_t chunks = num_groups > 0 ? (group_cap + per_item - 1) / per_item : 0;
  const int64_t items = (int64_t)num_groups * chunks;
  if (items + num_seqs > 65535) return PKV_ERR_INVALID_ARG;  // grid z
  // the cascade always runs the hardware FP8 conversion: no factor 256 in
  // the scales whatever the A/B switch chose for the plain kernels
  if (pl.fp8 && !pl.dyn && !pl.cfg.hw_cvt) {
    a.qk_scale *= 1.0f / 256.0f;
    a.out_scale *= 1.0f / 256.0f;
  }
  if (num_groups > 0 && cl.s_max > 0) {
    a.casc_prefix = prefix_blocks;
    a.casc_groups = prefix_groups;
    a.casc_items = (int32_t)items;
    a.casc_chunks = (int32_t)chunks;
    a.casc_cap = group_cap;
    a.casc_m = members;
    a.casc_mi = per_item;
    a.casc_max = cl.s_max;
  }
  // Batches of up to kFlatCascadeSeqs sequences: a flat grid, KV head
  // fastest, that holds the prefix items and then the tail partitions in the
  // given order with no gaps: as many as the caller counted (tail_units), or
  // else an upper bound from max_context_len, past which the workgroups find
  // nothing and leave.  Larger batches: (partition, KV head, item or
  // sequence).
  dim3 grid((unsigned)cl.x_dim, (unsigned)a.hkv, (unsigned)(a.casc_items + num_seqs));
  const int64_t units =
      (int64_t)a.casc_items * std::max(1, cl.n_pp) +
      (tail_units > 0 ? (int64_t)tail_units : (int64_t)num_seqs * std::max(1, cl.n_pt));
  if (num_seqs <= kFlatCascadeSeqs && units * a.hkv < (1ll << 24)) {
    a.casc_flat = 1;
    a.casc_pp = std::max(1, cl.n_pp);
    grid = dim3((unsigned)(units * a.hkv));
    if (tail_map != nullptr) {  // tail_units is then its length
      a.casc_tail_map = reinterpret_cast<const int2*>(tail_map);
      a.casc_tail_count = tail_units;
    }
  }
  (void)hipGetLastError();
  if (pl.dyn)
    launch_partition_casc_dyn(nw, grid, s, a);
  else if (pl.fp8)
    append ? launch_partition_casc<true, true>(nw, grid, s, a)
           : launch_partition_casc<true, false>(nw, grid, s, a);
  else
    append ? launch_partition_casc<false, true>(nw, grid, s, a)
           : launch_partition_casc<false, false>(nw, grid, s, a);
  const pkv_status st = launch_status();
  if (st != PKV_OK) return st;
  return run_reduce(pl, num_seqs, s);
}

static pkv_status check_groups(int32_t num_groups, int32_t group_cap, int32_t max_prefix_blocks,
                               const int32_t* prefix_groups, const int32_t* prefix_blocks,
                               int32_t tail_units, const int32_t* tail_map) {
  if (num_groups < 0 || max_prefix_blocks < 0 || tail_units < 0) return PKV_ERR_INVALID_ARG;
  if (tail_map != nullptr && (tail_units == 0 || !aligned(tail_map, 8)))
    return PKV_ERR_INVALID_ARG;
  if (num_groups > 0 && (group_cap <= 0 || !prefix_groups || !prefix_blocks))
    return PKV_ERR_INVALID_ARG;
  return PKV_OK;
}

extern "C" pkv_status pkv_paged_attention_decode_cascade(
    float* out, const void* q, const void* key, const void* value, void* k_pool, void* v_pool,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* shared_prefix_blocks, const int32_t* prefix_blocks,
    const int32_t* prefix_groups, int32_t num_groups, int32_t group_cap,
    int32_t max_prefix_blocks, const int32_t* seq_order, int32_t tail_units,
    const int32_t* tail_map, int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
    const pkv_cache_layout* layout, float sm_scale, float k_scale, float v_scale,
    int32_t partition_size, void* workspace, uint64_t workspace_bytes, void* stream) {
  if ((key == nullptr) != (value == nullptr)) return PKV_ERR_INVALID_ARG;
  pkv_status st =
      check_groups(num_groups, group_cap, max_prefix_blocks, prefix_groups, prefix_blocks,
                   tail_units, tail_map);
  if (st != PKV_OK) return st;
  DecodePlan pl;
  // the plain plan's workspace is never larger than the cascade's
  st = plan_decode(out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens,
                   shared_prefix_blocks, num_seqs, num_q_heads, max_context_len, layout,
                   sm_scale, k_scale, v_scale, nullptr, nullptr, partition_size, workspace,
                   workspace_bytes, true, &pl,
                              static_cast<hipStream_t>(stream));
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  if (key) {
    st = set_append(&pl, num_seqs, key, value, k_pool, v_pool);
    if (st != PKV_OK) return st;
  }
  return run_cascade(pl, prefix_blocks, prefix_groups, num_groups, group_cap,
                     max_prefix_blocks, seq_order, tail_units, tail_map, num_seqs, num_q_heads,
                     max_context_len,
                     workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

extern "C" pkv_status pkv_paged_attention_decode_cascade_dynamic(
    float* out, const void* q, const void* k_pool, const void* v_pool,
    const float* k_block_scales, const float* v_block_scales, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, const int32_t* shared_prefix_blocks,
    const int32_t* prefix_blocks, const int32_t* prefix_groups, int32_t num_groups,
    int32_t group_cap, int32_t max_prefix_blocks, const int32_t* seq_order, int32_t tail_units,
    const int32_t* tail_map, int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
    const pkv_cache_layout* layout, float sm_scale, int32_t partition_size, void* workspace,
    uint64_t workspace_bytes, void* stream) {
  if (!k_block_scales || !v_block_scales) return PKV_ERR_INVALID_ARG;
  pkv_status st =
      check_groups(num_groups, group_cap, max_prefix_blocks, prefix_groups, prefix_blocks,
                   tail_units, tail_map);
  if (st != PKV_OK) return st;
  DecodePlan pl;
  st = plan_decode(out, q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens,
                   shared_prefix_blocks, num_seqs, num_q_heads, max_context_len, layout,
                   sm_scale, 1.0f, 1.0f, k_block_scales, v_block_scales, partition_size,
                   workspace, workspace_bytes, true, &pl,
                              static_cast<hipStream_t>(stream));
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  return run_cascade(pl, prefix_blocks, prefix_groups, num_groups, group_cap,
                     max_prefix_blocks, seq_order, tail_units, tail_map, num_seqs, num_q_heads,
                     max_context_len,
                     workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

extern "C" pkv_status pkv_paged_attention_decode_dynamic(
    float* out, const void* q, const void* k_pool, const void* v_pool,
    const float* k_block_scales, const float* v_block_scales, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, const int32_t* shared_prefix_blocks,
    int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
    const pkv_cache_layout* layout, float sm_scale, int32_t partition_size, void* workspace,
    uint64_t workspace_bytes, void* stream) {
  if (!k_block_scales || !v_block_scales) return PKV_ERR_INVALID_ARG;
  DecodePlan pl;
  pkv_status st = plan_decode(out, q, k_pool, v_pool, block_tables, max_blocks_per_seq,
                              context_lens, shared_prefix_blocks, num_seqs, num_q_heads,
                              max_context_len, layout, sm_scale, 1.0f, 1.0f, k_block_scales,
                              v_block_scales, partition_size, workspace, workspace_bytes, true,
                              &pl,
                              static_cast<hipStream_t>(stream));
  if (st != PKV_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = run_partitions(pl, num_seqs, s);
  if (st != PKV_OK) return st;
  return run_reduce(pl, num_seqs, s);
}
