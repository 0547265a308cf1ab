/*
 * pkv_oracle.c — plain, slow CPU oracle for the paged KV cache hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant generator
 * with the HIP implementation: every formula below is written from the pages
 * and from the definition of the number format.
 *
 * Pages (cited by title and section):
 *   [FP8-128K] "Optimización de KV Cache con PagedAttention y Cuantización FP8
 *              para Contextos Largos (128K)"
 *   [PRIMER-8] "LLM Primer VI, Capítulo 8 — Gestión de caché KV de nueva
 *              generación"
 *   [GLOSSARY] "PagedAttention y Gestión de KV-Cache"
 *
 * Arithmetic is fp64 throughout; the only narrow values are the ones the
 * method itself stores (fp16 inputs, FP8 codes, the fp32 quotient x / scale).
 *
 * Parity pins (checked by tests/test_oracle_*.py, never by this file):
 *   - e4m3 decode: all 256 codes against a library view-cast and the format's
 *     landmark values;
 *   - e4m3 encode: brute-force nearest-code search; pinned against a library
 *     cast and against hand-derived tie and saturation cases;
 *   - write: bytes land at the documented layout offsets (golden table);
 *   - decode attention: a library scaled-dot-product attention on the
 *     logically ordered rows, closed forms (one token, equal keys, zero
 *     query, two tokens), and invariances (block permutation, shared vs
 *     copied prefix, grouped-query vs repeated heads);
 *   - per-block dynamic scales: one-call fills against a library cast,
 *     growth by a power of two (old codes drop one binade exactly), the
 *     fresh-block reset, the floor and non-finite inputs, error bounds after
 *     repeated growth, and decode against library attention on rows rebuilt
 *     with their own block's scale.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_BS 16 /* tokens per block: [FP8-128K] §3, [PRIMER-8] §8.1 */

/* ------------------------------------------------------------------ numbers */

/* IEEE binary16 bits -> value: 1 sign bit, 5 exponent bits (bias 15), 10
 * mantissa bits; exponent 0 is subnormal, exponent 31 is inf/NaN. */
double oracle_f16_to_double(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* m/1024 * 2^-14 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp(1.0 + m / 1024.0, e - 15);
  return s ? -v : v;
}

/* OCP FP8 E4M3FN code -> value ([FP8-128K] §6.2 and §8 name the E4M3 format;
 * the variant with largest finite 448 is the one whose scale is amax/448).
 * Sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 holds the
 * subnormals m/8 * 2^-6; S.1111.111 is NaN; there are no infinities. */
double oracle_e4m3_decode(uint8_t c) {
  int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7)
    return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* The values of the 127 finite non-negative codes and of all 65536 fp16 bit
 * patterns, filled once when the library is loaded, from the two definitions
 * above: a lookup gives exactly what calling them gives, without repeating
 * the exponent arithmetic for every element of a large pool. */
static double orc_code_value[0x7F];
static double orc_f16_value[65536];
static void orc_fill_tables(void) __attribute__((constructor));
static void orc_fill_tables(void) {
  for (int c = 0; c <= 0x7E; ++c)
    orc_code_value[c] = oracle_e4m3_decode((uint8_t)c);
  for (int h = 0; h < 65536; ++h)
    orc_f16_value[h] = oracle_f16_to_double((uint16_t)h);
}

/* Nearest E4M3FN code to the fp32 value u, found by trying every finite
 * non-negative code (the definition of round-to-nearest written out).  On an
 * exact tie the code with mantissa LSB 0 (the even code) wins.  Values whose
 * magnitude is at least the largest finite value 448, and infinities, take
 * 448 (saturating conversion); NaN takes the NaN code 0x7F with u's sign. */
uint8_t oracle_e4m3_encode(float u) {
  uint8_t sign = signbit(u) ? 0x80 : 0x00;
  if (isnan(u))
    return (uint8_t)(0x7F | sign);
  double a = fabs((double)u);
  if (a >= 448.0)
    return (uint8_t)(0x7E | sign);
  int best = 0;
  double best_d = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    double d = fabs(orc_code_value[c] - a);
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best_d = d;
      best = c;
    }
  }
  return (uint8_t)(best | sign);
}

/* Element-wise oracle_e4m3_encode over an array of fp32 values. */
void oracle_e4m3_encode_array(const float* u, int64_t n, uint8_t* codes) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    codes[i] = oracle_e4m3_encode(u[i]);
}

/* The fp32 quotient the write rounds: correctly rounded x / scale.  The
 * division is done in fp64 and rounded once to fp32; with 53 >= 2*24 + 2 bits
 * that equals the correctly rounded fp32 quotient. */
float oracle_quotient(double x, float scale) { return (float)(x / (double)scale); }

/* Encode n fp16 values with one scale (codes[i] = E4M3(x[i] / scale)).  The
 * encoder depends only on the 16-bit input for a fixed scale, so each of the
 * 65536 inputs is encoded once by the brute-force search and then looked up;
 * the result is the same as calling oracle_e4m3_encode per element. */
void oracle_quantize_f16(const uint16_t* x, int64_t n, float scale, uint8_t* codes) {
  uint8_t* lut = (uint8_t*)malloc(65536);
#pragma omp parallel for schedule(static)
  for (int h = 0; h < 65536; ++h)
    lut[h] = oracle_e4m3_encode(oracle_quotient(oracle_f16_to_double((uint16_t)h), scale));
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    codes[i] = lut[x[i]];
  free(lut);
}

/* ------------------------------------------------------------------- layout */

/* Element offset of (token t, channel d) inside one (block, kv head) tile of
 * BS x D elements; x = elements per 16 bytes (16 for FP8, 8 for fp16).  This
 * is the layout libpkv documents for its pools (the pages prescribe none):
 * K is chunked by 16-byte runs of channels, V is tiled in groups of 4 tokens
 * by 16 channels. */
static int64_t orc_k_offset(int t, int d, int x) {
  return (int64_t)(d / x) * (ORC_BS * x) + (int64_t)t * x + d % x;
}
static int64_t orc_v_offset(int t, int d, int x) {
  int n = d / 16, v = x / 4;
  return (int64_t)(n / v) * (64 * x) + (int64_t)((t / 4) * 16 + d % 16) * x + (n % v) * 4 + t % 4;
}
int64_t oracle_k_offset(int t, int d, int elem_bytes) { return orc_k_offset(t, d, 16 / elem_bytes); }
int64_t oracle_v_offset(int t, int d, int elem_bytes) { return orc_v_offset(t, d, 16 / elem_bytes); }

/* Byte address of element (block, kv head, t, d) in a pool. */
static int64_t orc_addr(int is_v, int64_t block, int h, int t, int d, int Hkv, int D, int e) {
  int x = 16 / e;
  int64_t tile = (block * Hkv + h) * (int64_t)(ORC_BS * D);
  int64_t within = is_v ? orc_v_offset(t, d, x) : orc_k_offset(t, d, x);
  return (tile + within) * e;
}

/* Read one cached element as a real number: fp16 bits widened, FP8 code
 * decoded and multiplied by the tensor's scale ([FP8-128K] §4 and §8). */
static double orc_load(const uint8_t* pool, int is_v, int64_t block, int h, int t, int d, int Hkv,
                       int D, int fp8, double scale) {
  if (fp8)
    return oracle_e4m3_decode(pool[orc_addr(is_v, block, h, t, d, Hkv, D, 1)]) * scale;
  uint16_t bits;
  memcpy(&bits, pool + orc_addr(is_v, block, h, t, d, Hkv, D, 2), 2);
  return oracle_f16_to_double(bits);
}

/* Slot of logical position pos of a sequence: its block table names the
 * physical block of logical block pos / BS, and the token sits at pos % BS in
 * it ([PRIMER-8] §8.1; [GLOSSARY] §2 figure: logical 0 -> 7, 1 -> 2, 2 -> 11). */
int64_t oracle_slot(const int32_t* table_row, int64_t pos) {
  return (int64_t)table_row[pos / ORC_BS] * ORC_BS + pos % ORC_BS;
}

/* -------------------------------------------------------------------- write */

/* Store T new K/V rows ([T][Hkv][D] fp16 bits) into their slots.  fp16 pools
 * get the bits as they are; FP8 pools get E4M3(x / scale) ([FP8-128K] §4:
 * the new rows are turned into 8-bit values as they are written).  A negative
 * slot, or one past the pool, is skipped.  The code of an element depends only
 * on its 16 input bits and the scale, so each of the 65536 inputs is encoded
 * once per scale by the brute-force search and then looked up. */
void oracle_reshape_and_cache(const uint16_t* key, const uint16_t* value, uint8_t* k_pool,
                              uint8_t* v_pool, const int64_t* slots, int T, int Hkv, int D,
                              int num_blocks, int fp8, float k_scale, float v_scale) {
  int e = fp8 ? 1 : 2;
  uint8_t *klut = NULL, *vlut = NULL;
  if (fp8) {
    klut = (uint8_t*)malloc(65536);
    vlut = (uint8_t*)malloc(65536);
#pragma omp parallel for schedule(static)
    for (int h = 0; h < 65536; ++h) {
      double x = oracle_f16_to_double((uint16_t)h);
      klut[h] = oracle_e4m3_encode(oracle_quotient(x, k_scale));
      vlut[h] = oracle_e4m3_encode(oracle_quotient(x, v_scale));
    }
  }
#pragma omp parallel for schedule(static)
  for (int i = 0; i < T; ++i) {
    int64_t s = slots[i];
    if (s < 0 || s >= (int64_t)num_blocks * ORC_BS)
      continue;
    int64_t block = s / ORC_BS;
    int t = (int)(s % ORC_BS);
    for (int h = 0; h < Hkv; ++h)
      for (int d = 0; d < D; ++d) {
        int64_t src = ((int64_t)i * Hkv + h) * D + d;
        int64_t ka = orc_addr(0, block, h, t, d, Hkv, D, e);
        int64_t va = orc_addr(1, block, h, t, d, Hkv, D, e);
        if (fp8) {
          k_pool[ka] = klut[key[src]];
          v_pool[va] = vlut[value[src]];
        } else {
          memcpy(k_pool + ka, key + src, 2);
          memcpy(v_pool + va, value + src, 2);
        }
      }
  }
  free(klut);
  free(vlut);
}

/* ------------------------------------------------------------------- decode */

/* Decode attention for a batch, one query token per sequence.  For sequence b
 * and query head h (KV head kv = h / G, G = Hq / Hkv consecutive query heads
 * per KV head, the 8:1 grouping of [FP8-128K] §2):
 *   k_t, v_t = cached rows of logical token t < L_b, found through the block
 *              table ([PRIMER-8] §8.1: gathered by indirection),
 *   s_t      = sm_scale * (q . k_t),
 *   out      = sum_t exp(s_t - max s) v_t / sum_t exp(s_t - max s).
 * L_b = 0 gives zeros.  out is fp64 [B][Hq][D].  The (b, h) pairs are
 * independent and are spread over `threads` OpenMP threads (0 = default). */
static void orc_decode(double* out, const uint16_t* q, const uint8_t* k_pool,
                       const uint8_t* v_pool, const int32_t* block_tables, int max_blocks,
                       const int32_t* context_lens, int B, int Hq, int Hkv, int D, int fp8,
                       float sm_scale, float k_scale, float v_scale, const float* k_bscales,
                       const float* v_bscales, int threads) {
  int G = Hq / Hkv;
  double ks = fp8 ? (double)k_scale : 1.0, vs = fp8 ? (double)v_scale : 1.0;
#ifdef _OPENMP
  if (threads > 0)
    omp_set_num_threads(threads);
#else
  (void)threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < (int64_t)B * Hq; ++bh) {
    int b = (int)(bh / Hq), h = (int)(bh % Hq), kv = h / G;
    int L = context_lens[b];
    double* o = out + bh * D;
    for (int d = 0; d < D; ++d)
      o[d] = 0.0;
    if (L <= 0)
      continue;
    const int32_t* row = block_tables + (int64_t)b * max_blocks;
    double* qd = (double*)malloc(sizeof(double) * D);
    double* s = (double*)malloc(sizeof(double) * L);
    for (int d = 0; d < D; ++d)
      qd[d] = oracle_f16_to_double(q[bh * D + d]);
    double m = -INFINITY;
    for (int t = 0; t < L; ++t) {
      int64_t block = row[t / ORC_BS];
      double kst = k_bscales ? (double)k_bscales[block * Hkv + kv] : ks;
      double dot = 0.0;
      for (int d = 0; d < D; ++d)
        dot += qd[d] * orc_load(k_pool, 0, block, kv, t % ORC_BS, d, Hkv, D, fp8, kst);
      s[t] = (double)sm_scale * dot;
      if (s[t] > m)
        m = s[t];
    }
    double den = 0.0;
    for (int t = 0; t < L; ++t) {
      int64_t block = row[t / ORC_BS];
      double w = exp(s[t] - m);
      double vst = v_bscales ? (double)v_bscales[block * Hkv + kv] : vs;
      den += w;
      for (int d = 0; d < D; ++d)
        o[d] += w * orc_load(v_pool, 1, block, kv, t % ORC_BS, d, Hkv, D, fp8, vst);
    }
    for (int d = 0; d < D; ++d)
      o[d] /= den;
    free(qd);
    free(s);
  }
}

/* Number of OpenMP threads a parallel region would use (for reports). */
void oracle_paged_attention_decode(double* out, const uint16_t* q, const uint8_t* k_pool,
                                   const uint8_t* v_pool, const int32_t* block_tables,
                                   int max_blocks, const int32_t* context_lens, int B, int Hq,
                                   int Hkv, int D, int fp8, float sm_scale, float k_scale,
                                   float v_scale, int threads) {
  orc_decode(out, q, k_pool, v_pool, block_tables, max_blocks, context_lens, B, Hq, Hkv, D, fp8,
             sm_scale, k_scale, v_scale, NULL, NULL, threads);
}

/* Decode over an FP8 pool whose blocks carry their own scales: the element
 * (block, kv head, t, d) stands for E4M3(code) * scales[block][kv head]
 * ([FP8-128K] §8, dynamic scaling: one scale per cache block). */
void oracle_paged_attention_decode_dynamic(double* out, const uint16_t* q, const uint8_t* k_pool,
                                           const uint8_t* v_pool, const float* k_bscales,
                                           const float* v_bscales, const int32_t* block_tables,
                                           int max_blocks, const int32_t* context_lens, int B,
                                           int Hq, int Hkv, int D, float sm_scale, int threads) {
  orc_decode(out, q, k_pool, v_pool, block_tables, max_blocks, context_lens, B, Hq, Hkv, D, 1,
             sm_scale, 1.0f, 1.0f, k_bscales, v_bscales, threads);
}

/* ------------------------------------------------------ chunked prefill */

/* Attention for a chunk of prompt tokens over the paged cache ([FP8-128K]
 * §5: with chunked prefill a long prompt is cut into packets of tokens that
 * run between decode steps).  Sequence b's chunk is its last n_b tokens:
 * rows query_start[b] .. query_start[b+1]-1 of q, whose keys and values are
 * already in the cache, so the sequence holds L_b = context_lens[b] tokens.
 * Row i of the chunk sits at position p = L_b - n_b + i and attends, causally,
 * to the tokens 0..p of its sequence, with each KV head serving G = Hq / Hkv
 * query heads.  Plain softmax(sm_scale * q.k) v in fp64, tokens in order.
 * With k_bscales / v_bscales (FP8 only) each cached element stands for
 * E4M3(code) * the scale of its own (block, kv head), as in decode. */
static void orc_prefill(double* out, const uint16_t* q, const uint8_t* k_pool,
                        const uint8_t* v_pool, const int32_t* block_tables, int max_blocks,
                        const int32_t* context_lens, const int32_t* query_start, int B, int Hq,
                        int Hkv, int D, int fp8, float sm_scale, float k_scale, float v_scale,
                        const float* k_bscales, const float* v_bscales, int threads) {
  int G = Hq / Hkv;
  double kfac = fp8 ? (double)k_scale : 1.0;
  double vfac = fp8 ? (double)v_scale : 1.0;
  int64_t rows = query_start[B];
#ifdef _OPENMP
  if (threads > 0)
    omp_set_num_threads(threads);
#else
  (void)threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t rh = 0; rh < rows * Hq; ++rh) {
    int64_t r = rh / Hq;
    int h = (int)(rh % Hq), kvh = h / G;
    int b = 0;
    while (query_start[b + 1] <= r)
      ++b;
    int n = query_start[b + 1] - query_start[b];
    int L = context_lens[b];
    int64_t pos = (int64_t)L - n + (r - query_start[b]);
    double* o = out + rh * D;
    for (int d = 0; d < D; ++d)
      o[d] = 0.0;
    if (pos < 0)
      continue; /* a chunk longer than its sequence: such rows see nothing */
    const int32_t* row = block_tables + (int64_t)b * max_blocks;
    int64_t cnt = pos + 1;
    double* qd = (double*)malloc(sizeof(double) * D);
    double* sc = (double*)malloc(sizeof(double) * cnt);
    for (int d = 0; d < D; ++d)
      qd[d] = oracle_f16_to_double(q[rh * D + d]);
    double m = -INFINITY;
    for (int64_t t = 0; t < cnt; ++t) {
      int64_t block = row[t / ORC_BS];
      double kst = k_bscales ? (double)k_bscales[block * Hkv + kvh] : kfac;
      double dot = 0.0;
      for (int d = 0; d < D; ++d)
        dot += qd[d] * orc_load(k_pool, 0, block, kvh, (int)(t % ORC_BS), d, Hkv, D, fp8, kst);
      sc[t] = (double)sm_scale * dot;
      if (sc[t] > m)
        m = sc[t];
    }
    double wsum = 0.0;
    for (int64_t t = 0; t < cnt; ++t) {
      int64_t blk = row[t / ORC_BS];
      double w = exp(sc[t] - m);
      double vst = v_bscales ? (double)v_bscales[blk * Hkv + kvh] : vfac;
      wsum += w;
      for (int d = 0; d < D; ++d)
        o[d] += w * orc_load(v_pool, 1, blk, kvh, (int)(t % ORC_BS), d, Hkv, D, fp8, vst);
    }
    for (int d = 0; d < D; ++d)
      o[d] /= wsum;
    free(qd);
    free(sc);
  }
}

void oracle_paged_prefill_attention(double* out, const uint16_t* q, const uint8_t* k_pool,
                                    const uint8_t* v_pool, const int32_t* block_tables,
                                    int max_blocks, const int32_t* context_lens,
                                    const int32_t* query_start, int B, int Hq, int Hkv, int D,
                                    int fp8, float sm_scale, float k_scale, float v_scale,
                                    int threads) {
  orc_prefill(out, q, k_pool, v_pool, block_tables, max_blocks, context_lens, query_start, B, Hq,
              Hkv, D, fp8, sm_scale, k_scale, v_scale, NULL, NULL, threads);
}

/* Chunked prefill over an FP8 pool whose (block, kv head) tiles carry their
 * own K and V scales ([FP8-128K] §5 chunked prefill over the cache of §8's
 * dynamic scaling). */
void oracle_paged_prefill_attention_dynamic(double* out, const uint16_t* q,
                                            const uint8_t* k_pool, const uint8_t* v_pool,
                                            const float* k_bscales, const float* v_bscales,
                                            const int32_t* block_tables, int max_blocks,
                                            const int32_t* context_lens,
                                            const int32_t* query_start, int B, int Hq, int Hkv,
                                            int D, float sm_scale, int threads) {
  orc_prefill(out, q, k_pool, v_pool, block_tables, max_blocks, context_lens, query_start, B, Hq,
              Hkv, D, 1, sm_scale, 1.0f, 1.0f, k_bscales, v_bscales, threads);
}

/* ------------------------------------------------- write with block scales */

/* Store T new K/V rows into an FP8 pool whose (block, kv head) tiles carry
 * their own scale ([FP8-128K] §8, dynamic scaling: the MaxAbs of each block is
 * measured as the cache is written and the scale follows it).  The pages fix
 * neither the floor nor what happens to a block filled over several calls;
 * the reading implemented here, per call and per (block b, head h), for K
 * and V separately, with W the offsets of b this call writes:
 *   1. a = largest |x| over the finite elements of the new rows in W;
 *   2. the block is fresh when offset 0 is in W (its first token arrives
 *      now): its old scale and its other slots are disregarded;
 *   3. s_old = 0 if fresh, else the stored scale;
 *      s_new = max(s_old, fp32(a / 448), 2^-126), so the largest element maps
 *      to 448 and a scale is never zero;
 *   4. if not fresh and s_new > s_old, every slot of b outside W is
 *      re-encoded: code' = E4M3(fp32(E4M3value(code) * fp32(s_old / s_new)))
 *      (a NaN code stays NaN) -- the old rows are only held as codes;
 *   5. each new element becomes E4M3(fp32(x / s_new)); the stored scale
 *      becomes s_new.
 * Slots must be distinct within a call; negative or out-of-pool slots are
 * skipped. */
static double orc_abs_finite(uint16_t bits) {
  double x = orc_f16_value[bits];
  return isfinite(x) ? fabs(x) : 0.0;
}

void oracle_reshape_and_cache_dynamic(const uint16_t* key, const uint16_t* value,
                                      uint8_t* k_pool, uint8_t* v_pool, float* k_bscales,
                                      float* v_bscales, const int64_t* slots, int T, int Hkv,
                                      int D, int num_blocks) {
  const float floor_scale = (float)ldexp(1.0, -126);
  uint32_t* written = (uint32_t*)calloc((size_t)num_blocks, sizeof(uint32_t));
  double* amax = (double*)calloc((size_t)num_blocks * Hkv * 2, sizeof(double));
  float* s_new = (float*)calloc((size_t)num_blocks * Hkv * 2, sizeof(float));
  /* 1. offsets written, then MaxAbs of the new rows per (block, head, K/V)
   *    (each head's maxima are its own: heads run in parallel) */
  for (int i = 0; i < T; ++i) {
    int64_t sl = slots[i];
    if (sl >= 0 && sl < (int64_t)num_blocks * ORC_BS)
      written[sl / ORC_BS] |= 1u << (sl % ORC_BS);
  }
#pragma omp parallel for schedule(static)
  for (int h = 0; h < Hkv; ++h)
    for (int i = 0; i < T; ++i) {
      int64_t sl = slots[i];
      if (sl < 0 || sl >= (int64_t)num_blocks * ORC_BS)
        continue;
      int64_t b = sl / ORC_BS;
      double* ak = &amax[(b * Hkv + h) * 2];
      for (int d = 0; d < D; ++d) {
        int64_t src = ((int64_t)i * Hkv + h) * D + d;
        double xk = orc_abs_finite(key[src]), xv = orc_abs_finite(value[src]);
        if (xk > ak[0])
          ak[0] = xk;
        if (xv > ak[1])
          ak[1] = xv;
      }
    }
  /* 2-4. new scales, and old slots re-encoded where a scale grew */
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t b = 0; b < num_blocks; ++b) {
    if (!written[b])
      continue;
    int fresh = (written[b] & 1u) != 0;
    for (int h = 0; h < Hkv; ++h)
      for (int is_v = 0; is_v < 2; ++is_v) {
        float* stored = is_v ? &v_bscales[b * Hkv + h] : &k_bscales[b * Hkv + h];
        uint8_t* pool = is_v ? v_pool : k_pool;
        float s_old = fresh ? 0.0f : *stored;
        float s = oracle_quotient(amax[(b * Hkv + h) * 2 + is_v], 448.0f);
        if (s < s_old)
          s = s_old;
        if (s < floor_scale)
          s = floor_scale;
        s_new[(b * Hkv + h) * 2 + is_v] = s;
        if (!fresh && s > s_old) {
          float r = oracle_quotient((double)s_old, s);
          for (int t = 0; t < ORC_BS; ++t) {
            if (written[b] & (1u << t))
              continue;
            for (int d = 0; d < D; ++d) {
              uint8_t* c = &pool[orc_addr(is_v, b, h, t, d, Hkv, D, 1)];
              if ((*c & 0x7F) == 0x7F)
                continue; /* NaN stays NaN */
              *c = oracle_e4m3_encode((float)(oracle_e4m3_decode(*c) * (double)r));
            }
          }
        }
        *stored = s;
      }
  }
  /* 5. the new rows, encoded with their block's new scale */
#pragma omp parallel for schedule(static)
  for (int i = 0; i < T; ++i) {
    int64_t sl = slots[i];
    if (sl < 0 || sl >= (int64_t)num_blocks * ORC_BS)
      continue;
    int64_t b = sl / ORC_BS;
    int t = (int)(sl % ORC_BS);
    for (int h = 0; h < Hkv; ++h)
      for (int d = 0; d < D; ++d) {
        int64_t src = ((int64_t)i * Hkv + h) * D + d;
        float sk = s_new[(b * Hkv + h) * 2], sv = s_new[(b * Hkv + h) * 2 + 1];
        k_pool[orc_addr(0, b, h, t, d, Hkv, D, 1)] =
            oracle_e4m3_encode(oracle_quotient(orc_f16_value[key[src]], sk));
        v_pool[orc_addr(1, b, h, t, d, Hkv, D, 1)] =
            oracle_e4m3_encode(oracle_quotient(orc_f16_value[value[src]], sv));
      }
  }
  free(written);
  free(amax);
  free(s_new);
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
