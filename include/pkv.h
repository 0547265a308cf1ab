/*
 * pkv.h — C ABI of libpkv: a paged KV cache and decode-phase PagedAttention
 * for AMD Instinct MI355X (gfx950).
 *
 * Sources the operations follow (cited by page title and section):
 *   [FP8-128K] "Optimización de KV Cache con PagedAttention y Cuantización FP8
 *              para Contextos Largos (128K)" (thecalata.com)
 *   [PRIMER-8] "LLM Primer VI, Capítulo 8 — Gestión de caché KV de nueva
 *              generación" (actionbridge.io)
 *   [KV-SLOW]  "KV Cache y PagedAttention: por qué se reduce la velocidad de tu
 *              servidor LLM" (gyaansetu.com, repost of a dev.to article)
 *   [GLOSSARY] "PagedAttention y Gestión de KV-Cache" (gotburnout.io glossary)
 *
 * What the library computes
 *   The KV cache is cut into fixed 16-token blocks held in one flat pool per
 *   tensor (K and V); the physical blocks of a sequence need not be adjacent,
 *   and a per-sequence block table maps logical block j to a physical block id
 *   ([FP8-128K] §3; [PRIMER-8] §8.1; [GLOSSARY] §2 block-table figure).
 *   The decode kernel takes that table as an extra input and gathers keys and
 *   values through it instead of slicing a contiguous slab ([PRIMER-8] §8.1).
 *   New K/V rows can be stored as fp16 or converted on the fly to 8-bit
 *   floating point E4M3, halving the cache ([FP8-128K] §4; the E4M3 format
 *   is named in §6.2 and §8).
 *   One query token per sequence is decoded per call ([PRIMER-8], closing
 *   section on Chapter 9; [KV-SLOW] "¿Qué es el KV cache?").
 *
 * Conventions for every function below
 *   - Status codes: PKV_OK (0) or a negative pkv_status; nothing throws.
 *   - Device pointers are caller-owned HIP device memory; the library never
 *     allocates device memory.  "stream" is a hipStream_t passed as void*
 *     (NULL = the null stream).  Device calls are asynchronous on that stream;
 *     argument errors are detected on the host before anything is launched.
 *   - Contents of device tables (block ids, lengths, slots) cannot be checked
 *     on the host without a copy; kernels never access memory outside the
 *     buffers described by the sizes passed in (out-of-range ids are skipped),
 *     but the numerical result for invalid table contents is unspecified.
 *   - Host handles (pkv_pool) are not thread-safe; the caller serialises.
 *
 * Cache layout (fixed by this library; the pages do not prescribe one)
 *   block_size BS = 16 tokens, head_dim D = 128, element size e = 2 (fp16) or
 *   1 (FP8).  Both pools are [num_blocks][num_kv_heads][BS*D] elements, so the
 *   tile of one (block, kv head) is BS*D*e contiguous bytes (4 KiB fp16,
 *   2 KiB FP8).  Inside a tile the element of token t (0..15) and channel
 *   d (0..127) sits at element offset
 *     K:  (d / x) * (BS * x) + t * x + (d % x),        x = 16 / e
 *     V:  (n / v) * (64 * x) + ((t / 4) * 16 + d % 16) * x + (n % v) * 4 + t % 4,
 *         n = d / 16, v = x / 4
 *   i.e. both tiles are stored in the order the gfx950 matrix-core operands
 *   consume them, so one wavefront reads a whole tile with 16-byte loads that
 *   cover 1 KiB of contiguous memory per instruction.
 *   A token's slot is phys_block * 16 + position % 16.
 *
 * FP8 encoding (PKV_FP8_E4M3FN)
 *   OCP E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits,
 *   exponent 0 subnormal, S.1111.111 NaN, no infinities, largest finite 448.
 *   code = E4M3(u) with u = x / scale computed as a correctly rounded fp32
 *   division; rounding to nearest, ties to the even code; finite values at or
 *   above 448 in magnitude (and infinities) saturate to +-448; NaN maps to
 *   0x7F | sign.  Decoding is code_value * scale.  One fp32 scale per pool
 *   (a per-tensor scale), supplied by the caller ([FP8-128K] §8 describes the
 *   dynamic and the calibrated ways of obtaining it).
 */
#ifndef PKV_H
#define PKV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_BLOCK_SIZE 16
#define PKV_HEAD_DIM 128
#define PKV_MAX_GQA_GROUP 16

typedef int32_t pkv_status;
enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1,    /* null/misaligned pointer, bad size or count */
  PKV_ERR_UNSUPPORTED = -2,    /* block_size != 16, head_dim != 128, group > 16, unknown dtype */
  PKV_ERR_NO_FREE_BLOCKS = -3, /* pool exhausted; state unchanged ([FP8-128K] §6.1) */
  PKV_ERR_HIP = -4,            /* a HIP launch failed */
  PKV_ERR_WORKSPACE = -5,      /* decode workspace smaller than required */
  PKV_ERR_BAD_HANDLE = -6,     /* unknown or freed sequence id, null pool */
  PKV_ERR_REFCOUNT = -7        /* refcount would underflow (double free) */
};

typedef enum { PKV_F16 = 0, PKV_FP8_E4M3FN = 1 } pkv_dtype;

/* Geometry of one K pool and its V pool (they share it). */
typedef struct {
  int32_t num_blocks;   /* physical blocks in the pool */
  int32_t block_size;   /* tokens per block; must be 16 for device calls */
  int32_t num_kv_heads; /* KV heads stored per block */
  int32_t head_dim;     /* must be 128 for device calls */
  int32_t dtype;        /* pkv_dtype */
} pkv_cache_layout;

/* Human-readable name of a status code (static storage, never NULL). */
const char* pkv_status_string(pkv_status status);

/* ------------------------------------------------------------------ sizing */

/* Bytes of KV cache one token occupies across a model:
 * 2 (K and V) * n_layers * n_kv_heads * d_head * elem_bytes
 * ([FP8-128K] §2, the sizing formula and its Llama-3.1-70B example).
 * Returns 0 if any argument is not positive. */
uint64_t pkv_bytes_per_token(int32_t n_layers, int32_t n_kv_heads, int32_t d_head,
                             int32_t elem_bytes);

/* Bytes of ONE pool (K or V) with this layout; 0 for an invalid layout. */
uint64_t pkv_pool_bytes(const pkv_cache_layout* layout);

/* Longest split-KV partition (tokens) the decode will use for this shape:
 * `requested` if it is a positive multiple of 16, else (requested == 0) the
 * library's choice; -1 if `requested` or `dtype` is invalid.  Each sequence
 * of L tokens is cut into ceil(L / P) partitions of equal whole-block length,
 * each at most P tokens. */
int32_t pkv_decode_partition_size(int32_t num_seqs, int32_t num_kv_heads,
                                  int32_t max_context_len, int32_t dtype, int32_t requested);

/* Workspace bytes pkv_paged_attention_decode needs for this shape, cache
 * dtype and partition request (same rules as pkv_decode_partition_size); 0
 * if no merge is needed (every sequence fits one partition) or the arguments
 * are invalid. */
uint64_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t max_context_len,
                                    int32_t dtype, int32_t partition_size);

/* ------------------------------------------------------------ table checks */

/* Check block tables and lengths held in HOST memory: for every sequence b,
 * 0 <= context_lens[b] <= min(max_context_len, 16 * max_blocks_per_seq) and
 * each of its first ceil(L_b / 16) entries names a block of the pool,
 * 0 <= id < num_blocks (the decode kernel reads the table as an extra input
 * to find each token's physical block: [PRIMER-8] §8.1).  Returns
 * INVALID_ARG at the first sequence that breaks this (its index in
 * *bad_seq_out, else -1 there; bad_seq_out may be NULL) or for bad sizes
 * (num_seqs < 0, max_blocks_per_seq <= 0, num_blocks <= 0, null arrays with
 * num_seqs > 0).  Pure host function. */
pkv_status pkv_validate_tables(const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t num_seqs,
                               int32_t max_context_len, int32_t num_blocks,
                               int32_t* bad_seq_out);

/* Debug checks of device tables.  While on, every decode and prefill call
 * first copies its block table and lengths to the host (synchronising its
 * stream) and returns INVALID_ARG, launching nothing, if pkv_validate_tables
 * rejects them; without it the kernels clamp lengths and skip ids outside
 * the pool.  Off by default; the environment variable PKV_DEBUG_CHECKS set to
 * anything but "" or "0" turns it on at load.  A debug call cannot be
 * captured into a HIP graph (it copies to the host).  pkv_set_debug_checks
 * returns the previous setting; process-wide. */
int32_t pkv_set_debug_checks(int32_t on);
int32_t pkv_get_debug_checks(void);

/* ------------------------------------------------------------ device calls */

/* Store new K/V rows into their cache slots ([FP8-128K] §4: the new rows are
 * converted to 8 bits as they are written; [PRIMER-8] §8.1: slots live in
 * physical blocks named by the block table).
 *   key, value    device fp16 [num_tokens][num_kv_heads][128], contiguous,
 *                 16-byte aligned.
 *   k_pool/v_pool device pools laid out as described at the top of this file.
 *   slot_mapping  device int64 [num_tokens]; slot = block * 16 + offset;
 *                 a negative slot means "skip this token"; slots at or beyond
 *                 num_blocks * 16 are skipped as well.
 *   k_scale/v_scale  per-tensor scales, used only for PKV_FP8_E4M3FN; must be
 *                 finite and > 0 then.
 * fp16 pools receive the 16 input bits unchanged; FP8 pools receive the code
 * defined under "FP8 encoding" above.  A slot named twice in one call holds
 * one of the two rows afterwards, which one unspecified.  Blocks whose 16
 * slots the call fills in order from consecutive tokens (any alignment of
 * the tokens within the call) are written as whole tiles; other slots row
 * by row.  num_tokens == 0 is a no-op. */
pkv_status pkv_reshape_and_cache(const void* key, const void* value, void* k_pool,
                                 void* v_pool, const int64_t* slot_mapping,
                                 int32_t num_tokens, const pkv_cache_layout* layout,
                                 float k_scale, float v_scale, void* stream);

/* Decode attention over the paged cache: for each sequence b and query head h,
 *   out[b][h][:] = softmax_t( sm_scale * q[b][h] . K_t ) . V_t ,  t < L_b,
 * with K_t, V_t the rows of KV head h / (num_q_heads / num_kv_heads) of the
 * sequence's tokens in logical order, gathered through block_tables
 * ([PRIMER-8] §8.1; grouped-query heads as in [FP8-128K] §2, where 8 query
 * heads share each KV head).  FP8 rows are decoded as code * k_scale or
 * code * v_scale.  L_b = 0 yields zeros.  The result equals ordinary attention
 * over the same tokens in logical order, whatever physical blocks hold them.
 *   out           device fp32 [num_seqs][num_q_heads][128]
 *   q             device fp16 [num_seqs][num_q_heads][128], 16-byte aligned
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]
 *   context_lens  device int32 [num_seqs]; L_b includes the token being
 *                 decoded; values are clamped to [0, min(max_context_len,
 *                 16 * max_blocks_per_seq)].
 *   shared_prefix_blocks  optional device int32 [num_seqs] (NULL = none): the
 *                 number of leading blocks of each sequence that other
 *                 sequences of the batch also read (a shared prompt, a fork's
 *                 parent; pkv_seq_shared_prefix_blocks reports it).  A cache
 *                 hint only: those tiles are loaded through the caches so the
 *                 sibling sequences can hit, all others are streamed past
 *                 them.  The result does not depend on it.
 *   max_context_len  host upper bound on every L_b (sizes the workspace).
 *   num_q_heads must be a multiple of layout->num_kv_heads with a group of at
 *   most 16.
 *   partition_size   longest split-KV partition in tokens: 0 = library
 *                 choice, else a positive multiple of 16.  A sequence of L
 *                 tokens is cut into ceil(L / partition_size) partitions of
 *                 equal whole-block length.  Each partition yields a partial
 *                 (max, sum, unnormalised output) and a second kernel merges
 *                 them with the log-sum-exp rule.
 *   workspace     device scratch of at least pkv_decode_workspace_bytes(...)
 *                 bytes, 256-byte aligned; its contents are internal.
 * Launches the partition kernel and, when some sequence spans more than one
 * partition, the merge kernel, both on `stream`. */
pkv_status pkv_paged_attention_decode(float* out, const void* q, const void* k_pool,
                                      const void* v_pool, const int32_t* block_tables,
                                      int32_t max_blocks_per_seq,
                                      const int32_t* context_lens,
                                      const int32_t* shared_prefix_blocks, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t max_context_len,
                                      const pkv_cache_layout* layout, float sm_scale,
                                      float k_scale, float v_scale,
                                      int32_t partition_size, void* workspace,
                                      uint64_t workspace_bytes, void* stream);

/* The two halves of pkv_paged_attention_decode, for callers that time or
 * schedule them separately.  Same arguments and rules; calling
 * pkv_decode_partitions then pkv_decode_reduce with identical arguments and
 * workspace is exactly pkv_paged_attention_decode.  pkv_decode_partitions
 * writes `out` directly for every sequence that fits one partition;
 * pkv_decode_reduce writes the rest. */
pkv_status pkv_decode_partitions(float* out, const void* q, const void* k_pool,
                                 const void* v_pool, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 const int32_t* shared_prefix_blocks, int32_t num_seqs,
                                 int32_t num_q_heads,
                                 int32_t max_context_len, const pkv_cache_layout* layout,
                                 float sm_scale, float k_scale, float v_scale,
                                 int32_t partition_size, void* workspace,
                                 uint64_t workspace_bytes, void* stream);
pkv_status pkv_decode_reduce(float* out, const int32_t* context_lens, int32_t num_seqs,
                             int32_t num_q_heads, int32_t max_context_len,
                             int32_t max_blocks_per_seq, const pkv_cache_layout* layout,
                             float v_scale, int32_t partition_size, void* workspace,
                             uint64_t workspace_bytes, void* stream);

/* A decode step in one call: write each sequence's newest token into the
 * cache, then attend over its whole context, that token included -- the
 * cache write of [FP8-128K] §4 (new rows converted to 8 bits as they are
 * stored) followed by the decode attention above.
 * Sequence b's newest token is at position L_b - 1 (L_b = context_lens[b]
 * after the clamp described above); its slot is
 *   block_tables[b][(L_b - 1) / 16] * 16 + (L_b - 1) % 16,
 * so its block must already be in the table (pkv_seq_append assigns it) and
 * must not be shared with another sequence (copy-on-write done first).
 *   key, value    device fp16 [num_seqs][num_kv_heads][128], contiguous,
 *                 16-byte aligned: the new token's K and V rows.
 *   k_pool/v_pool the pools, read and written.
 *   k_scale/v_scale  per-tensor scales (FP8): the new rows are stored as the
 *                 codes pkv_reshape_and_cache would store, and all rows are
 *                 decoded with them.
 * Other arguments as in pkv_paged_attention_decode.  The pools and `out` end
 * up exactly as after pkv_reshape_and_cache (slot_mapping as above) then
 * pkv_paged_attention_decode with the same arguments; L_b = 0 writes nothing;
 * a block id outside [0, num_blocks) is skipped, as that write skips it.
 * The kernel that reads a sequence's last block also stores its newest rows
 * and uses them from registers, so no separate write launch is made (with
 * the PKV_DECODE_PREFETCH / PKV_FP8_* A/B variants a small write kernel
 * runs first).  pkv_decode_partitions_append is its first half, completed by
 * pkv_decode_reduce with the same arguments. */
pkv_status pkv_paged_attention_decode_append(
    float* out, const void* q, const void* key, const void* value, void* k_pool, void* v_pool,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* shared_prefix_blocks, int32_t num_seqs, int32_t num_q_heads,
    int32_t max_context_len, const pkv_cache_layout* layout, float sm_scale, float k_scale,
    float v_scale, int32_t partition_size, void* workspace, uint64_t workspace_bytes,
    void* stream);
pkv_status pkv_decode_partitions_append(
    float* out, const void* q, const void* key, const void* value, void* k_pool, void* v_pool,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* shared_prefix_blocks, int32_t num_seqs, int32_t num_q_heads,
    int32_t max_context_len, const pkv_cache_layout* layout, float sm_scale, float k_scale,
    float v_scale, int32_t partition_size, void* workspace, uint64_t workspace_bytes,
    void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * pkv_paged_attention_decode_append with no workspace argument.  Its
 * split-KV partials live in a fixed array of PKV_NOALLOC_SCRATCH_BYTES that
 * the library holds on each device it runs on until the process ends; the
 * call itself allocates nothing.  Same arguments, kernels and results as
 * pkv_paged_attention_decode_append.  WORKSPACE if the shape needs more than
 * the array (pkv_decode_workspace_bytes tells), HIP if the array's address
 * cannot be found.  Every call on a device uses that device's one array:
 * calls that overlap in time on one device (other streams, other threads)
 * race and must not be made. */
#define PKV_NOALLOC_SCRATCH_BYTES (64ull << 20)
pkv_status pkv_paged_attention_decode_append_noalloc(
    float* out, const void* q, const void* key, const void* value, void* k_pool, void* v_pool,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* shared_prefix_blocks, int32_t num_seqs, int32_t num_q_heads,
    int32_t max_context_len, const pkv_cache_layout* layout, float sm_scale, float k_scale,
    float v_scale, int32_t partition_size, void* stream);

/* Decode over shared prefixes as a cascade.  Sequences that share their
 * leading blocks (a common system prompt, or the branches of a parallel
 * sample: [PRIMER-8] §8.1, [GLOSSARY] §3.02) hold the same physical blocks
 * there.  Here those blocks are attended once per group: one wave serves up
 * to 16 / G members of a group (G query heads each, one MFMA column per
 * head) over every prefix tile, storing one split-KV partial per member;
 * each sequence's tail (the blocks after its prefix) is split into
 * partitions as in pkv_paged_attention_decode, and the log-sum-exp merge
 * combines prefix and tail partials.  The result equals the plain decode
 * over the same tables within rounding (the split-KV identity).
 *   prefix_blocks  device int32 [num_seqs]: S_b, the leading blocks of
 *                  sequence b attended by its group; 0 = none.  Used only
 *                  if 0 < S_b <= max_prefix_blocks and 16 * S_b < L_b (the
 *                  newest token stays in the tail); otherwise sequence b is
 *                  decoded on its own, and groups must leave it out.
 *   prefix_groups  device int32 [num_groups][group_cap]: the batch indices
 *                  of each group's members, -1 for an empty slot.  The first
 *                  slot of a group holds a member (a row starting with -1,
 *                  or with a sequence that has no prefix, is skipped whole);
 *                  all members of a group
 *                  have the same S_b and the same first S_b table entries;
 *                  every sequence with a used S_b > 0 is in exactly one
 *                  group.  (pkv_pool_prefix_groups builds these.)  Results
 *                  for sequences that break this are unspecified; no memory
 *                  outside the arguments is touched.
 *   max_prefix_blocks  host: the largest S_b; sizes the workspace
 *                  (pkv_decode_cascade_workspace_bytes).
 *   seq_order      optional device int32 [num_seqs] (NULL = batch order): a
 *                  permutation of the batch; the sequences' tails are
 *                  scheduled in this order after the prefix items.  Longest
 *                  tails first (pkv_pool_prefix_groups gives that order)
 *                  keeps the longest workgroups from starting last.  An
 *                  entry outside [0, num_seqs) is skipped; a sequence not
 *                  listed gets unspecified output (no memory outside the
 *                  arguments is touched).
 *   tail_units     host: the tail work of the batch, summed over the
 *                  sequences seq_order lists (every one without it) of
 *                  max(1, ceil(tail blocks / (P / 16))) -- the partitions of
 *                  each tail, one for a sequence with no tail tokens to
 *                  write zeros -- as pkv_pool_cascade_tail_units counts it
 *                  from the pool; 0 = unknown.  It sizes the launch: with
 *                  the exact count every workgroup takes one unit, and
 *                  prefix and tail units follow each other with no empty
 *                  workgroups.  Any positive value gives the same result (a
 *                  smaller one makes workgroups take several units, a larger
 *                  one leaves some idle); 0 launches an upper bound derived
 *                  from max_context_len.
 *   tail_map       optional device int32 [tail_units][2], 8-byte aligned:
 *                  the (batch index, tail partition) of every tail unit in
 *                  schedule order, as pkv_pool_cascade_tail_map writes it
 *                  for this batch, order and partition size; tail_units is
 *                  then its length (INVALID_ARG if 0).  With it, a
 *                  workgroup finds its tail unit with one load instead of a
 *                  scan over the lengths (two dependent round trips to
 *                  memory).  NULL = the scan.  An entry outside the batch or
 *                  with a negative partition is skipped; a map that does not
 *                  list every tail partition gives unspecified output for
 *                  those sequences (no memory outside the arguments is
 *                  touched).  Used with batches of at most 4096 sequences
 *                  (larger ones need no unit search).
 *   key, value     the newest tokens' rows as in
 *                  pkv_paged_attention_decode_append, written in the same
 *                  launch; both null = decode only.
 * Other arguments as in pkv_paged_attention_decode_append.  The kernel
 * variant is the default family whatever PKV_* variant switches say.
 * Errors: INVALID_ARG for one of key/value null, negative counts (tail_units
 * included), groups
 * without arrays, or more than 65535 items plus sequences
 * (num_groups * ceil(group_cap / floor(16 / G)) + num_seqs); WORKSPACE if the
 * workspace is smaller than pkv_decode_cascade_workspace_bytes. */
pkv_status pkv_paged_attention_decode_cascade(
    float* out, const void* q, const void* key, const void* value, void* k_pool, void* v_pool,
    const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* shared_prefix_blocks, const int32_t* prefix_blocks,
    const int32_t* prefix_groups, int32_t num_groups, int32_t group_cap,
    int32_t max_prefix_blocks, const int32_t* seq_order, int32_t tail_units,
    const int32_t* tail_map, int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
    const pkv_cache_layout* layout, float sm_scale, float k_scale, float v_scale,
    int32_t partition_size, void* workspace, uint64_t workspace_bytes, void* stream);

/* The cascade over a cache with per-(block, KV head) FP8 scales (the
 * decode of pkv_paged_attention_decode_dynamic, with the prefix groups,
 * order and workspace of pkv_paged_attention_decode_cascade; decode only:
 * the newest rows are written first by pkv_reshape_and_cache_dynamic).
 * FP8 layouts only (UNSUPPORTED otherwise); null block scales:
 * INVALID_ARG. */
pkv_status pkv_paged_attention_decode_cascade_dynamic(
    float* out, const void* q, const void* k_pool, const void* v_pool,
    const float* k_block_scales, const float* v_block_scales, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, const int32_t* shared_prefix_blocks,
    const int32_t* prefix_blocks, const int32_t* prefix_groups, int32_t num_groups,
    int32_t group_cap, int32_t max_prefix_blocks, const int32_t* seq_order, int32_t tail_units,
    const int32_t* tail_map, int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
    const pkv_cache_layout* layout, float sm_scale, int32_t partition_size, void* workspace,
    uint64_t workspace_bytes, void* stream);

/* Workspace of pkv_paged_attention_decode_cascade: room for each sequence's
 * prefix partitions (ceil(16 * max_prefix_blocks / P)) and tail partitions;
 * 0 when no sequence needs a merge or on invalid arguments. */
uint64_t pkv_decode_cascade_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t max_context_len,
                                            int32_t max_prefix_blocks, int32_t dtype,
                                            int32_t partition_size);

/* Copy whole blocks (every KV head, K and V) for copy-on-write: a shared
 * block is duplicated before a sequence writes into it ([KV-SLOW] "Cómo
 * PagedAttention soluciona esto"; [GLOSSARY] §3.01).
 *   src_dst_pairs device int32 [num_pairs][2] (source block, destination
 *                 block); pairs with an id outside [0, num_blocks) are skipped.
 * Destinations must be distinct and must not be sources of another pair. */
pkv_status pkv_copy_blocks(void* k_pool, void* v_pool, const pkv_cache_layout* layout,
                           const int32_t* src_dst_pairs, int32_t num_pairs, void* stream);

/* ------------------------------------------------------- chunked prefill
 *
 * [FP8-128K] §5: with chunked prefill a long prompt is processed in packets of
 * tokens between decode steps.  This call is the attention of one packet:
 * sequence b's chunk is its last n_b = query_start[b+1] - query_start[b]
 * tokens, whose keys and values the caller has already written into the
 * cache (pkv_reshape_and_cache), so the sequence holds L_b = context_lens[b]
 * tokens.  Chunk row i sits at position p = L_b - n_b + i and attends
 * causally to tokens 0..p:
 *   out[r][h][:] = softmax_t(sm_scale * q[r][h] . k_t) v_t over t = 0..p,
 * with k_t, v_t read through block_tables[b] for KV head h / G as in decode.
 *   out          device fp32 [rows][num_q_heads][128], rows = query_start[B];
 *   q            device fp16 [rows][num_q_heads][128];
 *   query_start  device int32 [num_seqs + 1], non-decreasing, query_start[0] =
 *                0 (empty chunks allowed);
 *   max_query_len  host upper bound on every n_b (sizes the grid);
 *   max_context_len  host clamp on every L_b, as in decode;
 *   other arguments as in pkv_paged_attention_decode (group of at most 16).
 * Rows whose position is negative (a chunk longer than its sequence) are
 * written as zeros.  Value slots past L_b may hold anything.  Arithmetic: FP8
 * codes are converted to fp16 exactly, products on fp16 MFMA with fp32
 * accumulation, probabilities rounded to fp16.  No workspace. */
pkv_status pkv_paged_prefill_attention(float* out, const void* q, const void* k_pool,
                                       const void* v_pool, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                                       const int32_t* query_start, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t max_query_len,
                                       int32_t max_context_len, const pkv_cache_layout* layout,
                                       float sm_scale, float k_scale, float v_scale,
                                       void* stream);

/* --------------------------------------------- per-block dynamic FP8 scales
 *
 * [FP8-128K] §8, dynamic scaling: instead of one scale per tensor, each
 * (block, KV head) tile of K and of V carries its own fp32 scale, measured
 * from the MaxAbs of the values written into it as the cache is written.
 * FP8 pools only (PKV_ERR_UNSUPPORTED otherwise).
 *   k_block_scales, v_block_scales  device fp32 [num_blocks][num_kv_heads],
 *                 caller-owned, updated in place by the write; an element of
 *                 tile (b, h) stands for E4M3value(code) * scales[b][h].
 *
 * Write rule, per call and per tile (K and V apart), with W the offsets of
 * the block this call writes (the pages leave open how a block filled over
 * several calls is scaled; this is the library's reading):
 *   - the block is fresh when offset 0 is in W: its first token arrives now,
 *     so its stored scale and its other slots are disregarded;
 *   - s_new = max(s_old (0 if fresh), fp32(m / 448), 2^-126) with m the
 *     largest magnitude among the finite new values: the block's MaxAbs maps
 *     to 448 and a scale is never zero;
 *   - if a non-fresh tile's scale grows, its slots outside W are re-encoded,
 *     code' = E4M3(fp32(E4M3value(code) * fp32(s_old / s_new))), NaN codes
 *     kept (the earlier rows exist only as codes);
 *   - new elements become E4M3(fp32(x / s_new)) (RNE, saturating, NaN kept).
 * Slots must be distinct within a call; calls are ordered by the stream. */

/* Scratch bytes pkv_reshape_and_cache_dynamic needs for this layout:
 * num_blocks * (2 * num_kv_heads + 1) 32-bit words, rounded up to 256; 0 for
 * a non-FP8 or invalid layout. */
uint64_t pkv_reshape_dynamic_workspace_bytes(const pkv_cache_layout* layout);

/* Write T new K/V rows with per-block scales (rule above).  Arguments as in
 * pkv_reshape_and_cache, plus the two scale arrays and a device workspace of
 * at least pkv_reshape_dynamic_workspace_bytes(layout) bytes, 256-byte
 * aligned, whose contents are internal (no clearing needed).  Three kernel
 * launches on `stream`. */
pkv_status pkv_reshape_and_cache_dynamic(const void* key, const void* value, void* k_pool,
                                         void* v_pool, float* k_block_scales,
                                         float* v_block_scales, const int64_t* slot_mapping,
                                         int32_t num_tokens, const pkv_cache_layout* layout,
                                         void* workspace, uint64_t workspace_bytes,
                                         void* stream);

/* Decode attention over an FP8 pool with per-block scales: as
 * pkv_paged_attention_decode, with each tile's K and V scale read from the
 * arrays in place of the per-tensor k_scale and v_scale (so there are none).
 * The workspace is sized by pkv_decode_workspace_bytes for the FP8 dtype.
 * Table entries outside [0, num_blocks) read as zeros, as in the plain call. */
pkv_status pkv_paged_attention_decode_dynamic(
    float* out, const void* q, const void* k_pool, const void* v_pool,
    const float* k_block_scales, const float* v_block_scales, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens,
    const int32_t* shared_prefix_blocks, int32_t num_seqs, int32_t num_q_heads,
    int32_t max_context_len, const pkv_cache_layout* layout, float sm_scale,
    int32_t partition_size, void* workspace, uint64_t workspace_bytes, void* stream);

/* Chunked prefill over an FP8 pool with per-block scales ([FP8-128K] §5 over
 * the cache of §8): as pkv_paged_prefill_attention, with each tile's K and V
 * scale read from the arrays in place of the per-tensor scales.  Within a
 * workgroup the probabilities of a tile are multiplied by its V scale over
 * the largest V scale met so far before rounding to fp16: as one fp16 value
 * while that largest scale is at most 8/448, as an fp16 hi + lo pair after
 * it (one rounding moves an output by at most 2^-11 of the largest |V| it
 * multiplies).  No workspace;
 * PKV_ERR_UNSUPPORTED for fp16 pools, PKV_ERR_INVALID_ARG for a null scale
 * array. */
pkv_status pkv_paged_prefill_attention_dynamic(
    float* out, const void* q, const void* k_pool, const void* v_pool,
    const float* k_block_scales, const float* v_block_scales, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, const int32_t* query_start,
    int32_t num_seqs, int32_t num_q_heads, int32_t max_query_len, int32_t max_context_len,
    const pkv_cache_layout* layout, float sm_scale, void* stream);

/* pkv_copy_blocks for a pool with per-block scales: the destination also
 * takes the source's scale rows (copy-on-write of a partly filled block). */
pkv_status pkv_copy_blocks_dynamic(void* k_pool, void* v_pool, float* k_block_scales,
                                   float* v_block_scales, const pkv_cache_layout* layout,
                                   const int32_t* src_dst_pairs, int32_t num_pairs,
                                   void* stream);

/* ------------------------------------------------ host block pool and tables */

/* A pool of physical block ids with reference counts, and the sequences that
 * map logical blocks onto them ([PRIMER-8] §8.1: fixed blocks in a flat pool,
 * per-sequence block tables, refcounted sharing; [KV-SLOW]: blocks are taken
 * only as a sequence grows).  Host memory only; the caller copies block tables
 * and slots to the device. */
typedef struct pkv_pool pkv_pool;

/* Create a pool of num_blocks free blocks of block_size tokens.  The free
 * list is popped in ascending id order if shuffle_seed == 0, else in an order
 * shuffled with that seed. */
pkv_status pkv_pool_create(int32_t num_blocks, int32_t block_size, uint64_t shuffle_seed,
                           pkv_pool** out);
void pkv_pool_destroy(pkv_pool* pool);
int32_t pkv_pool_num_blocks(const pkv_pool* pool);
/* Blocks on the free list (held by no sequence and not in the prefix cache). */
int32_t pkv_pool_num_free(const pkv_pool* pool);
/* Fraction of blocks in use, (num_blocks - available) / num_blocks, where
 * available = free blocks + evictable prefix-cache blocks: the cache usage
 * gauge that [FP8-128K] §7 says to watch (alert above 0.90). */
double pkv_pool_usage(const pkv_pool* pool);
/* Reference count of a block (number of sequences whose table holds it);
 * -1 for an id out of range. */
int32_t pkv_pool_refcount(const pkv_pool* pool, int32_t block);

/* New empty sequence; its id is written to *seq_out. */
pkv_status pkv_seq_create(pkv_pool* pool, int32_t* seq_out);
/* New sequence sharing every block of `parent` (each refcount + 1), with the
 * parent's length: the branching of [PRIMER-8] §8.1 and [GLOSSARY] §3.02. */
pkv_status pkv_seq_fork(pkv_pool* pool, int32_t parent, int32_t* child_out);
/* Extend a sequence by n_tokens and return their slots.
 *   slots_out      host int64 [n_tokens] (may be NULL when n_tokens == 0)
 *   cow_pairs_out  host int32 [2]: if the sequence's partially filled last block
 *                  is shared, it is replaced by a fresh block and the pair
 *                  (old, new) is written here for pkv_copy_blocks;
 *   n_cow_out      number of pairs written (0 or 1).
 * Blocks are taken from the free list only when a new block is needed.
 * All or nothing: PKV_ERR_NO_FREE_BLOCKS leaves every state unchanged. */
pkv_status pkv_seq_append(pkv_pool* pool, int32_t seq, int32_t n_tokens, int64_t* slots_out,
                          int32_t* cow_pairs_out, int32_t* n_cow_out);
/* One token for each of seqs[0..n), in that order: a decode step's slot
 * assignment in one call ([PRIMER-8] §8.1, blocks allocated on demand).
 * Each sequence is appended as by pkv_seq_append with one token.
 *   slots_out      host int64 [n]: the new token's slot of each sequence
 *   cow_pairs_out  host int32 [n][2]: the copy-on-write pairs, packed; their
 *                  count in *n_cow_out (copy them before writing the tokens)
 *   *n_done_out    sequences appended.  On an error (the first failing
 *                  sequence's status, e.g. NO_FREE_BLOCKS) the sequences
 *                  before it are appended and it and those after it are
 *                  unchanged. */
pkv_status pkv_seq_append_each(pkv_pool* pool, const int32_t* seqs, int32_t n,
                               int64_t* slots_out, int32_t* cow_pairs_out, int32_t* n_cow_out,
                               int32_t* n_done_out);
/* The tail work of a cascade decode of seqs[0..n) (pkv_pool_prefix_groups'
 * batch, whose prefix_blocks and max_prefix_blocks it takes): for each
 * sequence, with L its length in the pool and S its prefix blocks where
 * 0 < S <= max_prefix_blocks and 16 * S < L (else S = 0), the count
 * max(1, ceil((ceil(L / 16) - S) / (partition_size / 16))), summed into
 * *units_out -- the tail_units argument of
 * pkv_paged_attention_decode_cascade.  partition_size: the split the decode
 * uses (pkv_decode_partition_size), a positive multiple of 16.
 * BAD_HANDLE for an unknown sequence; INVALID_ARG for bad sizes. */
pkv_status pkv_pool_cascade_tail_units(const pkv_pool* pool, const int32_t* seqs, int32_t n,
                                       const int32_t* prefix_blocks,
                                       int32_t max_prefix_blocks, int32_t partition_size,
                                       int64_t* units_out);
/* The tail_map argument of pkv_paged_attention_decode_cascade: the tail
 * units pkv_pool_cascade_tail_units counts, listed in the decode's schedule
 * order.  For each batch index b in order[0..n) (0..n-1 when order is NULL),
 * its tail partitions 0 .. max(1, ceil((ceil(L / 16) - S) / (P / 16))) - 1
 * as pairs (b, partition), L and S as for pkv_pool_cascade_tail_units.
 *   prefix_blocks  host int32 [n], max_prefix_blocks: as returned by
 *                  pkv_pool_prefix_groups for seqs;
 *   order          host int32 [n] or NULL: the seq_order the decode gets (a
 *                  permutation of 0..n-1);
 *   map_out        host int32 [map_cap][2];
 *   *units_out     the units listed (the decode's tail_units).
 * BAD_HANDLE for an unknown sequence; INVALID_ARG for bad sizes, an order
 * entry outside [0, n), or more units than map_cap (nothing is written
 * past map_cap). */
pkv_status pkv_pool_cascade_tail_map(const pkv_pool* pool, const int32_t* seqs, int32_t n,
                                     const int32_t* prefix_blocks, int32_t max_prefix_blocks,
                                     int32_t partition_size, const int32_t* order,
                                     int32_t* map_out, int64_t map_cap, int64_t* units_out);
/* Release a sequence: each of its blocks loses one reference; at zero it
 * returns to the free list, or becomes evictable if the prefix cache holds it
 * ([GLOSSARY] §4.02: pages of a cancelled request go back to the pool at once,
 * else memory leaks). */
pkv_status pkv_seq_free(pkv_pool* pool, int32_t seq);
/* Copy a sequence's block table into out[0..n) with n = number of blocks;
 * *n_out = n always; PKV_ERR_INVALID_ARG if cap < n (nothing copied). */
pkv_status pkv_seq_block_table(const pkv_pool* pool, int32_t seq, int32_t* out, int32_t cap,
                               int32_t* n_out);
/* Tokens held by a sequence; -1 for an unknown id. */
int64_t pkv_seq_len(const pkv_pool* pool, int32_t seq);
/* Number of live sequences. */
int32_t pkv_pool_num_seqs(const pkv_pool* pool);
/* Leading blocks of a sequence that are shared with another sequence
 * (reference count > 1) -- the shared_prefix_blocks hint of the decode;
 * -1 for an unknown id. */
int32_t pkv_seq_shared_prefix_blocks(const pkv_pool* pool, int32_t seq);
/* Prefix groups of a decode batch for pkv_paged_attention_decode_cascade.
 * seqs[0..n) are the batch's sequences in batch order.  Entries whose first
 * block is the same shared block ([PRIMER-8] §8.1: forks of one prompt hold
 * the same pages) form a group; its prefix is the longest run of leading
 * table entries that all its members hold, shortened so that every member
 * keeps at least one token after it.  A first block held by one entry, or a
 * prefix of 0 blocks, gives no group.  A group of more than group_cap entries
 * is split into groups of at most group_cap.
 *   prefix_blocks_out  host int32 [n]: each entry's prefix blocks, 0 = none
 *   groups_out         host int32 [cap_groups][group_cap]: batch indices of
 *                      each group's members in batch order, -1 padded
 *   *n_groups_out      groups found; *max_prefix_out their largest prefix
 *   order_out          optional host int32 [n] (NULL = not wanted): batch
 *                      indices by decreasing tail (tokens after the prefix),
 *                      ties in batch order -- the cascade's seq_order
 * BAD_HANDLE for an unknown sequence id; INVALID_ARG for bad sizes or if
 * more than cap_groups groups are found (then only the two counts are set).
 * Reads the pool only. */
pkv_status pkv_pool_prefix_groups(const pkv_pool* pool, const int32_t* seqs, int32_t n,
                                  int32_t group_cap, int32_t cap_groups,
                                  int32_t* prefix_blocks_out, int32_t* groups_out,
                                  int32_t* n_groups_out, int32_t* max_prefix_out,
                                  int32_t* order_out);

/* ------------------------------------------------------------- prefix cache
 *
 * A map from prompt chunks to filled blocks ([PRIMER-8] §8.3: the prompt is
 * hashed in block-sized chunks; on a hit the new request's table points at
 * the cached block and that prefill is skipped; on a miss the chunk is
 * prefilled and its block registered; [GLOSSARY] §3.01: requests with one
 * system prompt read the same physical pages).  A chunk's key is a 64-bit hash
 * of its block_size token ids chained onto the previous chunk's key, so a key
 * names a whole prefix; an entry also keeps its chunk's tokens and its
 * parent's key and a lookup matches only when both agree, so a hash collision
 * can never alias another prefix's keys and values.  Only full blocks are
 * cached.  The cache's hold on a block is not a reference: a cached block no
 * sequence holds is "evictable"; it counts as available, and when the free
 * list is empty a new block is taken from the least recently hit or
 * registered evictable block, whose entry is dropped.  A cached block is never
 * written again: appends write only into a sequence's partially filled last
 * block. */

/* New sequence for a prompt of n_tokens token ids: its leading full chunks
 * that are cached are mapped onto the cached blocks (each gains a reference),
 * up to the first chunk that misses.  *n_cached_out = tokens covered (a
 * multiple of block_size, possibly n_tokens); the sequence's length is that
 * count, and the caller appends and prefills the rest.  Takes no free block. */
pkv_status pkv_seq_create_cached(pkv_pool* pool, const int32_t* tokens, int32_t n_tokens,
                                 int32_t* seq_out, int32_t* n_cached_out);
/* Register the filled full blocks of a sequence whose first n_tokens token
 * ids are `tokens` (call after their keys and values are written).  Chunks
 * already cached for the same prefix are kept; registration stops at a chunk
 * whose key is owned by a different prefix or whose block is already cached
 * for a different chunk.  Chunks beyond the sequence's length are ignored. */
pkv_status pkv_seq_cache_prefix(pkv_pool* pool, int32_t seq, const int32_t* tokens,
                                int32_t n_tokens);
/* Counters: chunks that hit and missed in pkv_seq_create_cached so far, and
 * the cached and evictable blocks now.  Any output pointer may be NULL. */
pkv_status pkv_prefix_cache_stats(const pkv_pool* pool, int64_t* hit_blocks,
                                  int64_t* miss_blocks, int32_t* cached_blocks,
                                  int32_t* evictable_blocks);
/* Drop every entry; evictable blocks go to the free list in LRU order. */
void pkv_prefix_cache_clear(pkv_pool* pool);

/* ------------------------------------------------------------------- swap
 *
 * Page-granular eviction ([KV-SLOW] "Cómo PagedAttention soluciona esto":
 * when the cache is full, small pages move to CPU memory rather than whole
 * sequences; [GLOSSARY] glossary entry on KV-cache offloading: the cache is
 * moved temporarily from GPU memory to system RAM).  The pool keeps a swap
 * space of host slots, each holding one block (every KV head, K and V, in the
 * pool's tile layout).  A sequence's blocks can be swapped out a run at a
 * time; a sequence with swapped blocks cannot be decoded, appended to,
 * forked or registered in the prefix cache until pkv_seq_swap_in brings them
 * all back (into whatever device blocks are free).  Its block table shows -1
 * for a swapped block. */

/* Size the swap space: num_host_blocks host slots, handed out in ascending
 * order.  PKV_ERR_INVALID_ARG while any slot is in use. */
pkv_status pkv_pool_set_swap_space(pkv_pool* pool, int32_t num_host_blocks);
/* Free host slots; -1 for a bad handle. */
int32_t pkv_pool_num_free_host(const pkv_pool* pool);
/* Blocks of a sequence now in host slots; -1 for an unknown id. */
int32_t pkv_seq_num_swapped(const pkv_pool* pool, int32_t seq);
/* Move logical blocks [first_block, first_block + n_blocks) of a sequence to
 * host slots.  Each must be on the device and held by this sequence alone
 * (PKV_ERR_REFCOUNT otherwise: a shared page stays for its other holders); a
 * block's prefix-cache entry is dropped.  The device blocks return to the
 * free list.  pairs_out: host int32 [n_blocks][2] (device block, host slot),
 * in logical order, for pkv_swap_blocks(to_host = 1) -- which must run
 * before the freed blocks are written again.  All or nothing:
 * PKV_ERR_NO_FREE_BLOCKS when the swap space is short, nothing changed. */
pkv_status pkv_seq_swap_out(pkv_pool* pool, int32_t seq, int32_t first_block, int32_t n_blocks,
                            int32_t* pairs_out);
/* Bring every swapped block of a sequence back into device blocks taken as
 * an append takes them (free list, then least recently used cache-only
 * blocks).  *n_out = number of such blocks always; pairs_out: host int32
 * [cap][2] (host slot, device block), for pkv_swap_blocks(to_host = 0).
 * PKV_ERR_INVALID_ARG if cap is short, PKV_ERR_NO_FREE_BLOCKS if the device
 * is: nothing changed in either case. */
pkv_status pkv_seq_swap_in(pkv_pool* pool, int32_t seq, int32_t* pairs_out, int32_t cap,
                           int32_t* n_out);

/* Copy blocks between the device pools and the host swap space.
 *   host_k, host_v  pinned host memory the device can address (hipHostMalloc,
 *                 or a pinned torch tensor), [num_host_blocks][num_kv_heads]
 *                 [16 * 128] elements each, the pool's tile layout;
 *   pairs         device int32 [num_pairs][2]: (device block, host slot) when
 *                 to_host = 1, (host slot, device block) when to_host = 0;
 *                 pairs with an id out of range are skipped.
 * Host buffers the runtime does not know as pinned, device-reachable memory
 * (hipHostGetDevicePointer fails) give PKV_ERR_INVALID_ARG before any launch.
 * Bound by the host link, not HBM.  Asynchronous on `stream`: the host copy
 * is complete once the stream is. */
pkv_status pkv_swap_blocks(void* k_pool, void* v_pool, void* host_k, void* host_v,
                           int32_t num_host_blocks, const pkv_cache_layout* layout,
                           const int32_t* pairs, int32_t num_pairs, int32_t to_host,
                           void* stream);

/* ------------------------------------------------------ memory ceilings */

/* Reads that bound the decode from above, for measurement.  [PRIMER-8] §8.1
 * compares a paged kernel with one reading a contiguous slab; these two give
 * both sides of that comparison without attention arithmetic.
 * pkv_hbm_read_probe streams `bytes` (a multiple of 16) of device memory at
 * `buf` (16-byte aligned) once with 16-byte non-temporal lane loads: each of
 * `workgroups` workgroups (0 = 2048) reads its own contiguous slab in 32 KiB
 * steps.
 * pkv_tile_gather_probe reads every K and V tile of every sequence through
 * its block table, as the decode kernel does (same loads, same cache policy;
 * arguments as in pkv_paged_attention_decode; ids outside the pool read
 * nothing).  Both fold what they read into one word per lane and store it to
 * sink[0] (device uint32) only if it equals `key`, so nothing measurable is
 * written.
 * pkv_hbm_mix_probe is the ceiling for the cache write (§4 of [FP8-128K]
 * moves fp16 rows into the cache): it reads `reads_per_write` (1 or 2)
 * source planes of `dst_bytes` each, laid one after the other at `src`, and
 * writes their XOR, `dst_bytes` (a multiple of 16), to `dst`, every load and
 * store non-temporal, each of `workgroups` (0 = 2048) workgroups streaming
 * its own slab.  Both buffers 16-byte aligned device memory, owned by the
 * caller; they must not overlap.  All three are asynchronous on `stream`;
 * bad arguments return PKV_ERR_INVALID_ARG before any launch. */
pkv_status pkv_hbm_read_probe(const void* buf, uint64_t bytes, int32_t workgroups,
                              uint32_t* sink, uint32_t key, void* stream);
pkv_status pkv_hbm_mix_probe(const void* src, void* dst, uint64_t dst_bytes,
                             int32_t reads_per_write, int32_t workgroups, void* stream);
pkv_status pkv_tile_gather_probe(const void* k_pool, const void* v_pool,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t max_context_len, const pkv_cache_layout* layout,
                                 uint32_t* sink, uint32_t key, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
