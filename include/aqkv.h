/*
 * aqkv.h -- compressed KV-cache key quantisation and decode attention on
 * packed bits, for AMD Instinct MI355X (gfx950).  C ABI of libaqkv.so.
 *
 * The method is the one the TurboQuant article (kwkr.cn, "TurboQuant:
 * near-optimal KV cache quantization for LLM inference (3-bit keys, 2-bit
 * values)") describes, plus the pure-QJL keys with per-layer sketch size of
 * the A-QJL article (zingnex.cn, "A-QJL: adaptive layer-wise KV cache
 * compression"):
 *
 *   keys    (TurboQuant §二, §五): n = ||x||; y = Pi (x / n); idx_j = number of
 *           decision boundaries below y_j (w = b - 1 Lloyd-Max bits per
 *           coordinate); r = x - n Pi^T c[idx]; signs of S r (one bit per
 *           sketch row); gamma = ||r||.  w = 0 is pure QJL (A-QJL, section
 *           "QJL"): signs of S x, only n stored.
 *   values  (TurboQuant component table, §七): per token, per group of
 *           `value_group` contiguous channels, min-max quantisation to
 *           `value_bits` bits.
 *   decode  (TurboQuant §五, §六): the query is rotated (Pi q) and sketched
 *           (S q) once; the score of cached token t is
 *             n_t <Pi q, c[idx_t]> + sqrt(pi/2)/m * gamma_t * <S q, 2 bits_t - 1>
 *           (an unbiased estimate of <q, k_t>), computed on the packed bits;
 *           softmax(score * softmax_scale) weights the dequantised values
 *           code * scale + min.  No fp key is ever materialised.
 *
 * Conventions for every call
 * --------------------------
 * - Pointers marked (dev) are device memory on the current HIP device, owned
 *   by the caller; they must stay valid until the enqueued work finishes.
 *   Pointers marked (host) are host memory.  The library allocates nothing
 *   and keeps no state between calls.
 * - Compute calls only enqueue work on `stream` (a hipStream_t; NULL = the
 *   default stream) and never synchronise.  Calls on the same stream are
 *   ordered; concurrent calls that write the same cache rows race.
 * - Arguments are validated on the host before anything is enqueued.  On an
 *   error the call returns a negative aqkv_status and writes nothing.  A
 *   launch failure reported by the HIP runtime returns AQKV_ERR_HIP.  Nothing
 *   prints, aborts or throws across this interface.
 *
 * Cache layout: block records.  The tokens of a slot (slot s = b * H + h of
 * the K/V view) are grouped in blocks of 32 (capacity is a multiple of 32);
 * block c of slot s is one contiguous record at byte
 * (s * capacity / 32 + c) * block_bytes of the cache buffer, so a decoder
 * streams each 32-token block with a few large contiguous reads.  A record
 * holds six fields one after the other, each 32 token rows of its own row
 * format (offsets and sizes from aqkv_cache_layout):
 *   bit rows   32-bit little-endian words of 32 consecutive elements; element
 *              j = 4 i + k of a word (i in 0..7, k in 0..3) is bit 8 k + i.
 *   key_codes  w * d / 8 bytes per row: w bit rows of d bits; row p holds bit
 *              p of every coordinate's index.  (absent when w == 0.)
 *   key_signs  m / 8 bytes per row: one bit row, bit 1 = non-negative
 *              projection.
 *   key_norm   ||x|| per row: fp32, or IEEE half when side_f16 is set.
 *   key_rnorm  ||r|| per row (absent when w == 0): fp32, or half as key_norm.
 *   val_codes  d * value_bits / 8 bytes per row; the 32 rows of a record are
 *              one code block in which channel 32 g + 16 h + n (group g, half
 *              h, column n) of token 4 i + r (r in 0..3, i in 0..7) is at
 *                value_bits 2: word (16 g + n) * 4 + r, bits 8 h + 16 (i & 1) + 2 (i >> 1);
 *                value_bits 4: word ((16 g + n) * 4 + r) * 2 + h, bits 16 (i & 1) + 4 (i >> 1).
 *   val_side   scale and min of every value group, 2 * e * d / value_group
 *              bytes per row (e = 4 for fp32, 2 for half when side_f16 is
 *              set), stored group-major in the record so that one 4e-byte
 *              read returns what a decoder lane needs: the scale (j = 0) and
 *              min (j = 1) of group g for token t = 8 a + 4 h + b (b in 0..3,
 *              h in 0..1) is element ((g * 16 + 4 a + b) * 2 + h) * 2 + j of
 *              the field.
 * Side information in half precision (side_f16 = 1; the bytes-for-precision
 * knob beside the TurboQuant article's head_dim 256 compression figure, §一
 * Paper Validation table): every code (index, sign, value code) is decided
 * exactly as with fp32 side information; only the stored n, gamma, scale and
 * min are rounded, from their fp32 values, to the nearest half (ties to even),
 * finite values beyond the half range saturating to +-65504, and every
 * decoder reads back those halves.  At d = 256, 3-bit keys and 2-bit values a
 * row then takes 196 bytes instead of 232 (5.22x against bf16 K and V rather
 * than 4.41x).
 * The cache buffer must be 16-byte aligned (every block_bytes is a multiple
 * of 16).
 */
#ifndef AQKV_H
#define AQKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AQKV_OK = 0,
  AQKV_ERR_NULL = -1,        /* a required pointer is NULL */
  AQKV_ERR_SHAPE = -2,       /* unsupported or inconsistent sizes / bit widths */
  AQKV_ERR_ALIGN = -3,       /* a pointer or stride breaks the alignment rules */
  AQKV_ERR_CAPACITY = -4,    /* token_offset + tokens exceeds the cache capacity */
  AQKV_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required */
  AQKV_ERR_DTYPE = -6,       /* unknown element type */
  AQKV_ERR_HIP = -7,         /* the HIP runtime reported an error */
  AQKV_ERR_UNSUPPORTED = -8, /* valid request the library does not implement */
  AQKV_ERR_SCRATCH = -9      /* needs more than the library's static scratch (allocation-free call) */
} aqkv_status;

typedef enum { AQKV_FP32 = 0, AQKV_BF16 = 1 } aqkv_dtype;

/* Codec configuration, fixed per cache. */
typedef struct {
  int32_t head_dim;    /* d: 64, 128 or 256 */
  int32_t mse_bits;    /* w = b - 1 Lloyd-Max bits per coordinate, 0..3 (0 = pure QJL) */
  int32_t sketch_dim;  /* m: QJL sketch rows, multiple of 64, 64..1024 (m = d for TurboQuant keys) */
  int32_t value_bits;  /* 2 or 4 */
  int32_t value_group; /* channels per value group: 32 */
  int32_t side_f16;    /* 0: n, gamma, value scale and min stored as fp32; 1: as IEEE half */
} aqkv_config;

/* Per-layer parameters (TurboQuant §二: Pi from a QR decomposition and S
 * Gaussian, one seed per layer; Lloyd-Max codebook computed offline). */
typedef struct {
  const float *rotation;   /* (dev) Pi [d][d] row-major fp32, y = Pi x; required iff mse_bits > 0 */
  const float *sketch;     /* (dev) S [m][d] row-major fp32, z = S r */
  const float *centroids;  /* (dev) [2^w] ascending fp32; required iff mse_bits > 0 */
  const float *boundaries; /* (dev) [2^w - 1] ascending fp32; required iff mse_bits > 0 */
} aqkv_layer;

/* The compressed cache: n_slots * capacity / 32 block records (layout above). */
typedef struct {
  uint8_t *blocks;   /* (dev) the records, 16-byte aligned */
  int64_t n_slots;   /* batch * kv heads */
  int64_t capacity;  /* token rows per slot, a multiple of 32 */
} aqkv_cache;

/* A strided 4-D K or V tensor [batch][heads][tokens][d] in device memory.
 * Element (b, h, t, j) is at data + (b*batch_stride + h*head_stride +
 * t*token_stride + j) elements: channels are contiguous.  Strides must be
 * multiples of 8 elements. */
typedef struct {
  const void *data;   /* (dev) */
  aqkv_dtype dtype;
  int64_t batch, heads, tokens;
  int64_t batch_stride, head_stride, token_stride;
} aqkv_kv_view;

/* One 64-bit number per cache field. */
typedef struct {
  int64_t key_codes, key_signs, key_norm, key_rnorm, val_codes, val_side;
} aqkv_fields;

/* Block-record geometry for a configuration. */
typedef struct {
  aqkv_fields row_bytes;  /* bytes per token row of each field (0 = absent) */
  aqkv_fields offset;     /* byte offset of each field inside a record */
  int64_t block_bytes;    /* bytes of one 32-token record = 32 * sum(row_bytes) */
} aqkv_layout;

/* ---------------------------------------------------------------- host only */

/* Human-readable name of a status code (static string). */
const char *aqkv_status_string(aqkv_status status);

/* Checks a configuration and reports the block-record geometry (out may be
 * NULL to only validate).  AQKV_ERR_SHAPE for unsupported head_dim /
 * mse_bits / sketch_dim / value_bits / value_group / side_f16 (0 or 1).  A cache of n_slots x
 * capacity tokens takes n_slots * capacity / 32 * block_bytes bytes. */
aqkv_status aqkv_cache_layout(const aqkv_config *cfg, aqkv_layout *out);

/* Lloyd-Max codebook for one coordinate of a uniformly random unit vector in
 * R^head_dim (TurboQuant §二: the rotated coordinates share one scaled-Beta
 * law; the quantiser is its continuous 1-D k-means).  Computed on the host
 * in double precision; writes 2^bits ascending centroids and the 2^bits - 1
 * midpoint boundaries, both rounded to fp32.  (host) outputs.
 * bits in 1..4, head_dim in 3..4096. */
aqkv_status aqkv_build_codebook(int32_t head_dim, int32_t bits, float *centroids, float *boundaries);

/* Random orthogonal rotation from a Gaussian matrix (TurboQuant §二: a QR
 * decomposition): Householder QR of gaussian [d][d] (host, row-major
 * double), Pi = Q diag(sign(diag R)), written row-major fp32 to rotation
 * (host).  d in 1..4096. */
aqkv_status aqkv_build_rotation(int32_t d, const double *gaussian, float *rotation);

/* Randomised Hadamard rotation (NexusQuant article, stage 4, the Hadamard
 * rotation: a Hadamard matrix spreads every coordinate's energy over all d,
 * removing outliers): Pi = H diag(s) / sqrt(d), H Sylvester's Hadamard matrix
 * (H_ij = (-1)^popcount(i & j)), s_j = +1 where gaussian[j] >= 0 (the first
 * row of the layer's d x d Gaussian draw, host double), else -1; written
 * row-major fp32 to rotation (host).  d a power of two up to 4096.  A drop-in
 * replacement for aqkv_build_rotation's output: the key quantiser notices that
 * every entry has one magnitude and multiplies by +-1 operands, one matrix
 * pass instead of two. */
aqkv_status aqkv_build_hadamard_rotation(int32_t d, const double *gaussian, float *rotation);

/* Workspace bytes aqkv_quantize_keys needs for this configuration. */
size_t aqkv_quantize_keys_workspace_bytes(const aqkv_config *cfg);

/* Workspace bytes aqkv_decode_attention needs for these sizes. */
size_t aqkv_decode_workspace_bytes(const aqkv_config *cfg, int32_t batch, int32_t n_q_heads,
                                   int32_t n_kv_heads, int64_t context_len);

/* -------------------------------------------------------------- GPU compute */

/* Key quantisation (TurboQuant §二 three-stage pipeline; §五 quantize() ->
 * MSE indices, QJL sign bytes, residual norm, original norm; A-QJL pure QJL
 * when mse_bits == 0).  Quantises tokens [0, k->tokens) of every slot of k
 * into cache rows [token_offset, token_offset + k->tokens) (chunked append,
 * TurboQuant §六 CompressedKVStore).  k->batch * k->heads must equal
 * cache->n_slots; the key element type is fp32 or bf16.  Writes key_codes,
 * key_signs, key_norm and key_rnorm; workspace is scratch of at least
 * aqkv_quantize_keys_workspace_bytes(cfg) bytes (dev, 256-byte aligned).
 * A zero key stores n = 0, gamma = 0, the index of y = 0 and all sign bits 1. */
aqkv_status aqkv_quantize_keys(const aqkv_config *cfg, const aqkv_layer *layer,
                               const aqkv_kv_view *k, int64_t token_offset,
                               const aqkv_cache *cache, void *workspace, size_t workspace_bytes,
                               void *stream);

/* The per-layer half of aqkv_quantize_keys, for callers that quantise many
 * chunks with one layer (a decode loop appending one token per step): writes
 * into workspace (dev, 256-byte aligned, aqkv_quantize_keys_workspace_bytes
 * bytes) the matrix-core operands built from layer->rotation and
 * layer->sketch (the product S Pi^T included).  The workspace then stays valid
 * for aqkv_quantize_keys_prepared with the same cfg for as long as the caller
 * leaves it and the layer's rotation and sketch unchanged. */
aqkv_status aqkv_prepare_key_operands(const aqkv_config *cfg, const aqkv_layer *layer, void *workspace,
                                      size_t workspace_bytes, void *stream);

/* aqkv_quantize_keys on a workspace prepared by aqkv_prepare_key_operands (same
 * cfg and layer): the same results, without the operand pass.  layer supplies
 * the codebook (centroids, boundaries); its rotation and sketch are not read.
 * The workspace is only read. */
aqkv_status aqkv_quantize_keys_prepared(const aqkv_config *cfg, const aqkv_layer *layer,
                                        const aqkv_kv_view *k, int64_t token_offset,
                                        const aqkv_cache *cache, const void *workspace,
                                        size_t workspace_bytes, void *stream);

/* Value quantisation (TurboQuant component table and §七: conventional
 * min-max grouped quantisation with bit packing).  Per token, per group of
 * value_group contiguous channels: min, scale = (max - min) / (2^vb - 1),
 * code = clamp(rint((v - min) / scale), 0, 2^vb - 1), all in IEEE fp32; code 0
 * when scale == 0.  Same view / offset rules as aqkv_quantize_keys; writes
 * val_codes and val_side. */
aqkv_status aqkv_quantize_values(const aqkv_config *cfg, const aqkv_kv_view *v, int64_t token_offset,
                                 const aqkv_cache *cache, void *stream);

/* Query preparation (TurboQuant §六: the query is rotated, q Pi^T, and
 * pre-sketched, q S^T, once per query).  q is [n_q][d] (dev, contiguous, fp32
 * or bf16); writes q_rot = Pi q [n_q][d] (dev fp32; may be NULL when
 * mse_bits == 0) and q_sketch = S q [n_q][m] (dev fp32). */
aqkv_status aqkv_prepare_query(const aqkv_config *cfg, const aqkv_layer *layer, const void *q,
                               aqkv_dtype dtype, int64_t n_q, float *q_rot, float *q_sketch,
                               void *stream);

/* Decode attention on the packed cache (TurboQuant §五 estimator, §六 fused
 * decode with online softmax).  For every batch b and query head hq (kv head
 * hq / (n_q_heads / n_kv_heads), slot b * n_kv_heads + that head) over
 * cache rows [0, context_len):
 *   score_t = n_t <q_rot, c[idx_t]> + sqrt(pi/2)/m gamma_t <q_sketch, 2 bits_t - 1>
 *   out     = sum_t softmax_t(score * softmax_scale) (code_t * scale_t + min_t)
 * q_rot [batch][n_q_heads][d] and q_sketch [batch][n_q_heads][m] come from
 * aqkv_prepare_query (dev fp32).  out is [batch][n_q_heads][d] (dev fp32).
 * scores, if not NULL, receives the unscaled estimates [batch][n_q_heads]
 * [context_len] (dev fp32).  context_len == 0 writes out = 0.  workspace
 * (dev, 256-byte aligned) must hold aqkv_decode_workspace_bytes(...) bytes.
 * cache->n_slots must equal batch * n_kv_heads and n_q_heads must be a
 * multiple of n_kv_heads. */
aqkv_status aqkv_decode_attention(const aqkv_config *cfg, const aqkv_layer *layer,
                                  const aqkv_cache *cache, int32_t batch, int32_t n_q_heads,
                                  int32_t n_kv_heads, int64_t context_len, const float *q_rot,
                                  const float *q_sketch, float softmax_scale, float *scores,
                                  float *out, void *workspace, size_t workspace_bytes, void *stream);

/* Decode attention over the compressed history and a recent-token window
 * (TurboQuant §六: the latest tokens are kept at full precision in a ring
 * buffer and only the older history goes through the compressed path; one
 * softmax covers both).  Cache rows [0, context_len) of each slot are scored
 * and weighted exactly as by aqkv_decode_attention; the n_window tokens of
 * k_window / v_window ([batch][n_kv_heads][n_window][d] views, fp32 or bf16,
 * both the same dtype and n_window, n_window <= 1024; the order of the tokens
 * does not matter, so a ring buffer is passed as it is) get the exact logit
 * <q, k> * softmax_scale (fp32 accumulation) and their own values.  q is the
 * unrotated query [batch][n_q_heads][d] (dev fp32, contiguous); q_rot and
 * q_sketch are its aqkv_prepare_query outputs.  scores, if not NULL, receives
 * the compressed rows' estimates only ([batch][n_q_heads][context_len]).
 * context_len == 0 (no history yet) attends the window alone; both empty
 * writes out = 0.  Same workspace size and other rules as
 * aqkv_decode_attention. */
aqkv_status aqkv_decode_attention_window(const aqkv_config *cfg, const aqkv_layer *layer,
                                         const aqkv_cache *cache, int32_t batch, int32_t n_q_heads,
                                         int32_t n_kv_heads, int64_t context_len, const float *q,
                                         const float *q_rot, const float *q_sketch,
                                         const aqkv_kv_view *k_window, const aqkv_kv_view *v_window,
                                         float softmax_scale, float *scores, float *out, void *workspace,
                                         size_t workspace_bytes, void *stream);

/* Workspace bytes aqkv_decode_attention_topk needs for these sizes (0 on bad
 * arguments). */
size_t aqkv_decode_topk_workspace_bytes(const aqkv_config *cfg, int32_t batch, int32_t n_q_heads,
                                        int32_t n_kv_heads, int64_t context_len, int64_t budget);

/* Decode attention over a query-aware selection of the cached tokens (QUOKA
 * article §1: pre-aggregation over the KV heads, cosine-similarity scoring,
 * dynamic top-K selection).  For every KV slot the query heads that share it
 * are reduced to one selection query, the sum of their unit vectors; every
 * cache row t in [0, context_len) is scored by cos_t = est_t / n_t (est_t the
 * estimator of <q_sel, k_t>, n_t the stored norm; 0 for a zero key), and the
 * min(budget, context_len) rows with the largest cos_t (ties to the lower
 * row) are chosen.  Each query head then attends those rows only, exactly as
 * aqkv_decode_attention attends all of them.  q is the unrotated query
 * [batch][n_q_heads][d] (dev fp32, contiguous); q_rot and q_sketch are its
 * aqkv_prepare_query outputs.  selected, if not NULL, receives the chosen rows
 * of every slot in increasing order ([batch * n_kv_heads][min(budget,
 * context_len)] int32, dev).  budget in 1..2^20; context_len at most
 * 2^31 - 2^20 rows (row indices are 32-bit), AQKV_ERR_UNSUPPORTED beyond.
 * workspace (dev, 256-byte aligned) must hold
 * aqkv_decode_topk_workspace_bytes(...) bytes.  Other rules as
 * aqkv_decode_attention. */
aqkv_status aqkv_decode_attention_topk(const aqkv_config *cfg, const aqkv_layer *layer,
                                       const aqkv_cache *cache, int32_t batch, int32_t n_q_heads,
                                       int32_t n_kv_heads, int64_t context_len, const float *q,
                                       const float *q_rot, const float *q_sketch, int64_t budget,
                                       float softmax_scale, int32_t *selected, float *out,
                                       void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes aqkv_decode_attention_topk_blocks needs for these sizes (0
 * on bad arguments). */
size_t aqkv_decode_topk_blocks_workspace_bytes(const aqkv_config *cfg, int32_t batch, int32_t n_q_heads,
                                               int32_t n_kv_heads, int64_t context_len, int64_t budget);

/* The same query-aware selection at the granularity of the cache's 32-row
 * block records (QUOKA article §2: the KV cache organised as contiguous
 * memory blocks; a reading, the article ranks keys, not blocks): a record
 * ranks by the largest cos_t of its rows below context_len, and the
 * nb = min(ceil(budget / 32), ceil(context_len / 32)) records with the largest
 * ranks (ties to the lower record) are chosen; each query head then attends
 * every row below context_len of the chosen records, exactly as
 * aqkv_decode_attention attends all rows.  Reading whole records keeps every
 * load a contiguous stream, where a row-level choice touches most of the
 * cache's bytes through its rows' shared block words.  selected, if not NULL,
 * receives the chosen records of every slot in increasing order
 * ([batch * n_kv_heads][nb] int32, dev).  Shapes the matrix-core decoder does
 * not cover (for one query head per slot and for n_q_heads / n_kv_heads)
 * return AQKV_ERR_UNSUPPORTED.  Other arguments and rules as
 * aqkv_decode_attention_topk, workspace of
 * aqkv_decode_topk_blocks_workspace_bytes(...) bytes. */
aqkv_status aqkv_decode_attention_topk_blocks(const aqkv_config *cfg, const aqkv_layer *layer,
                                              const aqkv_cache *cache, int32_t batch, int32_t n_q_heads,
                                              int32_t n_kv_heads, int64_t context_len, const float *q,
                                              const float *q_rot, const float *q_sketch, int64_t budget,
                                              float softmax_scale, int32_t *selected, float *out,
                                              void *workspace, size_t workspace_bytes, void *stream);

/* -------------------------------------------------- allocation-free variant */

/* For callers that cannot allocate device memory or hand over a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): aqkv_decode_attention with its split partials in a static
 * device scratch of the library instead of a caller workspace.  Same
 * arguments, results and rules as aqkv_decode_attention without workspace /
 * workspace_bytes; calls nothing that allocates.  The scratch holds
 * aqkv_decode_static_scratch_bytes() bytes (8 MiB) on every device the
 * library runs on, kept until the process ends; a call whose partials
 * (aqkv_decode_workspace_bytes for the same sizes) exceed it returns
 * AQKV_ERR_SCRATCH before enqueuing anything.  Every call on one device
 * shares that device's scratch, so calls that overlap on one device (on
 * different streams, or from several threads) race; calls ordered on one
 * stream do not.  The first call on a device looks up the device's copy of
 * the scratch (once per device; thread-safe). */
size_t aqkv_decode_static_scratch_bytes(void);
aqkv_status aqkv_decode_attention_noalloc(const aqkv_config *cfg, const aqkv_layer *layer,
                                          const aqkv_cache *cache, int32_t batch, int32_t n_q_heads,
                                          int32_t n_kv_heads, int64_t context_len, const float *q_rot,
                                          const float *q_sketch, float softmax_scale, float *scores,
                                          float *out, void *stream);

/* ------------------------------------------------------- measurement helper */

/* Reads `bytes` of device memory at `data` once, as a stream of non-temporal
 * 16-byte loads spread over the whole GPU: the practical ceiling of HBM reads
 * against which the decode's streaming rate is compared (no step of the
 * method).  Every lane folds what it read into one word and stores it to
 * *sink (dev, one uint32) only if that word is 0xFFFFFFFF: a dependency that
 * keeps every load without a store or atomic per block (either measurably
 * slows the stream), not a result.  data and bytes must be multiples of 16.
 * Enqueues on `stream` only. */
aqkv_status aqkv_read_stream(const void *data, size_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* AQKV_H */
