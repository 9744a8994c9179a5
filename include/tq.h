/*
 * libtq — TurboQuant KV-cache compression, compressed-KV decode attention and
 * inner-product search for AMD MI355X (gfx950).
 *
 * The method (riverfrot "TurboQuant" post, sections 4.1-4.3; uiyeonassociation
 * "TurboQuant" post, two-stage compression): a vector x is stored as its norm
 * n = |x|, the Lloyd-Max codes of the rotated unit vector x~ = R (x / n), and —
 * for the inner-product ("PROD") variant — the norm rho of the rotated
 * residual r~ = x~ - c[idx] plus the signs of S r~ (the QJL sketch). The
 * inner product with an unquantised y is then estimated without bias as
 *
 *     <y, x>  ~  n * ( <R y, c[idx]> + gamma * rho * <S R y, 2 z - 1> ),
 *     gamma = sqrt(pi / 2) / d.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All device buffers are owned by the caller; libtq never allocates device
 *    memory. Its one piece of mutable device state is the fixed scratch
 *    array of tq_decode_attn_noalloc (one per GPU); every other call keeps
 *    no mutable global state and is thread-safe.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every
 *    device entry point only enqueues work on it and returns; nothing
 *    synchronises.
 *  - Validation happens before any device call; on error nothing is written
 *    and the return value is negative (see tq_status). No C++ exception
 *    crosses the ABI.
 *  - Device base pointers must be 16-byte aligned (TQ_ERR_MISALIGNED).
 *  - Inputs must be finite; this is a precondition, not checked on the GPU.
 *    Norms must stay below 65504 (they are stored as IEEE half).
 *
 * Packed layouts (this library's own; the pages only require that no
 * per-block scale or zero-point be stored, riverfrot section 4.2). A code of
 * B bits is stored as B bit-planes (plane p = bit p of the code, LSB first);
 * PROD adds one sign plane (p = B, bit = 1 when (S r~)_j >= 0). P = B + [PROD].
 *  - TQ_LAYOUT_KEYS (coordinate-contiguous; keys and search databases):
 *    tiles of 16 vectors; uint32 word index ((tile * d/32 + g) * 16 + t) * P + p
 *    holds coordinates 32 g .. 32 g + 31 (bit i = coordinate 32 g + i) of
 *    vector 16 tile + t.
 *  - TQ_LAYOUT_VALUES (token-contiguous; values): tiles of 32 vectors in
 *    blocks of two (64 vectors); word index (tile * d + j) * P + p holds
 *    coordinate j of 32 vectors of its block. Vector 64 k + t (t = 0..63)
 *    lies in tile 2 k + (t / 8) mod 2 at bit 16 (t mod 2) + 4 (t / 16) +
 *    (t mod 8) / 2: bits 4 i + r (i = 0..7) of tile 2 k + s hold vectors
 *    64 k + 16 (i mod 4) + 8 s + 2 r + i / 4. The packed size rounds n up to
 *    a whole block.
 *  Vectors past n in the last tile (block) are all-zero bits. Norms are
 *  separate arrays of IEEE half (uint16 bits), one per vector.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = -1,  /* null pointer, negative size, inconsistent shapes */
  TQ_ERR_UNSUPPORTED = -2,  /* d not a multiple of 32 or out of range, bits out of range */
  TQ_ERR_MISALIGNED = -3,   /* a device base pointer is not 16-byte aligned */
  TQ_ERR_NO_CONVERGE = -4,  /* Lloyd-Max did not converge within max_iter */
  TQ_ERR_HIP = -5,          /* a HIP launch failed */
  TQ_ERR_WORKSPACE = -6,    /* workspace missing or smaller than the size query says */
  TQ_ERR_SCRATCH = -7       /* the call needs more workspace than TQ_DECODE_SCRATCH_BYTES */
} tq_status;

typedef enum { TQ_MSE = 0, TQ_PROD = 1 } tq_variant;
typedef enum { TQ_F32 = 0, TQ_BF16 = 1 } tq_dtype;
typedef enum { TQ_LAYOUT_KEYS = 0, TQ_LAYOUT_VALUES = 1 } tq_layout;
/* Classes of tq_kv_bit_allocation. */
typedef enum { TQ_KV_UNIFORM = 0, TQ_KV_ASYMMETRIC = 1, TQ_KV_MIXED = 2 } tq_kv_alloc;

#define TQ_MAX_MSE_BITS 4
#define TQ_MAX_LEVELS 16
#define TQ_MAX_GROUPS 4
#define TQ_MAX_DIM 2048

/* One quantiser (riverfrot sections 4.1-4.3). The codebook is held by value
 * (ascending, 2^mse_bits centroids and 2^mse_bits - 1 thresholds; entries past
 * those are ignored); R and S are device pointers to d x d row-major fp32
 * matrices owned by the caller (R orthogonal, S i.i.d. N(0,1); S is NULL for
 * TQ_MSE). SR is optional (NULL from tq_quantizer_init): a device buffer
 * filled by tq_fold_qjl, with which decode forms S R q in one product. The
 * decode and search kernels require the mirror-symmetric codebook
 * tq_quantizer_init produces (c_i = -c_{L-1-i}). */
typedef struct {
  int d;             /* vector dimension: multiple of 32, 32..2048 */
  int mse_bits;      /* B: Lloyd-Max bits per coordinate, 1..4 */
  tq_variant variant;
  const float* R;
  const float* S;
  const float* SR;   /* optional: tq_fold_qjl output for this R and S */
  float centroids[TQ_MAX_LEVELS];
  float thresholds[TQ_MAX_LEVELS - 1];
} tq_quantizer;

/* One channel group of a compressed KV cache: channels
 * [ch_offset, ch_offset + q.d) of every head vector, quantised by q.
 * Sequence (b, kv_head) starts at vector (b * Hkv + kv_head) * seq_stride;
 * token t of it is vector (b * Hkv + kv_head) * seq_stride + t in `packed`
 * (layout TQ_LAYOUT_KEYS for keys, TQ_LAYOUT_VALUES for values), `norm` and
 * `rnorm`. seq_stride must be a multiple of 64. */
typedef struct {
  tq_quantizer q;
  int ch_offset;
  const void* packed;
  const uint16_t* norm;   /* half |x| per vector */
  const uint16_t* rnorm;  /* half rho per vector (PROD), NULL for MSE */
  int64_t seq_stride;
} tq_group;

/* A compressed K or V cache: 1..TQ_MAX_GROUPS groups tiling the head
 * channels 0..D-1 in order (config "outlier 32 channels at 3 bits, the rest at
 * 2 bits" is two groups after the caller permutes the outlier channels first). */
typedef struct {
  int n_groups;
  tq_group g[TQ_MAX_GROUPS];
} tq_kv_desc;

/* ---------------------------------------------------------------- host only */

/* Lloyd-Max codebook for the marginal of one coordinate of a uniformly
 * random unit vector in R^d, f_d(x) ~ (1 - x^2)^((d-3)/2) on [-1, 1]
 * (riverfrot section 4.1: rotated coordinates follow one Beta-type law;
 * section 4.2: Lloyd-Max takes the density and 2^b levels and returns the
 * boundaries {t_i} and representatives {c_i}, computed once per (d, b)).
 * Writes 2^mse_bits ascending centroids and 2^mse_bits - 1 thresholds (the
 * midpoints), mirror-symmetric, and optionally the total squared error D of
 * a unit vector. max_iter = 0 selects the default (200000). Host pointers.
 * Errors: INVALID_ARG (null outputs), UNSUPPORTED (d < 3 or > 2048, bits
 * outside 1..4), NO_CONVERGE. */
int tq_build_codebook(int d, int mse_bits, double* centroids, double* thresholds,
                      double* mse_out, int max_iter);

/* Fill *q: d, bits, variant, the device pointers R and S (not dereferenced
 * here), and the fp32-rounded codebook of tq_build_codebook. */
int tq_quantizer_init(tq_quantizer* q, int d, int mse_bits, tq_variant variant,
                      const float* R, const float* S);

/* Bytes of the packed codes of n vectors in `layout`, including the padding
 * of the last tile: ceil(n / tile) * tile * P * d / 8. 0 on bad arguments. */
size_t tq_packed_bytes(int d, int mse_bits, tq_variant variant, tq_layout layout, int64_t n);

/* Key/value bit widths from the ratio r = key_norm / value_norm of typical
 * key and value norms (riverfrot section 4.5: a quantised vector's error
 * scales with its squared norm, so keys with much larger norms need more
 * bits). Host only. The section's rule: r < 10 -> TQ_KV_UNIFORM, 3-bit keys
 * and values; 10 <= r <= 60 -> TQ_KV_ASYMMETRIC, 4-bit keys and 2-bit
 * values; r > 100 -> TQ_KV_MIXED (per channel group, e.g. the outlier
 * split of tq_kv_desc groups), with 4 and 2 as the base widths. The section
 * leaves 60 < r <= 100 open; it is read as asymmetric. Widths are total bits
 * per channel (a 4-bit TurboQuant_prod key is 3 codebook bits + 1 sign).
 * Returns the class, or INVALID_ARG for a norm that is not finite and
 * positive or a null output (nothing is written then). */
int tq_kv_bit_allocation(double key_norm, double value_norm, int* key_bits, int* value_bits);

/* Human-readable text for a tq_status value. */
const char* tq_status_string(int status);

/* Bytes of the buffer tq_fold_qjl fills for dimension d: (d * d + 4) floats
 * (0 on a bad d). */
size_t tq_fold_bytes(int d);

/* Precompute the query side of the QJL term (riverfrot section 4.3: the
 * query enters the sign estimator as S R q, q~ = R q being the rotated
 * query): SR[0 .. d*d) = S R (d x d row-major fp32) and SR[d*d] = the largest
 * Euclidean row norm of S R; SR[d*d+1 .. d*d+3] are zero. R and S are read on
 * `stream`, SR (tq_fold_bytes(d) bytes, device, caller-owned, 16-byte
 * aligned) is written on it. Store SR in tq_quantizer.SR: decode then forms
 * R q and S R q in one pass, bounding both operand ranges by the row norms
 * instead of by a second pass over the products. Errors: INVALID_ARG (not a
 * PROD quantiser, null pointers), UNSUPPORTED, MISALIGNED, HIP. */
int tq_fold_qjl(const tq_quantizer* q, float* SR, void* stream);

/* ------------------------------------------------------------ device calls */

/* Quantise n vectors x[i * x_stride_elems + 0 .. d-1] (fp32 or bf16, device)
 * (riverfrot sections 4.1-4.3, the online compression of each new K/V vector):
 *   n_i = |x_i|; x~ = R x_i / n_i; idx_j = #{k : x~_j >= t_k};
 *   PROD: r~ = x~ - c[idx], rho_i = |r~|, z_j = [(S r~)_j >= 0].
 * A zero vector stores n = 0, rho = 0, codes 2^B / 2 and signs 1.
 * Outputs (device): `packed` (tq_packed_bytes bytes, layout as above; it must
 * start at a tile boundary of the cache it belongs to), `norm` [n] half,
 * `rnorm` [n] half (PROD only; NULL for MSE). TQ_LAYOUT_VALUES needs d <= 256.
 * Contractions accumulate in fp32 (products of bf16 high/low parts on the
 * matrix cores, about 2^-17 of the terms' magnitudes). PROD keys of d > 128
 * run in batches of 65536 vectors through a device workspace of
 * 65536 * (d + d / 32) floats that the library allocates on a call's first
 * use on a device (so that call may block and return TQ_ERR_HIP if the
 * allocation fails) and keeps until the process ends; such calls that
 * overlap on one device (different streams or threads) race on it. */
int tq_quantize_kv(const tq_quantizer* q, tq_layout layout, tq_dtype in_dtype,
                   const void* x, int64_t n, int64_t x_stride_elems, void* packed,
                   uint16_t* norm, uint16_t* rnorm, void* stream);

/* Append: quantise n vectors exactly as tq_quantize_kv does (riverfrot
 * sections 4.1-4.3; the pages quantise each generated token online, section
 * 2.4) and write vector i into row rows[i] of an existing cache instead of
 * row i: one new token per (sequence, KV head) during decoding, or the rows
 * of a paged block. `rows` (device, int64 [n], 8-byte aligned) holds
 * distinct rows in [0, cache_rows); a row outside that range is skipped, and
 * two equal rows leave that row with an unspecified mix of the two vectors'
 * bits and norms. `packed`, `norm` and `rnorm`
 * are the cache's own arrays over its cache_rows rows (packed holds
 * tq_packed_bytes(d, bits, variant, layout, cache_rows) bytes and starts at
 * a tile boundary). A key row owns its words and is overwritten whole; a
 * value row owns one bit of each word of its tile, and only those
 * bits change (set or cleared atomically), so appends into rows that share a
 * tile may run in one call. Other rows are left as they are. Errors as for
 * tq_quantize_kv, plus INVALID_ARG for cache_rows <= 0 or a null `rows`
 * with n > 0. */
int tq_append_kv(const tq_quantizer* q, tq_layout layout, tq_dtype in_dtype,
                 const void* x, int64_t n, int64_t x_stride_elems, const int64_t* rows,
                 int64_t cache_rows, void* packed, uint16_t* norm, uint16_t* rnorm,
                 void* stream);

/* tq_append_kv for a key cache (TQ_LAYOUT_KEYS) and a value cache
 * (TQ_LAYOUT_VALUES) in one launch: row rows[i] of both caches receives
 * key xk[i] and value xv[i] (each quantised by its own quantiser, exactly as
 * tq_append_kv would). For a decoding step that appends one token per
 * (sequence, KV head) to both caches; the two caches share `rows` and
 * cache_rows. Errors as for tq_append_kv, for either half. */
int tq_append_kv_pair(const tq_quantizer* qk, const tq_quantizer* qv, tq_dtype in_dtype,
                      const void* xk, const void* xv, int64_t n, int64_t xk_stride_elems,
                      int64_t xv_stride_elems, const int64_t* rows, int64_t cache_rows,
                      void* kpacked, uint16_t* knorm, uint16_t* krnorm, void* vpacked,
                      uint16_t* vnorm, uint16_t* vrnorm, void* stream);

/* Workspace bytes tq_decode_attn needs for these shapes (0 on bad arguments). */
size_t tq_decode_workspace_bytes(const tq_kv_desc* k, const tq_kv_desc* v, int B, int Hq,
                                 int Hkv, int T_max);

/* Decode attention straight from the compressed cache (riverfrot sections
 * 2.2-2.3: the new query attends to every cached token, softmax(q K^T /
 * sqrt(d)) V; section 4.3: scores from the unbiased estimator with the query
 * unquantised; GQA: query head h reads KV head h / (Hq / Hkv)).
 *   q        [B, Hq, D] fp32 or bf16, D = total key channels (<= 256)
 *   seq_lens [B] int32 device, or NULL for T_max everywhere (0 <= len <= T_max)
 *   scale    logit scale, normally 1/sqrt(D)
 *   out      [B, Hq, Dv] fp32: sum_t softmax_t(scale * s_t) * v^_t with
 *            v^_t = n_t R_v^T c_v[idx_t] per value group (zeros if len = 0)
 *   scores_out NULL or [B, Hq, T_max] fp32: the raw estimates s_t (t < len)
 *   ws, ws_bytes: device workspace of at least tq_decode_workspace_bytes.
 * Keys must use TQ_LAYOUT_KEYS, values TQ_LAYOUT_VALUES and TQ_MSE.
 * Accumulation is fp32 (operands as digits: four fp6 digits per 32-channel
 * block for the query, three fp8 digits for the softmax weights); measured
 * against an fp64 evaluation of the same codes, outputs are within 4.9e-4
 * (normwise, per query head) and scores within 3.4e-4 of the row's largest
 * score across the test cases, inside the 2e-3 acceptance bound. Each
 * 32-channel block of a query head is scaled by its own power of two, so the
 * bound holds for any mix of magnitudes down to blocks whose largest entry is
 * about 2^-110 (below that the trailing digits, and then the block, drop to
 * zero). */
int tq_decode_attn(const tq_kv_desc* k, const tq_kv_desc* v, const void* q, tq_dtype q_dtype,
                   int B, int Hq, int Hkv, int T_max, const int32_t* seq_lens, float scale,
                   float* out, float* scores_out, void* ws, size_t ws_bytes, void* stream);

/* One decode step (riverfrot sections 2.2-2.3: the generated token's key
 * and value join the cache, compressed online as in sections 4.1-4.3, and
 * the new query attends to every cached token, this one included): the new
 * key and value rows of every (sequence, KV head) are quantised into the
 * cache, then the attention of tq_decode_attn runs over lengths seq_lens.
 * For head_dim-128 layouts whose PROD key groups carry S R (tq_fold_qjl) the
 * appends run inside the decode's query-transform launch, so the step takes
 * the launches of tq_decode_attn alone; otherwise they take launches of
 * their own before it.
 *   k_new    [B, Hkv, D] new key rows, v_new [B, Hkv, Dv] new value rows
 *            (fp32 or bf16 as kv_dtype, contiguous, 16-byte aligned)
 *   seq_lens [B] int32 device, required: lengths after the append. The new
 *            row of (b, g) goes to row (b Hkv + g) seq_stride + seq_lens[b] - 1
 *            of every group (the row tq_append_kv would write); a sequence
 *            with seq_lens[b] = 0 appends nothing.
 * The cache the descriptors point at is written (their const pointers are
 * the decode's view of it). Other arguments, the workspace
 * (tq_decode_workspace_bytes) and errors as for tq_decode_attn. */
int tq_decode_step(const tq_kv_desc* k, const tq_kv_desc* v, const void* k_new, const void* v_new,
                   tq_dtype kv_dtype, const void* q, tq_dtype q_dtype, int B, int Hq, int Hkv, int T_max,
                   const int32_t* seq_lens, float scale, float* out, float* scores_out, void* ws,
                   size_t ws_bytes, void* stream);

/* Size of the scratch array tq_decode_attn_noalloc uses as its workspace. */
#define TQ_DECODE_SCRATCH_BYTES ((size_t)16 << 20)

/* tq_decode_attn for callers that cannot allocate device memory (code under
 * stream capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same attention, arguments, results and errors, with no workspace
 * argument. Its workspace is a fixed array of TQ_DECODE_SCRATCH_BYTES in
 * every GPU's memory, part of the library's code object, held from the load
 * until the process ends; the call allocates nothing.
 *   - A call whose tq_decode_workspace_bytes exceeds TQ_DECODE_SCRATCH_BYTES
 *     returns TQ_ERR_SCRATCH before any device work (use tq_decode_attn).
 *   - All calls on one GPU share its array. Calls in one stream are ordered;
 *     calls that may overlap in time on one GPU (other streams, other host
 *     threads) race on it and must be serialised by the caller.
 *   - Nothing in the array needs clearing: every call writes each word of
 *     it that it reads, so leftovers of the last call do not matter.
 *   - TQ_ERR_HIP if the array's device address cannot be obtained (it is
 *     looked up once per device, on the first call with that device
 *     current). */
int tq_decode_attn_noalloc(const tq_kv_desc* k, const tq_kv_desc* v, const void* q, tq_dtype q_dtype,
                           int B, int Hq, int Hkv, int T_max, const int32_t* seq_lens, float scale,
                           float* out, float* scores_out, void* stream);

/* Workspace bytes tq_decode_attn_paged needs (0 on bad arguments). */
size_t tq_decode_paged_workspace_bytes(const tq_kv_desc* k, const tq_kv_desc* v, int B, int Hq,
                                       int Hkv, int T_max, int block_tokens);

/* tq_decode_attn over a paged cache (the same attention, riverfrot sections
 * 2.2-2.3 and 4.3): the cache of every group is a pool of num_blocks blocks
 * of block_tokens rows per KV head, and token t of sequence b, KV head g is
 * row (block_table[b * max_blocks + t / block_tokens] * Hkv + g) *
 * block_tokens + t % block_tokens of the group's packed, norm and rnorm
 * arrays (each group's seq_stride must equal block_tokens). block_table:
 * device int32 [B, max_blocks], with max_blocks * block_tokens >= T_max;
 * entries past a sequence's last block are not read for its scores, and a
 * block id outside [0, num_blocks) reads as an empty block (no fault; its
 * tokens are then not the cache's). block_tokens: a multiple of 256 (the
 * decode kernel's chunk), so that each workgroup's split lies in one block.
 * Head size 128 in the layouts the matrix-core decode compiles (otherwise
 * UNSUPPORTED). Other arguments and errors as for tq_decode_attn, with the
 * workspace sized by tq_decode_paged_workspace_bytes. */
int tq_decode_attn_paged(const tq_kv_desc* k, const tq_kv_desc* v, const void* q, tq_dtype q_dtype,
                         int B, int Hq, int Hkv, int T_max, const int32_t* seq_lens,
                         const int32_t* block_table, int max_blocks, int block_tokens,
                         int64_t num_blocks, float scale, float* out, float* scores_out, void* ws,
                         size_t ws_bytes, void* stream);

/* Workspace bytes tq_search_topk needs. */
size_t tq_search_workspace_bytes(const tq_group* db, int64_t N, int Q, int k);

/* Top-k database vectors by estimated inner product with each query
 * (uiyeonassociation post: TurboQuant codes used for vector search).
 *   db        one group, TQ_LAYOUT_KEYS, seq_stride ignored (vectors
 *             0..N-1, 1 <= N < 2^29)
 *   queries   [Q, d] fp32 device
 *   out_idx   [Q, k] int64, out_score [Q, k] fp32: descending score, equal
 *             scores in ascending index order. 1 <= k <= 64, k <= N.
 * Scores are the same estimator as decode, accumulated in fp32. */
int tq_search_topk(const tq_group* db, int64_t N, const float* queries, int Q, int k,
                   int64_t* out_idx, float* out_score, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
