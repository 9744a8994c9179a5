// Interfaces between the C-ABI layer (tq_api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq.h"

namespace tqk {

// Tile sizes of the packed layouts (see tq.h).
constexpr int kKeysTile = 16;
constexpr int kValuesTile = 32;
constexpr int kValuesBlock = 64;  // two value tiles whose vectors interleave

// Value layout: vector t (0..63) of a 64-vector block sits in tile
// value_tile(t) of the block, at bit value_bit(t) of that tile's words;
// value_tok inverts the pair. Each fp4 register the decode's matrix cores
// expand from a word (bits 4 i + r, i = 0..7, for register r) then holds the
// vectors 16 (i mod 4) + 8 s + 2 r + i / 4 of tile s: for r = 0..3 and one
// i, two pairs of adjacent vectors per tile, so the decode's attention
// weights for four consecutive vectors land in the bytes one conversion
// writes.
__host__ __device__ constexpr int value_tile(int t) { return (t >> 3) & 1; }
__host__ __device__ constexpr int value_bit(int t) { return 16 * (t & 1) + 4 * (t >> 4) + ((t & 7) >> 1); }
__host__ __device__ constexpr int value_tok(int s, int b) { return 16 * ((b >> 2) & 3) + 8 * s + 2 * (b & 3) + (b >> 4); }

inline int planes_of(const tq_quantizer& q) { return q.mse_bits + (q.variant == TQ_PROD ? 1 : 0); }

// Compute units of the current device, queried once per device and kept
// (256, the MI355X count, when no device answers: host-only size queries).
int device_cus();
// Workgroups of `fn` (threads per workgroup) one compute unit holds at once,
// queried once per (device, kernel) and kept; 1 when the query fails.
int kernel_wgs_per_cu(const void* fn, int threads);

hipError_t launch_quantize(const tq_quantizer& q, tq_layout layout, tq_dtype dt, const void* x, int64_t n,
                           int64_t stride, void* packed, uint16_t* norm, uint16_t* rnorm, hipStream_t s,
                           const int64_t* rows = nullptr, int64_t cache_rows = 0);
// Keys (key layout) and values (value layout) of the same rows appended in one
// launch.
hipError_t launch_append_pair(const tq_quantizer& qk, const tq_quantizer& qv, tq_dtype dt, const void* xk,
                              const void* xv, int64_t n, int64_t k_stride, int64_t v_stride, const int64_t* rows,
                              int64_t cache_rows, void* kpacked, uint16_t* knorm, uint16_t* krnorm, void* vpacked,
                              uint16_t* vnorm, uint16_t* vrnorm, hipStream_t s);

// The new rows of a decode step (tq_decode_step): row b Hkv + g of k_new /
// v_new is the new token of sequence b, KV head g, and goes to cache row
// (b Hkv + g) seq_stride + seq_lens[b] - 1 of every channel group.
struct StepRows {
  const void* k_new;        // [B][Hkv][D]
  const void* v_new;        // [B][Hkv][Dv]
  tq_dtype dt;
  const int32_t* seq_lens;  // [B] lengths after the append
};
// The appends of a decode step as launches of their own (quantize.hip).
hipError_t launch_append_step(const tq_kv_desc& k, const tq_kv_desc& v, const StepRows& st, int B, int Hkv,
                              hipStream_t s);

// Matrix-core quantiser for vectors of 32, 64, 96 or 128 channels (quantize_mfma.hip): rows
// 16-byte aligned.
bool quantize_mfma_supported(const tq_quantizer& q, tq_dtype dt, const void* x, int64_t stride);
// Matrix-core quantiser for vectors of more than 128 channels in the key
// layout (quantize_mfma.hip): two GEMM-shaped passes over batches of 65536
// vectors; with the sketch it keeps a device workspace of the batch's
// residuals (about 4 d bytes per vector), allocated on first use per
// device and kept until the process ends.
bool quantize_wide_supported(const tq_quantizer& q, tq_layout layout, tq_dtype dt, const void* x, int64_t stride);
hipError_t launch_quantize_wide(const tq_quantizer& q, tq_dtype dt, const void* x, int64_t n, int64_t stride,
                                void* packed, uint16_t* norm, uint16_t* rnorm, hipStream_t s);
hipError_t launch_quantize_mfma(const tq_quantizer& q, tq_layout layout, tq_dtype dt, const void* x, int64_t n,
                                int64_t stride, void* packed, uint16_t* norm, uint16_t* rnorm, hipStream_t s);

// Every check of a tq_decode_attn call except those of its workspace, in the
// same order; on TQ_OK *ws_need holds the workspace bytes the call needs.
int check_decode_call(const tq_kv_desc* k, const tq_kv_desc* v, const void* q, tq_dtype q_dtype, int B, int Hq,
                      int Hkv, int T_max, const int32_t* seq_lens, float scale, const float* out,
                      const float* scores_out, size_t* ws_need);

// Decode: workspace sizing and launch. Shapes are validated by the caller.
struct DecodePlan {
  int head_chunk;   // query heads per workgroup
  int n_chunks;     // head chunks per KV head
  int splits;       // sequence splits per (batch, KV head)
  int split_len;    // tokens per split (multiple of 256)
  int D;            // key channels
  int Dv;           // value channels
  size_t qprep_floats;
  size_t partial_floats;
};
DecodePlan plan_decode(const tq_kv_desc& k, const tq_kv_desc& v, int B, int Hq, int Hkv, int T_max);
hipError_t launch_decode(const tq_kv_desc& k, const tq_kv_desc& v, const void* q, tq_dtype qdt, int B, int Hq,
                         int Hkv, int T_max, const int32_t* seq_lens, float scale, float* out, float* scores_out,
                         void* ws, const DecodePlan& plan, hipStream_t s);

// Block table of a paged cache: the rows of (sequence b, KV head g) are
// block_tokens-row blocks of a pool of num_blocks blocks per head.
struct PageTable {
  const int32_t* table;  // device [B, max_blocks]
  int max_blocks;
  int block_tokens;      // a multiple of 256
  int64_t num_blocks;
};

// Matrix-core decode for 128-channel heads (decode_mfma.hip). With a block
// size, the split length divides it (a split never leaves its block).
bool mfma_decode_supported(const tq_kv_desc& k, const tq_kv_desc& v);
DecodePlan plan_decode_mfma(const tq_kv_desc& k, const tq_kv_desc& v, int B, int Hq, int Hkv, int T_max,
                            int block_tokens = 0);
hipError_t launch_decode_mfma(const tq_kv_desc& k, const tq_kv_desc& v, const void* q, tq_dtype qdt, int B, int Hq,
                              int Hkv, int T_max, const int32_t* seq_lens, float scale, float* out,
                              float* scores_out, void* ws, const DecodePlan& plan, hipStream_t s,
                              const PageTable* pages = nullptr, const StepRows* step = nullptr);
// Largest number of splits per sequence the combine handles.
int mfma_decode_max_splits();

// S R and its largest row norm (fold.hip).
hipError_t launch_fold(const tq_quantizer& q, float* SR, hipStream_t s);

// Search.
size_t search_workspace_bytes(const tq_group& db, int64_t N, int Q, int k);
// Matrix-core scores (search_mfma.hip): y~ = R y, y^ = S y~ into qt, qh
// ([Q][d] each) and the score matrix [Q][N].
bool search_mfma_supported(const tq_group& db);
// Bytes of workspace the matrix-core scan needs beyond y~, y^ and the scores.
size_t search_mfma_extra_bytes(const tq_group& db, int Q);
hipError_t launch_search_mfma_scores(const tq_group& db, int64_t N, const float* queries, int Q, float* qt,
                                     float* qh, float* scores, void* extra, hipStream_t s);
hipError_t launch_search(const tq_group& db, int64_t N, const float* queries, int Q, int k, int64_t* out_idx,
                         float* out_score, void* ws, hipStream_t s);

}  // namespace tqk
