// libtq C ABI: argument validation, workspace sizing and kernel dispatch.
// Every check runs before the first device call; on error nothing is written.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "internal.h"
#include "tq.h"

namespace tqk {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];  // 0 = not yet queried
std::mutex g_occ_mu;
struct OccEntry {
  int dev;
  const void* fn;
  int threads, per_cu;
};
OccEntry g_occ[256];
int g_occ_n = 0;
}  // namespace

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int c = g_cus[dev].load(std::memory_order_relaxed);
  if (c > 0) return c;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) return 256;
  g_cus[dev].store(c, std::memory_order_relaxed);
  return c;
}

int kernel_wgs_per_cu(const void* fn, int threads) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  std::lock_guard<std::mutex> lk(g_occ_mu);
  for (int i = 0; i < g_occ_n; ++i)
    if (g_occ[i].dev == dev && g_occ[i].fn == fn && g_occ[i].threads == threads) return g_occ[i].per_cu;
  int per = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, threads, 0) != hipSuccess || per < 1) per = 1;
  if (g_occ_n < (int)(sizeof(g_occ) / sizeof(g_occ[0]))) g_occ[g_occ_n++] = OccEntry{dev, fn, threads, per};
  return per;
}

}  // namespace tqk

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape, pointer and codebook checks of one quantiser.
int check_quantizer(const tq_quantizer* q) {
  if (!q) return TQ_ERR_INVALID_ARG;
  if (q->d < 32 || q->d > TQ_MAX_DIM || (q->d % 32) != 0) return TQ_ERR_UNSUPPORTED;
  if (q->mse_bits < 1 || q->mse_bits > TQ_MAX_MSE_BITS) return TQ_ERR_UNSUPPORTED;
  if (q->variant != TQ_MSE && q->variant != TQ_PROD) return TQ_ERR_INVALID_ARG;
  if (!q->R || (q->variant == TQ_PROD && !q->S)) return TQ_ERR_INVALID_ARG;
  if (!aligned16(q->R) || (q->S && !aligned16(q->S)) || (q->SR && !aligned16(q->SR))) return TQ_ERR_MISALIGNED;
  if (q->SR && q->variant != TQ_PROD) return TQ_ERR_INVALID_ARG;
  const int L = 1 << q->mse_bits;
  for (int i = 0; i < L; ++i) {
    if (!std::isfinite(q->centroids[i])) return TQ_ERR_INVALID_ARG;
    if (i > 0 && !(q->centroids[i] > q->centroids[i - 1])) return TQ_ERR_INVALID_ARG;
  }
  for (int i = 0; i < L - 1; ++i) {
    if (!std::isfinite(q->thresholds[i])) return TQ_ERR_INVALID_ARG;
    if (i > 0 && !(q->thresholds[i] > q->thresholds[i - 1])) return TQ_ERR_INVALID_ARG;
  }
  return TQ_OK;
}

// The estimator kernels rely on the mirror symmetry of the codebook.
bool symmetric(const tq_quantizer& q) {
  const int L = 1 << q.mse_bits;
  for (int i = 0; i < L; ++i)
    if (q.centroids[i] != -q.centroids[L - 1 - i]) return false;
  return true;
}

int check_desc(const tq_kv_desc* k, bool values, int* total_d) {
  if (!k || k->n_groups < 1 || k->n_groups > TQ_MAX_GROUPS) return TQ_ERR_INVALID_ARG;
  int ch = 0;
  for (int i = 0; i < k->n_groups; ++i) {
    const tq_group& g = k->g[i];
    int rc = check_quantizer(&g.q);
    if (rc != TQ_OK) return rc;
    if (!symmetric(g.q)) return TQ_ERR_INVALID_ARG;
    if (g.ch_offset != ch) return TQ_ERR_INVALID_ARG;
    if (values && g.q.variant != TQ_MSE) return TQ_ERR_UNSUPPORTED;
    if (!g.packed || !g.norm || (g.q.variant == TQ_PROD && !g.rnorm)) return TQ_ERR_INVALID_ARG;
    if (!aligned16(g.packed) || !aligned16(g.norm) || (g.rnorm && !aligned16(g.rnorm))) return TQ_ERR_MISALIGNED;
    if (g.seq_stride <= 0 || (g.seq_stride % tqk::kValuesBlock) != 0) return TQ_ERR_INVALID_ARG;
    ch += g.q.d;
  }
  *total_d = ch;
  return TQ_OK;
}

int check_decode(const tq_kv_desc* k, const tq_kv_desc* v, int B, int Hq, int Hkv, int T_max, int* D, int* Dv) {
  int rc = check_desc(k, false, D);
  if (rc != TQ_OK) return rc;
  rc = check_desc(v, true, Dv);
  if (rc != TQ_OK) return rc;
  if (*D > 256 || *Dv > 256) return TQ_ERR_UNSUPPORTED;
  if (B < 1 || Hq < 1 || Hkv < 1 || (Hq % Hkv) != 0 || T_max < 1) return TQ_ERR_INVALID_ARG;
  for (int i = 0; i < k->n_groups; ++i)
    if (k->g[i].seq_stride < T_max) return TQ_ERR_INVALID_ARG;
  for (int i = 0; i < v->n_groups; ++i)
    if (v->g[i].seq_stride < T_max) return TQ_ERR_INVALID_ARG;
  return TQ_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? TQ_OK : TQ_ERR_HIP; }

// Shapes of a paged decode: the matrix-core layouts only, blocks of a
// multiple of 256 rows, every group's rows per (block, KV head) equal to the
// block size, and no more splits than the combine takes.
int check_paged_shape(const tq_kv_desc* k, const tq_kv_desc* v, int B, int Hq, int Hkv, int T_max,
                      int block_tokens, int* D, int* Dv) {
  int rc = check_desc(k, false, D);
  if (rc != TQ_OK) return rc;
  rc = check_desc(v, true, Dv);
  if (rc != TQ_OK) return rc;
  if (*D > 256 || *Dv > 256) return TQ_ERR_UNSUPPORTED;
  if (B < 1 || Hq < 1 || Hkv < 1 || (Hq % Hkv) != 0 || T_max < 1) return TQ_ERR_INVALID_ARG;
  if (block_tokens < 256 || block_tokens % 256) return TQ_ERR_UNSUPPORTED;
  for (int i = 0; i < k->n_groups; ++i)
    if (k->g[i].seq_stride != block_tokens) return TQ_ERR_INVALID_ARG;
  for (int i = 0; i < v->n_groups; ++i)
    if (v->g[i].seq_stride != block_tokens) return TQ_ERR_INVALID_ARG;
  if (!tqk::mfma_decode_supported(*k, *v)) return TQ_ERR_UNSUPPORTED;
  const tqk::DecodePlan p = tqk::plan_decode_mfma(*k, *v, B, Hq, Hkv, T_max, block_tokens);
  if (p.splits > tqk::mfma_decode_max_splits()) return TQ_ERR_UNSUPPORTED;
  return TQ_OK;
}

// 128-channel heads run on the matrix cores; other head sizes on the
// general kernel of decode.hip.
tqk::DecodePlan decode_plan(const tq_kv_desc& k, const tq_kv_desc& v, int B, int Hq, int Hkv, int T_max) {
  return tqk::mfma_decode_supported(k, v) ? tqk::plan_decode_mfma(k, v, B, Hq, Hkv, T_max)
                                          : tqk::plan_decode(k, v, B, Hq, Hkv, T_max);
}

}  // namespace

extern "C" const char* tq_status_string(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_ERR_INVALID_ARG: return "invalid argument";
    case TQ_ERR_UNSUPPORTED: return "unsupported dimension or bit width";
    case TQ_ERR_MISALIGNED: return "device pointer not 16-byte aligned";
    case TQ_ERR_NO_CONVERGE: return "Lloyd-Max iteration did not converge";
    case TQ_ERR_HIP: return "HIP launch failed";
    case TQ_ERR_WORKSPACE: return "workspace missing or too small";
    case TQ_ERR_SCRATCH: return "needs more workspace than the fixed decode scratch (TQ_DECODE_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

extern "C" size_t tq_fold_bytes(int d) {
  if (d < 32 || d > TQ_MAX_DIM || (d % 32) != 0) return 0;
  return ((size_t)d * d + 4) * sizeof(float);
}

extern "C" int tq_fold_qjl(const tq_quantizer* q, float* SR, void* stream) {
  int rc = check_quantizer(q);
  if (rc != TQ_OK) return rc;
  if (q->variant != TQ_PROD || !SR) return TQ_ERR_INVALID_ARG;
  if (!aligned16(SR)) return TQ_ERR_MISALIGNED;
  return hip_status(tqk::launch_fold(*q, SR, static_cast<hipStream_t>(stream)));
}

extern "C" size_t tq_packed_bytes(int d, int mse_bits, tq_variant variant, tq_layout layout, int64_t n) {
  if (d < 32 || d > TQ_MAX_DIM || (d % 32) != 0 || mse_bits < 1 || mse_bits > TQ_MAX_MSE_BITS || n < 0) return 0;
  if (variant != TQ_MSE && variant != TQ_PROD) return 0;
  if (layout != TQ_LAYOUT_KEYS && layout != TQ_LAYOUT_VALUES) return 0;
  const int P = mse_bits + (variant == TQ_PROD ? 1 : 0);
  const int64_t tile = layout == TQ_LAYOUT_KEYS ? tqk::kKeysTile : tqk::kValuesBlock;
  const int64_t nr = (n + tile - 1) / tile * tile;
  return (size_t)nr * (size_t)P * (size_t)d / 8;
}

extern "C" int tq_append_kv_pair(const tq_quantizer* qk, const tq_quantizer* qv, tq_dtype in_dtype, const void* xk,
                                 const void* xv, int64_t n, int64_t xk_stride_elems, int64_t xv_stride_elems,
                                 const int64_t* rows, int64_t cache_rows, void* kpacked, uint16_t* knorm,
                                 uint16_t* krnorm, void* vpacked, uint16_t* vnorm, uint16_t* vrnorm, void* stream) {
  int rc = check_quantizer(qk);
  if (rc != TQ_OK) return rc;
  rc = check_quantizer(qv);
  if (rc != TQ_OK) return rc;
  if (in_dtype != TQ_F32 && in_dtype != TQ_BF16) return TQ_ERR_INVALID_ARG;
  if (n < 0 || xk_stride_elems < qk->d || xv_stride_elems < qv->d || cache_rows <= 0) return TQ_ERR_INVALID_ARG;
  if (qv->d > 256) return TQ_ERR_UNSUPPORTED;
  if (n == 0) return TQ_OK;
  if (!xk || !xv || !rows || !kpacked || !knorm || (qk->variant == TQ_PROD && !krnorm) || !vpacked || !vnorm ||
      (qv->variant == TQ_PROD && !vrnorm))
    return TQ_ERR_INVALID_ARG;
  if (!aligned16(xk) || !aligned16(xv) || !aligned16(kpacked) || !aligned16(knorm) || (krnorm && !aligned16(krnorm)) ||
      !aligned16(vpacked) || !aligned16(vnorm) || (vrnorm && !aligned16(vrnorm)) ||
      reinterpret_cast<uintptr_t>(rows) % alignof(int64_t) != 0)
    return TQ_ERR_MISALIGNED;
  return hip_status(tqk::launch_append_pair(*qk, *qv, in_dtype, xk, xv, n, xk_stride_elems, xv_stride_elems, rows,
                                            cache_rows, kpacked, knorm, qk->variant == TQ_PROD ? krnorm : nullptr,
                                            vpacked, vnorm, qv->variant == TQ_PROD ? vrnorm : nullptr,
                                            static_cast<hipStream_t>(stream)));
}

extern "C" int tq_kv_bit_allocation(double key_norm, double value_norm, int* key_bits, int* value_bits) {
  if (!key_bits || !value_bits) return TQ_ERR_INVALID_ARG;
  if (!std::isfinite(key_norm) || !std::isfinite(value_norm) || !(key_norm > 0.0) || !(value_norm > 0.0))
    return TQ_ERR_INVALID_ARG;
  const double r = key_norm / value_norm;
  if (r < 10.0) {
    *key_bits = 3;
    *value_bits = 3;
    return TQ_KV_UNIFORM;
  }
  *key_bits = 4;
  *value_bits = 2;
  return r <= 100.0 ? TQ_KV_ASYMMETRIC : TQ_KV_MIXED;
}

extern "C" int tq_quantize_kv(const tq_quantizer* q, tq_layout layout, tq_dtype in_dtype, const void* x, int64_t n,
                              int64_t x_stride_elems, void* packed, uint16_t* norm, uint16_t* rnorm, void* stream) {
  int rc = check_quantizer(q);
  if (rc != TQ_OK) return rc;
  if (layout != TQ_LAYOUT_KEYS && layout != TQ_LAYOUT_VALUES) return TQ_ERR_INVALID_ARG;
  if (in_dtype != TQ_F32 && in_dtype != TQ_BF16) return TQ_ERR_INVALID_ARG;
  if (n < 0 || x_stride_elems < q->d) return TQ_ERR_INVALID_ARG;
  if (layout == TQ_LAYOUT_VALUES && q->d > 256) return TQ_ERR_UNSUPPORTED;
  if (n == 0) return TQ_OK;
  if (!x || !packed || !norm || (q->variant == TQ_PROD && !rnorm)) return TQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(packed) || !aligned16(norm) || (rnorm && !aligned16(rnorm)))
    return TQ_ERR_MISALIGNED;
  uint16_t* rn = q->variant == TQ_PROD ? rnorm : nullptr;
  if (tqk::quantize_wide_supported(*q, layout, in_dtype, x, x_stride_elems))
    return hip_status(tqk::launch_quantize_wide(*q, in_dtype, x, n, x_stride_elems, packed, norm, rn,
                                                static_cast<hipStream_t>(stream)));
  if (tqk::quantize_mfma_supported(*q, in_dtype, x, x_stride_elems))
    return hip_status(tqk::launch_quantize_mfma(*q, layout, in_dtype, x, n, x_stride_elems, packed, norm, rn,
                                                static_cast<hipStream_t>(stream)));
  return hip_status(tqk::launch_quantize(*q, layout, in_dtype, x, n, x_stride_elems, packed, norm, rn,
                                         static_cast<hipStream_t>(stream)));
}

extern "C" int tq_append_kv(const tq_quantizer* q, tq_layout layout, tq_dtype in_dtype, const void* x, int64_t n,
                            int64_t x_stride_elems, const int64_t* rows, int64_t cache_rows, void* packed,
                            uint16_t* norm, uint16_t* rnorm, void* stream) {
  int rc = check_quantizer(q);
  if (rc != TQ_OK) return rc;
  if (layout != TQ_LAYOUT_KEYS && layout != TQ_LAYOUT_VALUES) return TQ_ERR_INVALID_ARG;
  if (in_dtype != TQ_F32 && in_dtype != TQ_BF16) return TQ_ERR_INVALID_ARG;
  if (n < 0 || x_stride_elems < q->d || cache_rows <= 0) return TQ_ERR_INVALID_ARG;
  if (layout == TQ_LAYOUT_VALUES && q->d > 256) return TQ_ERR_UNSUPPORTED;
  if (n == 0) return TQ_OK;
  if (!x || !rows || !packed || !norm || (q->variant == TQ_PROD && !rnorm)) return TQ_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(packed) || !aligned16(norm) || (rnorm && !aligned16(rnorm)) ||
      reinterpret_cast<uintptr_t>(rows) % alignof(int64_t) != 0)
    return TQ_ERR_MISALIGNED;
  uint16_t* rn = q->variant == TQ_PROD ? rnorm : nullptr;
  return hip_status(tqk::launch_quantize(*q, layout, in_dtype, x, n, x_stride_elems, packed, norm, rn,
                                         static_cast<hipStream_t>(stream), rows, cache_rows));
}

extern "C" size_t tq_decode_workspace_bytes(const tq_kv_desc* k, const tq_kv_desc* v, int B, int Hq, int Hkv,
                                            int T_max) {
  int D = 0, Dv = 0;
  if (check_decode(k, v, B, Hq, Hkv, T_max, &D, &Dv) != TQ_OK) return 0;
  const tqk::DecodePlan p = decode_plan(*k, *v, B, Hq, Hkv, T_max);
  return (p.qprep_floats + p.partial_floats) * sizeof(float);
}

namespace tqk {

int check_decode_call(const tq_kv_desc* k, const tq_kv_desc* v, const void* q, tq_dtype q_dtype, int B, int Hq,
                      int Hkv, int T_max, const int32_t* seq_lens, float scale, const float* out,
                      const float* scores_out, size_t* ws_need) {
  int D = 0, Dv = 0;
  int rc = check_decode(k, v, B, Hq, Hkv, T_max, &D, &Dv);
  if (rc != TQ_OK) return rc;
  if (!q || !out) return TQ_ERR_INVALID_ARG;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return TQ_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return TQ_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out) || (scores_out && !aligned16(scores_out)) ||
      (seq_lens && !aligned16(seq_lens)))
    return TQ_ERR_MISALIGNED;
  const tqk::DecodePlan p = decode_plan(*k, *v, B, Hq, Hkv, T_max);
  *ws_need = (p.qprep_floats + p.partial_floats) * sizeof(float);
  return TQ_OK;
}

}  // namespace tqk

extern "C" int tq_decode_attn(const tq_kv_desc* k, const tq_kv_desc* v, const void* q, tq_dtype q_dtype, int B,
                              int Hq, int Hkv, int T_max, const int32_t* seq_lens, float scale, float* out,
                              float* scores_out, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  const int rc = tqk::check_decode_call(k, v, q, q_dtype, B, Hq, Hkv, T_max, seq_lens, scale, out, scores_out, &need);
  if (rc != TQ_OK) return rc;
  if (ws && !aligned16(ws)) return TQ_ERR_MISALIGNED;
  if (!ws || ws_bytes < need) return TQ_ERR_WORKSPACE;
  const tqk::DecodePlan p = decode_plan(*k, *v, B, Hq, Hkv, T_max);
  if (tqk::mfma_decode_supported(*k, *v))
    return hip_status(tqk::launch_decode_mfma(*k, *v, q, q_dtype, B, Hq, Hkv, T_max, seq_lens, scale, out,
                                              scores_out, ws, p, static_cast<hipStream_t>(stream)));
  return hip_status(tqk::launch_decode(*k, *v, q, q_dtype, B, Hq, Hkv, T_max, seq_lens, scale, out, scores_out,
                                       ws, p, static_cast<hipStream_t>(stream)));
}

extern "C" int tq_decode_step(const tq_kv_desc* k, const tq_kv_desc* v, const void* k_new, const void* v_new,
                              tq_dtype kv_dtype, const void* q, tq_dtype q_dtype, int B, int Hq, int Hkv, int T_max,
                              const int32_t* seq_lens, float scale, float* out, float* scores_out, void* ws,
                              size_t ws_bytes, void* stream) {
  size_t need = 0;
  const int rc = tqk::check_decode_call(k, v, q, q_dtype, B, Hq, Hkv, T_max, seq_lens, scale, out, scores_out, &need);
  if (rc != TQ_OK) return rc;
  if (!k_new || !v_new || !seq_lens) return TQ_ERR_INVALID_ARG;
  if (kv_dtype != TQ_F32 && kv_dtype != TQ_BF16) return TQ_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new)) return TQ_ERR_MISALIGNED;
  if (ws && !aligned16(ws)) return TQ_ERR_MISALIGNED;
  if (!ws || ws_bytes < need) return TQ_ERR_WORKSPACE;
  const tqk::DecodePlan p = decode_plan(*k, *v, B, Hq, Hkv, T_max);
  const tqk::StepRows st{k_new, v_new, kv_dtype, seq_lens};
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (tqk::mfma_decode_supported(*k, *v))
    return hip_status(tqk::launch_decode_mfma(*k, *v, q, q_dtype, B, Hq, Hkv, T_max, seq_lens, scale, out,
                                              scores_out, ws, p, s, nullptr, &st));
  const hipError_t e = tqk::launch_append_step(*k, *v, st, B, Hkv, s);
  if (e != hipSuccess) return TQ_ERR_HIP;
  return hip_status(tqk::launch_decode(*k, *v, q, q_dtype, B, Hq, Hkv, T_max, seq_lens, scale, out, scores_out, ws,
                                       p, s));
}

extern "C" size_t tq_decode_paged_workspace_bytes(const tq_kv_desc* k, const tq_kv_desc* v, int B, int Hq, int Hkv,
                                                  int T_max, int block_tokens) {
  int D = 0, Dv = 0;
  if (check_paged_shape(k, v, B, Hq, Hkv, T_max, block_tokens, &D, &Dv) != TQ_OK) return 0;
  const tqk::DecodePlan p = tqk::plan_decode_mfma(*k, *v, B, Hq, Hkv, T_max, block_tokens);
  return (p.qprep_floats + p.partial_floats) * sizeof(float);
}

extern "C" int tq_decode_attn_paged(const tq_kv_desc* k, const tq_kv_desc* v, const void* q, tq_dtype q_dtype, int B,
                                    int Hq, int Hkv, int T_max, const int32_t* seq_lens, const int32_t* block_table,
                                    int max_blocks, int block_tokens, int64_t num_blocks, float scale, float* out,
                                    float* scores_out, void* ws, size_t ws_bytes, void* stream) {
  int D = 0, Dv = 0;
  int rc = check_paged_shape(k, v, B, Hq, Hkv, T_max, block_tokens, &D, &Dv);
  if (rc != TQ_OK) return rc;
  if (!q || !out || !block_table || max_blocks < 1 || num_blocks < 1) return TQ_ERR_INVALID_ARG;
  if ((int64_t)max_blocks * block_tokens < T_max) return TQ_ERR_INVALID_ARG;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return TQ_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return TQ_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out) || (scores_out && !aligned16(scores_out)) ||
      (seq_lens && !aligned16(seq_lens)) || (ws && !aligned16(ws)) ||
      reinterpret_cast<uintptr_t>(block_table) % alignof(int32_t) != 0)
    return TQ_ERR_MISALIGNED;
  const tqk::DecodePlan p = tqk::plan_decode_mfma(*k, *v, B, Hq, Hkv, T_max, block_tokens);
  if (!ws || ws_bytes < (p.qprep_floats + p.partial_floats) * sizeof(float)) return TQ_ERR_WORKSPACE;
  const tqk::PageTable pages{block_table, max_blocks, block_tokens, num_blocks};
  return hip_status(tqk::launch_decode_mfma(*k, *v, q, q_dtype, B, Hq, Hkv, T_max, seq_lens, scale, out, scores_out,
                                            ws, p, static_cast<hipStream_t>(stream), &pages));
}

extern "C" size_t tq_search_workspace_bytes(const tq_group* db, int64_t N, int Q, int k) {
  if (!db || check_quantizer(&db->q) != TQ_OK || N < 1 || N >= ((int64_t)1 << 29) || Q < 1 || k < 1 || k > 64 || k > N)
    return 0;
  return tqk::search_workspace_bytes(*db, N, Q, k);
}

extern "C" int tq_search_topk(const tq_group* db, int64_t N, const float* queries, int Q, int k, int64_t* out_idx,
                              float* out_score, void* ws, size_t ws_bytes, void* stream) {
  if (!db) return TQ_ERR_INVALID_ARG;
  int rc = check_quantizer(&db->q);
  if (rc != TQ_OK) return rc;
  if (!symmetric(db->q)) return TQ_ERR_INVALID_ARG;
  if (N < 1 || N >= ((int64_t)1 << 29) || Q < 1 || k < 1 || k > 64 || k > N) return TQ_ERR_INVALID_ARG;
  if (!db->packed || !db->norm || (db->q.variant == TQ_PROD && !db->rnorm) || !queries || !out_idx || !out_score)
    return TQ_ERR_INVALID_ARG;
  if (!aligned16(db->packed) || !aligned16(db->norm) || (db->rnorm && !aligned16(db->rnorm)) ||
      !aligned16(queries) || !aligned16(out_idx) || !aligned16(out_score) || (ws && !aligned16(ws)))
    return TQ_ERR_MISALIGNED;
  if (!ws || ws_bytes < tqk::search_workspace_bytes(*db, N, Q, k)) return TQ_ERR_WORKSPACE;
  return hip_status(tqk::launch_search(*db, N, queries, Q, k, out_idx, out_score, ws,
                                       static_cast<hipStream_t>(stream)));
}
