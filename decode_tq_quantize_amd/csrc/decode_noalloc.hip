// tq_decode_attn_noalloc: compressed-KV decode attention whose workspace is a
// fixed device array held by the library, for callers that cannot allocate
// device memory. The attention itself is tq_decode_attn's.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"
#include "tq.h"

// The workspace of every call on a device: the transformed queries and the
// per-split partial softmax states. Each device holds its own copy, at its
// own address, from the library's load until the process ends. In host code
// this name is only a handle for the symbol lookup, never a device address.
static __device__ __align__(256) unsigned char scratch[TQ_DECODE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device, null until looked up

// Device address of the current device's copy, looked up once per device.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TQ_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TQ_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return TQ_OK;
}

}  // namespace

extern "C" int tq_decode_attn_noalloc(const tq_kv_desc* k, const tq_kv_desc* v, const void* q, tq_dtype q_dtype,
                                      int B, int Hq, int Hkv, int T_max, const int32_t* seq_lens, float scale,
                                      float* out, float* scores_out, void* stream) {
  size_t need = 0;
  int rc = tqk::check_decode_call(k, v, q, q_dtype, B, Hq, Hkv, T_max, seq_lens, scale, out, scores_out, &need);
  if (rc != TQ_OK) return rc;
  if (need > TQ_DECODE_SCRATCH_BYTES) return TQ_ERR_SCRATCH;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != TQ_OK) return rc;
  return tq_decode_attn(k, v, q, q_dtype, B, Hq, Hkv, T_max, seq_lens, scale, out, scores_out, ws,
                        TQ_DECODE_SCRATCH_BYTES, stream);
}
