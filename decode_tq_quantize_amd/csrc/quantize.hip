// Online TurboQuant compression of KV vectors (gfx950): the launches of the
// general quantiser (any d that is a multiple of 32; every append), whose
// per-tile work is quantize_tile in quantize_tile.h (riverfrot "TurboQuant"
// post, sections 4.1-4.3). Bulk quantisation takes tiles of 32 vectors
// where they fit LDS; appends take small tiles so that a few vectors per
// sequence still spread over the compute units.
#include <algorithm>

#include "device_common.h"
#include "internal.h"
#include "quantize_tile.h"

namespace {

using tqq::QArgs;

// Up to two tensors per launch (the keys and values of one append): grid
// row blockIdx.y takes argument set y.
struct QArgsPair {
  QArgs a[2];
};

template <int TV, bool DIRECT = false>
__global__ __launch_bounds__(tqq::kQThreads) void quantize_kernel(QArgsPair pair) {
  extern __shared__ float smem[];
  tqq::quantize_tile<TV, tqq::jc_of<TV>(), DIRECT>(pair.a[blockIdx.y], blockIdx.x, smem);
}

size_t lds_bytes(int d, int TV) { return tqq::lds_bytes(d, TV, TV <= 4 ? 128 : 32); }

// count (1 or 2) argument sets, the first nround vectors of each
template <int TV, bool DIRECT = false>
hipError_t launch_tv(const QArgs* as, int count, int64_t nround, hipStream_t s) {
  QArgsPair pair{};
  pair.a[0] = as[0];
  pair.a[1] = as[count > 1 ? 1 : 0];
  const size_t lds = tqq::lds_bytes(std::max(pair.a[0].d, pair.a[1].d), TV, tqq::jc_of<TV>());
  hipError_t e = hipFuncSetAttribute((const void*)quantize_kernel<TV, DIRECT>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t blocks = (nround + TV - 1) / TV;
  hipLaunchKernelGGL((quantize_kernel<TV, DIRECT>), dim3((unsigned)blocks, (unsigned)count), dim3(tqq::kQThreads), lds,
                     s, pair);
  return hipGetLastError();
}

using tqq::make_args;

constexpr size_t kLdsLimit = 150 * 1024;
// Appends of at most this many vectors per tensor take the direct products
// (measured: batch 1 x 8 KV heads faster, batch 64 x 8 slower, its larger
// register footprint costing more than the latency it saves).
constexpr int64_t kDirectMaxN = 64;

// An append is a few vectors per sequence: small tiles, so that the vectors
// spread over the compute units (about 256 workgroups or more per tensor).
hipError_t launch_rows(const QArgs* as, int count, int64_t n, hipStream_t s) {
  const int d = count > 1 ? std::max(as[0].d, as[1].d) : as[0].d;
  auto fits = [&](int tv) { return n >= 256 * (int64_t)tv && lds_bytes(d, tv) <= kLdsLimit; };
  if (fits(32)) return launch_tv<32>(as, count, n, s);
  if (fits(16)) return launch_tv<16>(as, count, n, s);
  if (fits(8)) return launch_tv<8>(as, count, n, s);
  if (fits(4)) return launch_tv<4>(as, count, n, s);
  // a handful of vectors (a decode step at small batch): latency first
  if (n <= kDirectMaxN && d <= tqq::kDirectMaxD) return launch_tv<2, true>(as, count, n, s);
  return launch_tv<2>(as, count, n, s);
}

}  // namespace

namespace tqk {

hipError_t launch_quantize(const tq_quantizer& q, tq_layout layout, tq_dtype dt, const void* x, int64_t n,
                           int64_t stride, void* packed, uint16_t* norm, uint16_t* rnorm, hipStream_t s,
                           const int64_t* rows, int64_t cache_rows) {
  const QArgs a = make_args(q, layout, dt, x, n, stride, packed, norm, rnorm, rows, cache_rows);
  if (rows) return launch_rows(&a, 1, n, s);  // (rows are written one by one: no output tile to round to)
  const int tile = layout == TQ_LAYOUT_KEYS ? kKeysTile : kValuesBlock;
  const int64_t nround = (n + tile - 1) / tile * tile;
  if (layout == TQ_LAYOUT_VALUES || lds_bytes(q.d, 32) <= kLdsLimit) return launch_tv<32>(&a, 1, nround, s);
  if (lds_bytes(q.d, 16) <= kLdsLimit) return launch_tv<16>(&a, 1, nround, s);
  if (lds_bytes(q.d, 8) <= kLdsLimit) return launch_tv<8>(&a, 1, nround, s);
  return launch_tv<4>(&a, 1, nround, s);
}

hipError_t launch_append_step(const tq_kv_desc& k, const tq_kv_desc& v, const StepRows& st, int B, int Hkv,
                              hipStream_t s) {
  QArgs as[2 * TQ_MAX_GROUPS];
  const int n = tqq::step_args(k, v, st, B, Hkv, as);
  const int64_t nv = (int64_t)B * Hkv;
  for (int i = 0; i < n; i += 2) {
    const hipError_t e = launch_rows(as + i, i + 1 < n ? 2 : 1, nv, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_append_pair(const tq_quantizer& qk, const tq_quantizer& qv, tq_dtype dt, const void* xk,
                              const void* xv, int64_t n, int64_t k_stride, int64_t v_stride, const int64_t* rows,
                              int64_t cache_rows, void* kpacked, uint16_t* knorm, uint16_t* krnorm, void* vpacked,
                              uint16_t* vnorm, uint16_t* vrnorm, hipStream_t s) {
  const QArgs as[2] = {
      make_args(qk, TQ_LAYOUT_KEYS, dt, xk, n, k_stride, kpacked, knorm, krnorm, rows, cache_rows),
      make_args(qv, TQ_LAYOUT_VALUES, dt, xv, n, v_stride, vpacked, vnorm, vrnorm, rows, cache_rows)};
  return launch_rows(as, 2, n, s);
}

}  // namespace tqk
