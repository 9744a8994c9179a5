// Top-k inner-product search over TurboQuant codes (gfx950).
//
// uiyeonassociation "TurboQuant" post (results section): the same compressed
// vectors serve nearest-neighbour search by inner product. Each database
// vector's score against a query y is the unbiased estimate of <y, x>
// (riverfrot "TurboQuant" post, section 4.3):
//   s = n ( <R y, c[idx]> + gamma rho <S R y, 2 z - 1> ).
//
// Kernels:
//  sprep   y~ = R y and y^ = S y~ for every query (fp32)
//  scores  one workgroup per (256 database vectors, 8 queries): thread =
//          database vector, the queries' y~ / y^ staged in LDS
//  topk    one workgroup per query: every thread keeps a sorted top-k of its
//          strided share of the scores; the candidates are then ranked by
//          counting, for each, the candidates that beat it (higher score, or
//          equal score and lower index), and rank < k is written out.
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kQ = 8;           // queries per scores workgroup
constexpr int kMaxDim = TQ_MAX_DIM;

struct SArgs {
  const uint32_t* packed;
  const uint16_t* norm;
  const uint16_t* rnorm;
  const float* R;
  const float* S;
  int d, B, prod;
  float gamma;
  float cent[TQ_MAX_LEVELS];
  int64_t N;
  const float* queries;
  int Q, k;
  float* qprep;    // [Q, 2 d]
  float* scores;   // [Q, N]
  int64_t* out_idx;
  float* out_score;
};

__global__ __launch_bounds__(kThreads) void sprep_kernel(SArgs a) {
  extern __shared__ float sm[];  // 2 d floats
  float* yin = sm;
  float* yt = sm + a.d;
  const int qi = blockIdx.x, tid = threadIdx.x;
  for (int j = tid; j < a.d; j += kThreads) yin[j] = a.queries[(int64_t)qi * a.d + j];
  __syncthreads();
  float* dst = a.qprep + (int64_t)qi * 2 * a.d;
  for (int i = tid; i < a.d; i += kThreads) {
    float s = 0.f;
    for (int j = 0; j < a.d; ++j) s = fmaf(a.R[(int64_t)i * a.d + j], yin[j], s);
    yt[i] = s;
    dst[i] = s;
  }
  __syncthreads();
  for (int i = tid; i < a.d; i += kThreads) {
    float s = 0.f;
    if (a.prod)
      for (int j = 0; j < a.d; ++j) s = fmaf(a.S[(int64_t)i * a.d + j], yt[j], s);
    dst[a.d + i] = s;
  }
}

__global__ __launch_bounds__(kThreads) void scores_kernel(SArgs a) {
  extern __shared__ float sm[];  // kQ x 2 d
  __shared__ float cent[TQ_MAX_LEVELS];
  const int tid = threadIdx.x;
  const int q0 = blockIdx.y * kQ;
  const int nq = min(kQ, a.Q - q0);
  for (int e = tid; e < nq * 2 * a.d; e += kThreads) sm[e] = a.qprep[(int64_t)q0 * 2 * a.d + e];
  if (tid < TQ_MAX_LEVELS) cent[tid] = a.cent[tid];
  __syncthreads();
  const int64_t vi = (int64_t)blockIdx.x * kThreads + tid;
  if (vi >= a.N) return;
  const int64_t tile = vi / tqk::kKeysTile;
  const int tt = (int)(vi % tqk::kKeysTile);
  const int P = a.B + a.prod;
  const int Gw = a.d / 32;
  float mse[kQ], qjl[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q) mse[q] = qjl[q] = 0.f;
  for (int gw = 0; gw < Gw; ++gw) {
    const uint32_t* wp = a.packed + ((tile * Gw + gw) * tqk::kKeysTile + tt) * P;
    uint32_t w[TQ_MAX_MSE_BITS];
#pragma unroll
    for (int p = 0; p < TQ_MAX_MSE_BITS; ++p) w[p] = p < a.B ? wp[p] : 0u;
    const uint32_t wz = a.prod ? wp[a.B] : 0u;
    for (int i = 0; i < 32; ++i) {
      int idx = 0;
#pragma unroll
      for (int p = 0; p < TQ_MAX_MSE_BITS; ++p)
        if (p < a.B) idx |= (int)((w[p] >> i) & 1u) << p;
      const float cv = cent[idx];
      const float sg = ((wz >> i) & 1u) ? 1.f : -1.f;
      const int j = 32 * gw + i;
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        if (q < nq) {
          mse[q] = fmaf(sm[q * 2 * a.d + j], cv, mse[q]);
          qjl[q] = fmaf(sm[q * 2 * a.d + a.d + j], sg, qjl[q]);
        }
      }
    }
  }
  const float n = tqd::half_bits_to_f32(a.norm[vi]);
  const float rho = a.prod ? tqd::half_bits_to_f32(a.rnorm[vi]) : 0.f;
#pragma unroll
  for (int q = 0; q < kQ; ++q)
    if (q < nq) a.scores[(int64_t)(q0 + q) * a.N + vi] = n * (mse[q] + (a.prod ? a.gamma * rho * qjl[q] : 0.f));
}

// (s1, i1) ranks before (s2, i2)
__device__ __forceinline__ bool beats(float s1, int64_t i1, float s2, int64_t i2) {
  return s1 > s2 || (s1 == s2 && i1 < i2);
}

__global__ __launch_bounds__(kThreads) void topk_kernel(SArgs a, int nthreads) {
  extern __shared__ unsigned char raw[];
  float* ls = reinterpret_cast<float*>(raw);                      // nthreads * k scores
  int64_t* li = reinterpret_cast<int64_t*>(ls + nthreads * a.k);  // nthreads * k indices
  const int tid = threadIdx.x;
  const int qi = blockIdx.x;
  const int k = a.k;
  const float* sc = a.scores + (int64_t)qi * a.N;
  if (tid < nthreads) {
    float* ms = ls + tid * k;
    int64_t* mi = li + tid * k;
    int cnt = 0;
    for (int64_t i = tid; i < a.N; i += nthreads) {
      const float s = sc[i];
      if (cnt == k && !beats(s, i, ms[k - 1], mi[k - 1])) continue;
      int pos = cnt < k ? cnt : k - 1;
      while (pos > 0 && beats(s, i, ms[pos - 1], mi[pos - 1])) {
        ms[pos] = ms[pos - 1];
        mi[pos] = mi[pos - 1];
        --pos;
      }
      ms[pos] = s;
      mi[pos] = i;
      if (cnt < k) ++cnt;
    }
    for (int c = cnt; c < k; ++c) {
      ms[c] = -INFINITY;
      mi[c] = -1;
    }
  }
  __syncthreads();
  const int ncand = nthreads * k;
  for (int c = tid; c < ncand; c += kThreads) {
    const int64_t ic = li[c];
    if (ic < 0) continue;
    const float s = ls[c];
    int rank = 0;
    for (int o = 0; o < ncand && rank < k; ++o) {
      const int64_t io = li[o];
      if (io >= 0 && beats(ls[o], io, s, ic)) ++rank;
    }
    if (rank < k) {
      a.out_idx[(int64_t)qi * k + rank] = ic;
      a.out_score[(int64_t)qi * k + rank] = s;
    }
  }
}

int topk_threads(int k) {
  int t = 8192 / k;  // LDS: t * k * 12 bytes <= 96 KB
  t = t / 64 * 64;
  if (t > kThreads) t = kThreads;
  if (t < 64) t = 64;
  return t;
}

}  // namespace

namespace tqk {

size_t search_workspace_bytes(const tq_group& db, int64_t N, int Q, int k) {
  (void)k;
  return ((((size_t)Q * 2 * db.q.d + (size_t)Q * N) * sizeof(float) + 15) & ~(size_t)15) +
         search_mfma_extra_bytes(db, Q);
}

hipError_t launch_search(const tq_group& db, int64_t N, const float* queries, int Q, int k, int64_t* out_idx,
                         float* out_score, void* ws, hipStream_t s) {
  SArgs a{};
  a.packed = static_cast<const uint32_t*>(db.packed);
  a.norm = db.norm;
  a.rnorm = db.rnorm;
  a.R = db.q.R;
  a.S = db.q.S;
  a.d = db.q.d;
  a.B = db.q.mse_bits;
  a.prod = db.q.variant == TQ_PROD;
  a.gamma = (float)(sqrt(M_PI / 2.0) / db.q.d);
  for (int i = 0; i < TQ_MAX_LEVELS; ++i) a.cent[i] = db.q.centroids[i];
  a.N = N;
  a.queries = queries;
  a.Q = Q;
  a.k = k;
  a.qprep = static_cast<float*>(ws);
  a.scores = a.qprep + (size_t)Q * 2 * db.q.d;
  a.out_idx = out_idx;
  a.out_score = out_score;
  hipError_t e;
  if (search_mfma_supported(db)) {
    // matrix-core scores: y~ [Q][d], y^ [Q][d], then the score matrix
    char* extra = static_cast<char*>(ws) + ((((size_t)Q * 2 * a.d + (size_t)Q * N) * sizeof(float) + 15) & ~(size_t)15);
    e = launch_search_mfma_scores(db, N, queries, Q, a.qprep, a.qprep + (size_t)Q * a.d, a.scores, extra, s);
    if (e != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL(sprep_kernel, dim3(Q), dim3(kThreads), 2 * a.d * sizeof(float), s, a);
    const size_t lds_sc = (size_t)kQ * 2 * a.d * sizeof(float);
    e = hipFuncSetAttribute((const void*)scores_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_sc);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(scores_kernel, dim3((unsigned)((N + kThreads - 1) / kThreads), (Q + kQ - 1) / kQ),
                       dim3(kThreads), lds_sc, s, a);
  }
  const int nt = topk_threads(k);
  const size_t lds_tk = (size_t)nt * k * (sizeof(float) + sizeof(int64_t));
  e = hipFuncSetAttribute((const void*)topk_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_tk);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_kernel, dim3(Q), dim3(kThreads), lds_tk, s, a, nt);
  return hipGetLastError();
}

}  // namespace tqk
