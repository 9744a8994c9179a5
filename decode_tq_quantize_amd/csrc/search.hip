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
//  topk2   one workgroup per query: a threshold filter over the score row
//          with per-wave candidate lists, re-ranked by counting (below)
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
// Top-k of one score row by threshold filtering. One workgroup of 8 waves per query; wave w reads chunks
// w, w + 8, ... of 1024 scores (64 lanes x 16, four 16-byte loads per lane,
// the next chunk in flight while one is examined). Each wave keeps its best k
// in LDS, sorted, and its k-th best score as a threshold: a score below the
// threshold cannot enter, so in the common case a chunk costs 16 compares per
// lane. Scores at or above it are appended to a per-wave candidate list
// (ballot + prefix count); when 64 or more have gathered, the list and the
// current best k are re-ranked by counting, for each entry, the entries that
// beat it (higher score, or equal score and lower index). The 8 waves' lists
// are merged the same way at the end. Rows start at any 4-byte boundary: the
// buffer resource starts at the 16-byte boundary below the row and elements
// outside [0, N) are never candidates.
constexpr int kTk2Waves = 8;
constexpr int kTk2Cap = 64 + 128;  // best k (<= 64) + candidates (< 128)

__device__ __forceinline__ bool beats32(float s1, int i1, float s2, int i2) {
  return s1 > s2 || (s1 == s2 && i1 < i2);
}

__global__ __launch_bounds__(64 * kTk2Waves) void topk2_kernel(const float* scores, int64_t N, int k,
                                                           int64_t* out_idx, float* out_score) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  // per wave: entries [0, k) are its best k in rank order, [k, k + count) the
  // candidates gathered since the last re-ranking; .x = score bits, .y = index
  __shared__ uint2 E[kTk2Waves][kTk2Cap];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qi = blockIdx.x;
  const uintptr_t ra = reinterpret_cast<uintptr_t>(scores + (int64_t)qi * N);
  const int off0 = (int)((ra & 15) >> 2);
  const int nel = (int)N + off0;
  const __amdgpu_buffer_rsrc_t res = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(ra & ~(uintptr_t)15), (short)0, (int)(4 * nel), 0x00020000);
  const int nch = (nel + 1023) >> 10;
  // distinct placeholders that every real entry beats (-inf, indices above
  // any row index), in rank order
  E[w][lane] = make_uint2(__float_as_uint(-INFINITY), 0x7fff0000u + (uint32_t)(w * 64 + lane));
  float tau = -INFINITY;  // score of the wave's k-th best entry
  int count = 0;

  auto rerank = [&]() __attribute__((always_inline)) {
    const int n = k + count;
    float sv[3];
    int iv[3], rk[3] = {0, 0, 0};
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const int e = lane + 64 * t;
      const uint2 x = E[w][e < n ? e : 0];
      sv[t] = __uint_as_float(x.x);
      iv[t] = e < n ? (int)x.y : 0x7fffffff;
    }
    for (int o = 0; o < n; ++o) {
      const uint2 x = E[w][o];
      const float so = __uint_as_float(x.x);
      const int io = (int)x.y;
#pragma unroll
      for (int t = 0; t < 3; ++t) rk[t] += beats32(so, io, sv[t], iv[t]) ? 1 : 0;
    }
#pragma unroll
    for (int t = 0; t < 3; ++t)
      if (lane + 64 * t < n && rk[t] < k) E[w][rk[t]] = make_uint2(__float_as_uint(sv[t]), (uint32_t)iv[t]);
    tau = __uint_as_float(__builtin_amdgcn_readfirstlane(E[w][k - 1].x));
    count = 0;
  };

  // examine one chunk held in registers
  auto examine = [&](const u4 (&x)[4], int c) __attribute__((always_inline)) {
    bool any = false;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
#pragma unroll
      for (int e = 0; e < 4; ++e) any |= __uint_as_float(x[sl][e]) >= tau;
    if (__builtin_amdgcn_ballot_w64(any) == 0) return;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = __uint_as_float(x[sl][e]);
        const int i = c * 1024 + sl * 256 + lane * 4 + e - off0;
        const bool cand = v >= tau && i >= 0 && i < (int)N;
        const uint64_t m = __builtin_amdgcn_ballot_w64(cand);
        if (m != 0) {
          if (cand) {
            const int pos = k + count + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            E[w][pos] = make_uint2(__float_as_uint(v), (uint32_t)i);
          }
          count += __builtin_popcountll(m);
          if (count >= 64) rerank();
        }
      }
  };
  // chunk c of the row at lane offset voff (loads past the row's end return
  // zeros, and their elements are never candidates)
  auto load = [&](u4 (&x)[4], int c) __attribute__((always_inline)) {
    const uint32_t voff = (uint32_t)(lane * 16) + (uint32_t)c * 4096u;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) x[sl] = __builtin_amdgcn_raw_buffer_load_b128(res, voff + 1024 * sl, 0, 0);
  };
  // two chunks per iteration, each loaded one chunk ahead
  u4 xa[4], xb[4];
  load(xa, w);
  for (int c = w; c < nch; c += 2 * kTk2Waves) {
    load(xb, c + kTk2Waves);
    examine(xa, c);
    load(xa, c + 2 * kTk2Waves);
    examine(xb, c + kTk2Waves);
  }
  if (count > 0) rerank();
  __syncthreads();
  // merge: the 8 k entries of all waves, ranked by counting
  const int n = kTk2Waves * k;
  if (tid < n) {
    const uint2 x = E[tid / k][tid % k];
    const float sv = __uint_as_float(x.x);
    const int iv = (int)x.y;
    int rk = 0;
    for (int o = 0; o < n; ++o) {
      const uint2 y = E[o / k][o % k];
      rk += beats32(__uint_as_float(y.x), (int)y.y, sv, iv) ? 1 : 0;
    }
    if (rk < k) {
      out_idx[(int64_t)qi * k + rk] = iv;
      out_score[(int64_t)qi * k + rk] = sv;
    }
  }
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
  hipLaunchKernelGGL(topk2_kernel, dim3(Q), dim3(64 * kTk2Waves), 0, s, a.scores, N, k, out_idx, out_score);
  return hipGetLastError();
}

}  // namespace tqk
