// Inner-product search scores on the gfx950 matrix cores (uiyeonassociation
// "TurboQuant" post, vector search with TurboQuant codes; estimator of the
// riverfrot "TurboQuant" post, section 4.3):
//   s(y, x) = n ( <R y, c[idx]> + gamma rho <S R y, 2 z - 1> ).
//
// qgemm: C[m][i] = sum_j A[m][j] B[i][j] in fp32 (16 x 16 tiles through
//        LDS), giving y~ = R y for every query, then y^ = S y~.
// scan:  one workgroup per (256 database vectors, 64 queries). Both sums of
//        the estimator are one contraction over 2 d terms, run on
//        v_mfma_f32_16x16x4_f32 (fp32 operands and accumulation): the A
//        operand holds y~ and y^ (staged in LDS one 32-coordinate group at a
//        time), the B operand is decoded from the packed planes in registers
//        (the centroid c[idx] for the first sum, gamma rho (2 z - 1) for the
//        second). In MFMA step e of a group, lane group kq (lanes 16 kq ..
//        16 kq + 15) carries coordinate 32 g + 8 kq + e, so a lane reads bits
//        8 kq .. 8 kq + 7 of each plane word. Wave w owns database tiles
//        4 w .. 4 w + 3 of the block for all 4 query tiles (16 accumulators).
//        Scores (times n) go to the score matrix, which the top-k kernel of
//        search.hip reduces.
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kQB = 64;   // queries per scan workgroup
constexpr int kNB = 256;  // database vectors per scan workgroup
constexpr int kGT = 16;   // qgemm tile

__global__ __launch_bounds__(kGT * kGT) void qgemm_kernel(const float* __restrict__ A, int M,
                                                          const float* __restrict__ Bm, int d,
                                                          float* __restrict__ C) {
  __shared__ float ta[kGT][kGT + 1], tb[kGT][kGT + 1];
  const int tx = threadIdx.x % kGT, ty = threadIdx.x / kGT;
  const int m = blockIdx.y * kGT + ty, i = blockIdx.x * kGT + tx;
  const int mr = min(m, M - 1);
  float acc = 0.f;
  for (int j0 = 0; j0 < d; j0 += kGT) {
    ta[ty][tx] = A[(int64_t)mr * d + j0 + tx];
    tb[ty][tx] = Bm[(int64_t)(blockIdx.x * kGT + ty) * d + j0 + tx];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kGT; ++k) acc = fmaf(ta[ty][k], tb[tx][k], acc);
    __syncthreads();
  }
  if (m < M) C[(int64_t)m * d + i] = acc;
}

struct ScanArgs {
  const uint32_t* packed;
  const uint16_t* norm;
  const uint16_t* rnorm;
  const float* qt;  // [Q][d]
  const float* qh;  // [Q][d]
  float* scores;    // [Q][N]
  int64_t N;
  int Q, d, B, prod;
  float gamma;
  float cent[TQ_MAX_LEVELS];
};

__device__ __forceinline__ v4f mfma_f32(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int B, bool PROD>
__global__ __launch_bounds__(kThreads, 2) void scan_kernel(ScanArgs a) {
  constexpr int P = B + (PROD ? 1 : 0);
  __shared__ __attribute__((aligned(16))) float aq[2][kQB][32 + 4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kq = lane >> 4, nl = lane & 15;
  const int64_t vb = (int64_t)blockIdx.x * kNB;
  const int q0 = blockIdx.y * kQB;
  const int G = a.d / 32;
  const int64_t last_tile = (a.N - 1) / tqk::kKeysTile;
  // centroids as uniform values, selected per lane
  float cen[1 << B];
#pragma unroll
  for (int i = 0; i < (1 << B); ++i) cen[i] = a.cent[i];
  // this lane's database vectors (one per tile of the wave) and their norms
  int64_t tile[4];
  float nv[4], gr[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t v = vb + 16 * (4 * w + t) + nl;
    tile[t] = min((vb >> 4) + 4 * w + t, last_tile);
    const int64_t vr = v < a.N ? v : a.N - 1;
    nv[t] = tqd::half_bits_to_f32(a.norm[vr]);
    gr[t] = PROD ? a.gamma * tqd::half_bits_to_f32(a.rnorm[vr]) : 0.f;
  }
  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int g = 0; g < G; ++g) {
    // stage y~ and y^ of the 64 queries at coordinates 32 g .. 32 g + 31
    {
      const int pr = tid >> 7, m = (tid >> 1) & 63, half = tid & 1;
      const int qr = min(q0 + m, a.Q - 1);
      const float* src = (pr ? a.qh : a.qt) + (int64_t)qr * a.d + 32 * g + 16 * half;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        *reinterpret_cast<float4*>(&aq[pr][m][16 * half + 4 * k]) = reinterpret_cast<const float4*>(src)[k];
    }
    // this lane's plane words of group g for its 4 database vectors
    uint32_t wd[4][P];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t* p = a.packed + ((tile[t] * G + g) * tqk::kKeysTile + nl) * P;
#pragma unroll
      for (int pp = 0; pp < P; ++pp) wd[t][pp] = p[pp];
    }
    __syncthreads();
    // A operands: rows 16 qt + nl, steps e = 0..7 (coordinate 8 kq + e)
    float at[4][8], ah[4][8];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float4 u = *reinterpret_cast<const float4*>(&aq[0][16 * qt + nl][8 * kq + 4 * h]);
        at[qt][4 * h] = u.x; at[qt][4 * h + 1] = u.y; at[qt][4 * h + 2] = u.z; at[qt][4 * h + 3] = u.w;
        if (PROD) {
          const float4 v = *reinterpret_cast<const float4*>(&aq[1][16 * qt + nl][8 * kq + 4 * h]);
          ah[qt][4 * h] = v.x; ah[qt][4 * h + 1] = v.y; ah[qt][4 * h + 2] = v.z; ah[qt][4 * h + 3] = v.w;
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int bit = 8 * kq + e;
      float bm[4], bq[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        int idx = 0;
#pragma unroll
        for (int pp = 0; pp < B; ++pp) idx |= (int)((wd[t][pp] >> bit) & 1u) << pp;
        float c = cen[0];
#pragma unroll
        for (int i = 1; i < (1 << B); ++i) c = idx == i ? cen[i] : c;
        bm[t] = c;
        bq[t] = PROD ? (((wd[t][B % P] >> bit) & 1u) ? gr[t] : -gr[t]) : 0.f;
      }
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          acc[qt][t] = mfma_f32(at[qt][e], bm[t], acc[qt][t]);
          if (PROD) acc[qt][t] = mfma_f32(ah[qt][e], bq[t], acc[qt][t]);
        }
    }
    __syncthreads();  // aq is rewritten for the next group
  }
  // scores of queries 16 qt + 4 kq + r, vectors vb + 16 (4 w + t) + nl
#pragma unroll
  for (int qt = 0; qt < 4; ++qt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int qi = q0 + 16 * qt + 4 * kq + r;
      if (qi < a.Q) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int64_t v = vb + 16 * (4 * w + t) + nl;
          if (v < a.N) a.scores[(int64_t)qi * a.N + v] = nv[t] * acc[qt][t][r];
        }
      }
    }
}

}  // namespace

namespace tqk {

bool search_mfma_supported(const tq_group& db) { return db.q.d % 32 == 0 && db.q.d >= 32; }

hipError_t launch_search_mfma_scores(const tq_group& db, int64_t N, const float* queries, int Q, float* qt,
                                     float* qh, float* scores, hipStream_t s) {
  const int d = db.q.d;
  const dim3 gg(d / kGT, (Q + kGT - 1) / kGT);
  hipLaunchKernelGGL(qgemm_kernel, gg, dim3(kGT * kGT), 0, s, queries, Q, db.q.R, d, qt);
  if (db.q.variant == TQ_PROD) hipLaunchKernelGGL(qgemm_kernel, gg, dim3(kGT * kGT), 0, s, qt, Q, db.q.S, d, qh);
  ScanArgs a{};
  a.packed = static_cast<const uint32_t*>(db.packed);
  a.norm = db.norm;
  a.rnorm = db.rnorm;
  a.qt = qt;
  a.qh = db.q.variant == TQ_PROD ? qh : qt;
  a.scores = scores;
  a.N = N;
  a.Q = Q;
  a.d = d;
  a.B = db.q.mse_bits;
  a.prod = db.q.variant == TQ_PROD;
  a.gamma = (float)(sqrt(M_PI / 2.0) / d);
  for (int i = 0; i < TQ_MAX_LEVELS; ++i) a.cent[i] = db.q.centroids[i];
  using Fn = void (*)(ScanArgs);
  static const Fn fns[4][2] = {{scan_kernel<1, false>, scan_kernel<1, true>},
                               {scan_kernel<2, false>, scan_kernel<2, true>},
                               {scan_kernel<3, false>, scan_kernel<3, true>},
                               {scan_kernel<4, false>, scan_kernel<4, true>}};
  const dim3 grid((unsigned)((N + kNB - 1) / kNB), (Q + kQB - 1) / kQB);
  hipLaunchKernelGGL(fns[a.B - 1][a.prod ? 1 : 0], grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace tqk
