// S R for the query side of the QJL term (riverfrot "TurboQuant" post,
// section 4.3: the query enters the sign estimator as S R q) and the largest
// row norm of S R, which bounds |(S R q)_c| by |q| for any query.
#include <math.h>

#include "internal.h"

namespace {

constexpr int kTile = 16;

// One 16 x 16 tile of SR = S R per workgroup, fp32 accumulation in k order.
__global__ __launch_bounds__(kTile * kTile) void fold_kernel(const float* __restrict__ S, const float* __restrict__ R,
                                                          int d, float* __restrict__ SR) {
  __shared__ float ts[kTile][kTile + 1], tr[kTile][kTile + 1];
  const int tx = threadIdx.x % kTile, ty = threadIdx.x / kTile;
  const int row = blockIdx.y * kTile + ty, col = blockIdx.x * kTile + tx;
  float acc = 0.f;
  for (int k0 = 0; k0 < d; k0 += kTile) {
    ts[ty][tx] = S[(int64_t)row * d + k0 + tx];
    tr[ty][tx] = R[(int64_t)(k0 + ty) * d + col];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kTile; ++k) acc = fmaf(ts[ty][k], tr[k][tx], acc);
    __syncthreads();
  }
  SR[(int64_t)row * d + col] = acc;
}

// The largest row norm of SR (one workgroup), stored after the matrix.
__global__ __launch_bounds__(256) void rownorm_kernel(float* __restrict__ SR, int d) {
  __shared__ float red[4];
  float best = 0.f;
  for (int r = threadIdx.x; r < d; r += 256) {
    double n2 = 0.0;
    for (int c = 0; c < d; ++c) {
      const double v = SR[(int64_t)r * d + c];
      n2 += v * v;
    }
    best = fmaxf(best, (float)sqrt(n2));
  }
  for (int o = 32; o >= 1; o >>= 1) best = fmaxf(best, __shfl_xor(best, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x < 4) {
    const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    // rounded up by one part in 2^20 so that it bounds the fp32 products
    SR[(int64_t)d * d + threadIdx.x] = threadIdx.x == 0 ? m * (1.f + 1.f / 1048576.f) : 0.f;
  }
}

}  // namespace

namespace tqk {

hipError_t launch_fold(const tq_quantizer& q, float* SR, hipStream_t s) {
  const int d = q.d;  // a multiple of 32, so whole 16 x 16 tiles
  hipLaunchKernelGGL(fold_kernel, dim3(d / kTile, d / kTile), dim3(kTile * kTile), 0, s, q.S, q.R, d, SR);
  hipLaunchKernelGGL(rownorm_kernel, dim3(1), dim3(256), 0, s, SR, d);
  return hipGetLastError();
}

}  // namespace tqk
