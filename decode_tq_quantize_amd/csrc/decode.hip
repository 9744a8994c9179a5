// Decode attention straight from the compressed KV cache (gfx950).
//
// riverfrot "TurboQuant" post, sections 2.2-2.3: the new token's query
// attends to every cached key, softmax(q K^T / sqrt(d)), and the weights
// average the cached values; section 4.3: the key scores come from the
// unbiased estimator with the query unquantised,
//   s_t = n_t ( <R q, c[idx_t]> + gamma rho_t <S R q, 2 z_t - 1> ),
// and GQA (section 2.4) lets one KV head serve a group of query heads.
//
// Values are accumulated in their rotated domain: since v^_t = n_t R^T
// c[idx_t], sum_t p_t v^_t = R^T (sum_t p_t n_t c[idx_t]); the inverse
// rotation is applied once per (batch, head) in the combine kernel.
//
// Kernels:
//  qprep    q~ = R q and q^ = S q~ per key group for every (batch, head)
//  decode   one workgroup per (split, head chunk, batch * KV head); each wave
//           streams 64-token chunks: lane = token for the scores, an online
//           softmax per head, lane = coordinate for the value accumulation;
//           the four waves' (max, sum, acc) are merged into one partial.
//  combine  merges the split partials and applies R_v^T and 1 / sum.
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 64;       // tokens per wave step
constexpr int kMaxHC = 8;        // query heads per workgroup
constexpr int kMaxD = 256;       // key / value channels
constexpr int kMaxDPerLane = kMaxD / tqd::kWave;

struct GroupArgs {
  const uint32_t* packed;
  const uint16_t* norm;
  const uint16_t* rnorm;
  const float* R;
  const float* S;
  int64_t seq_stride;
  int ch;
  int d;
  int B;
  int prod;
  float gamma;
  float cent[TQ_MAX_LEVELS];
};

struct DecArgs {
  int nk, nv;
  GroupArgs k[TQ_MAX_GROUPS];
  GroupArgs v[TQ_MAX_GROUPS];
  const void* q;
  int qbf16;
  int B, Hq, Hkv, T_max, D, Dv;
  int HC, n_chunks, splits, split_len;
  const int32_t* seq_lens;
  float scale;
  float* out;
  float* scores_out;
  float* qprep;     // [B, Hq, 2 D]: q~ then q^ (zeros for MSE key groups)
  float* partial;   // [B, Hq, splits, Dv + 2]: m, l, acc
};

// ---------------------------------------------------------------- qprep
__global__ __launch_bounds__(kThreads) void qprep_kernel(DecArgs a) {
  __shared__ float qin[kMaxD];
  __shared__ float qt[kMaxD];
  const int bh = blockIdx.x;  // b * Hq + h
  const int tid = threadIdx.x;
  for (int j = tid; j < a.D; j += kThreads) qin[j] = tqd::load_elem(a.q, (int64_t)bh * a.D + j, a.qbf16);
  __syncthreads();
  float* dst = a.qprep + (int64_t)bh * 2 * a.D;
  for (int gi = 0; gi < a.nk; ++gi) {
    const GroupArgs& g = a.k[gi];
    for (int i = tid; i < g.d; i += kThreads) {
      float s = 0.f;
      for (int j = 0; j < g.d; ++j) s = fmaf(g.R[(int64_t)i * g.d + j], qin[g.ch + j], s);
      qt[g.ch + i] = s;
      dst[g.ch + i] = s;
    }
    __syncthreads();
    for (int i = tid; i < g.d; i += kThreads) {
      float s = 0.f;
      if (g.prod)
        for (int j = 0; j < g.d; ++j) s = fmaf(g.S[(int64_t)i * g.d + j], qt[g.ch + j], s);
      dst[a.D + g.ch + i] = s;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- decode
__global__ __launch_bounds__(kThreads) void decode_kernel(DecArgs a) {
  __shared__ float sq[kMaxHC][2 * kMaxD];           // q~ | q^ per head of the chunk
  __shared__ float kcent[TQ_MAX_GROUPS][TQ_MAX_LEVELS];
  __shared__ float vcent[TQ_MAX_GROUPS][TQ_MAX_LEVELS];
  __shared__ float pbuf[4][kMaxHC][kChunk];          // softmax weights, per wave
  __shared__ float nvbuf[4][TQ_MAX_GROUPS][kChunk];  // value norms, per wave
  __shared__ float wm[4][kMaxHC], wl[4][kMaxHC];
  __shared__ float wacc[4][kMaxHC][kMaxD];

  const int tid = threadIdx.x, lane = tid % tqd::kWave, wv = tid / tqd::kWave;
  const int split = blockIdx.x;
  const int chunk = blockIdx.y;
  const int bg = blockIdx.z;  // b * Hkv + g
  const int b = bg / a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int h0 = (bg % a.Hkv) * G + chunk * a.HC;
  const int HC = min(a.HC, G - chunk * a.HC);
  const int len = a.seq_lens ? min(max(a.seq_lens[b], 0), a.T_max) : a.T_max;
  const int ts = split * a.split_len;
  const int te = min(ts + a.split_len, len);

  for (int e = tid; e < HC * 2 * a.D; e += kThreads) {
    const int h = e / (2 * a.D), j = e % (2 * a.D);
    sq[h][j] = a.qprep[((int64_t)b * a.Hq + h0 + h) * 2 * a.D + j];
  }
  if (tid < TQ_MAX_GROUPS * TQ_MAX_LEVELS) {
    const int gi = tid / TQ_MAX_LEVELS, l = tid % TQ_MAX_LEVELS;
    kcent[gi][l] = gi < a.nk ? a.k[gi].cent[l] : 0.f;
    vcent[gi][l] = gi < a.nv ? a.v[gi].cent[l] : 0.f;
  }
  __syncthreads();

  float m[kMaxHC], l[kMaxHC], acc[kMaxHC][kMaxDPerLane];
#pragma unroll
  for (int h = 0; h < kMaxHC; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int r = 0; r < kMaxDPerLane; ++r) acc[h][r] = 0.f;
  }

  for (int c0 = ts + wv * kChunk; c0 < te; c0 += 4 * kChunk) {
    // ---- scores: lane = token
    const int t = c0 + lane;
    const bool valid = t < te;
    float s[kMaxHC];
#pragma unroll
    for (int h = 0; h < kMaxHC; ++h) s[h] = 0.f;
    if (valid) {
      for (int gi = 0; gi < a.nk; ++gi) {
        const GroupArgs& g = a.k[gi];
        const int64_t vi = (int64_t)bg * g.seq_stride + t;
        const int64_t tile = vi / tqk::kKeysTile;
        const int tt = (int)(vi % tqk::kKeysTile);
        const int P = g.B + g.prod;
        const int Gw = g.d / 32;
        float mse[kMaxHC], qjl[kMaxHC];
#pragma unroll
        for (int h = 0; h < kMaxHC; ++h) mse[h] = qjl[h] = 0.f;
        for (int gw = 0; gw < Gw; ++gw) {
          const uint32_t* wp = g.packed + ((tile * Gw + gw) * tqk::kKeysTile + tt) * P;
          uint32_t w[TQ_MAX_MSE_BITS];
#pragma unroll
          for (int p = 0; p < TQ_MAX_MSE_BITS; ++p) w[p] = p < g.B ? wp[p] : 0u;
          const uint32_t wz = g.prod ? wp[g.B] : 0u;
          for (int i = 0; i < 32; ++i) {
            int idx = 0;
#pragma unroll
            for (int p = 0; p < TQ_MAX_MSE_BITS; ++p)
              if (p < g.B) idx |= (int)((w[p] >> i) & 1u) << p;
            const float cv = kcent[gi][idx];
            const float sg = ((wz >> i) & 1u) ? 1.f : -1.f;
            const int j = g.ch + 32 * gw + i;
#pragma unroll
            for (int h = 0; h < kMaxHC; ++h) {
              if (h < HC) {
                mse[h] = fmaf(sq[h][j], cv, mse[h]);
                qjl[h] = fmaf(sq[h][a.D + j], sg, qjl[h]);
              }
            }
          }
        }
        const float n = tqd::half_bits_to_f32(g.norm[vi]);
        const float rho = g.prod ? tqd::half_bits_to_f32(g.rnorm[vi]) : 0.f;
#pragma unroll
        for (int h = 0; h < kMaxHC; ++h) s[h] += n * (mse[h] + (g.prod ? g.gamma * rho * qjl[h] : 0.f));
      }
      if (a.scores_out) {
        for (int h = 0; h < HC; ++h) a.scores_out[((int64_t)b * a.Hq + h0 + h) * a.T_max + t] = s[h];
      }
    }
    // ---- online softmax per head (wave-wide)
#pragma unroll
    for (int h = 0; h < kMaxHC; ++h) {
      if (h >= HC) continue;
      const float logit = valid ? a.scale * s[h] : -INFINITY;
      const float mx = tqd::wave_max(logit);
      const float mnew = fmaxf(m[h], mx);
      const float p = valid ? __expf(logit - mnew) : 0.f;
      const float corr = m[h] == -INFINITY ? 0.f : __expf(m[h] - mnew);
      l[h] = l[h] * corr + tqd::wave_sum(p);
      m[h] = mnew;
#pragma unroll
      for (int r = 0; r < kMaxDPerLane; ++r) acc[h][r] *= corr;
      pbuf[wv][h][lane] = p;
    }
    // ---- value accumulation: lane = coordinate (rotated domain)
    for (int gi = 0; gi < a.nv; ++gi) {
      const int64_t vbase = (int64_t)bg * a.v[gi].seq_stride + c0;
      nvbuf[wv][gi][lane] = c0 + lane < te ? tqd::half_bits_to_f32(a.v[gi].norm[vbase + lane]) : 0.f;
    }
    __builtin_amdgcn_wave_barrier();
    const int ntok = min(kChunk, te - c0);
#pragma unroll
    for (int r = 0; r < kMaxDPerLane; ++r) {
      const int j = lane + r * tqd::kWave;  // value channel of register slot r
      if (j >= a.Dv) continue;
      int gi = 0;
      while (gi + 1 < a.nv && j >= a.v[gi + 1].ch) ++gi;
      const GroupArgs& g = a.v[gi];
      const int jl = j - g.ch;
      const int P = g.B;
      // the chunk is one 64-vector block of the value layout (chunks start
      // at multiples of 64): two tiles whose words interleave its tokens
      const int64_t tile0 = ((int64_t)bg * g.seq_stride + c0) / tqk::kValuesBlock * 2;
      for (int half = 0; half < 2; ++half) {
        const uint32_t* wp = g.packed + ((tile0 + half) * g.d + jl) * P;
        uint32_t w[TQ_MAX_MSE_BITS];
#pragma unroll
        for (int p = 0; p < TQ_MAX_MSE_BITS; ++p) w[p] = p < P ? wp[p] : 0u;
        for (int i = 0; i < 32; ++i) {
          const int tl = tqk::value_tok(half, i);
          if (tl >= ntok) continue;
          int idx = 0;
#pragma unroll
          for (int p = 0; p < TQ_MAX_MSE_BITS; ++p)
            if (p < P) idx |= (int)((w[p] >> i) & 1u) << p;
          const float val = vcent[gi][idx] * nvbuf[wv][gi][tl];
#pragma unroll
          for (int h = 0; h < kMaxHC; ++h)
            if (h < HC) acc[h][r] = fmaf(pbuf[wv][h][tl], val, acc[h][r]);
        }
      }
    }
  }

  // ---- merge the four waves
#pragma unroll
  for (int h = 0; h < kMaxHC; ++h) {
    if (h >= HC) continue;
    if (lane == 0) {
      wm[wv][h] = m[h];
      wl[wv][h] = l[h];
    }
#pragma unroll
    for (int r = 0; r < kMaxDPerLane; ++r) {
      const int j = lane + r * tqd::kWave;
      if (j < a.Dv) wacc[wv][h][j] = acc[h][r];
    }
  }
  __syncthreads();
  for (int e = tid; e < HC * (a.Dv + 2); e += kThreads) {
    const int h = e / (a.Dv + 2), c = e % (a.Dv + 2);
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][h]);
    float val = 0.f;
    if (c == 0) {
      val = M;
    } else {
      for (int w = 0; w < 4; ++w) {
        const float f = wm[w][h] == -INFINITY ? 0.f : __expf(wm[w][h] - M);
        val += f * (c == 1 ? wl[w][h] : wacc[w][h][c - 2]);
      }
    }
    a.partial[(((int64_t)b * a.Hq + h0 + h) * a.splits + split) * (a.Dv + 2) + c] = val;
  }
}

// ---------------------------------------------------------------- combine
__global__ __launch_bounds__(kThreads) void combine_kernel(DecArgs a) {
  __shared__ float acc[kMaxD];
  __shared__ float tot;
  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const float* part = a.partial + (int64_t)bh * a.splits * (a.Dv + 2);
  float M = -INFINITY;
  for (int sp = 0; sp < a.splits; ++sp) M = fmaxf(M, part[sp * (a.Dv + 2)]);
  for (int c = tid; c < a.Dv + 1; c += kThreads) {
    float v = 0.f;
    for (int sp = 0; sp < a.splits; ++sp) {
      const float ms = part[sp * (a.Dv + 2)];
      const float f = ms == -INFINITY ? 0.f : __expf(ms - M);
      v = fmaf(f, part[sp * (a.Dv + 2) + 1 + c], v);
    }
    if (c == 0)
      tot = v;
    else
      acc[c - 1] = v;
  }
  __syncthreads();
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  for (int gi = 0; gi < a.nv; ++gi) {
    const GroupArgs& g = a.v[gi];
    for (int i = tid; i < g.d; i += kThreads) {
      float s = 0.f;
      for (int j = 0; j < g.d; ++j) s = fmaf(g.R[(int64_t)j * g.d + i], acc[g.ch + j], s);
      a.out[(int64_t)bh * a.Dv + g.ch + i] = s * inv;
    }
  }
}

void fill_group(GroupArgs& o, const tq_group& g) {
  o.packed = static_cast<const uint32_t*>(g.packed);
  o.norm = g.norm;
  o.rnorm = g.rnorm;
  o.R = g.q.R;
  o.S = g.q.S;
  o.seq_stride = g.seq_stride;
  o.ch = g.ch_offset;
  o.d = g.q.d;
  o.B = g.q.mse_bits;
  o.prod = g.q.variant == TQ_PROD;
  o.gamma = (float)(sqrt(M_PI / 2.0) / g.q.d);
  for (int i = 0; i < TQ_MAX_LEVELS; ++i) o.cent[i] = g.q.centroids[i];
}

}  // namespace

namespace tqk {

DecodePlan plan_decode(const tq_kv_desc& k, const tq_kv_desc& v, int B, int Hq, int Hkv, int T_max) {
  DecodePlan p{};
  int D = 0, Dv = 0;
  for (int i = 0; i < k.n_groups; ++i) D += k.g[i].q.d;
  for (int i = 0; i < v.n_groups; ++i) Dv += v.g[i].q.d;
  const int G = Hq / Hkv;
  p.head_chunk = G < kMaxHC ? G : kMaxHC;
  p.n_chunks = (G + p.head_chunk - 1) / p.head_chunk;
  const int64_t wgs_per_split = (int64_t)B * Hkv * p.n_chunks;
  int64_t splits = (2048 + wgs_per_split - 1) / wgs_per_split;
  if (splits < 1) splits = 1;
  int64_t sl = (T_max + splits - 1) / splits;
  sl = (sl + 255) / 256 * 256;
  if (sl < 256) sl = 256;
  p.split_len = (int)sl;
  p.splits = (int)((T_max + sl - 1) / sl);
  if (p.splits < 1) p.splits = 1;
  p.D = D;
  p.Dv = Dv;
  p.qprep_floats = (size_t)B * Hq * 2 * D;
  p.partial_floats = (size_t)B * Hq * p.splits * (Dv + 2);
  return p;
}

hipError_t launch_decode(const tq_kv_desc& k, const tq_kv_desc& v, const void* q, tq_dtype qdt, int B, int Hq,
                         int Hkv, int T_max, const int32_t* seq_lens, float scale, float* out, float* scores_out,
                         void* ws, const DecodePlan& plan, hipStream_t s) {
  DecArgs a{};
  a.nk = k.n_groups;
  a.nv = v.n_groups;
  for (int i = 0; i < a.nk; ++i) fill_group(a.k[i], k.g[i]);
  for (int i = 0; i < a.nv; ++i) fill_group(a.v[i], v.g[i]);
  a.q = q;
  a.qbf16 = qdt == TQ_BF16;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.T_max = T_max;
  a.D = plan.D;
  a.Dv = plan.Dv;
  a.HC = plan.head_chunk;
  a.n_chunks = plan.n_chunks;
  a.splits = plan.splits;
  a.split_len = plan.split_len;
  a.seq_lens = seq_lens;
  a.scale = scale;
  a.out = out;
  a.scores_out = scores_out;
  a.qprep = static_cast<float*>(ws);
  a.partial = a.qprep + plan.qprep_floats;
  hipLaunchKernelGGL(qprep_kernel, dim3(B * Hq), dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL(decode_kernel, dim3(plan.splits, plan.n_chunks, B * Hkv), dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL(combine_kernel, dim3(B * Hq), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace tqk
