// Decode attention from the compressed cache on the gfx950 matrix cores.
//
// What is computed is the same as in decode.hip (riverfrot "TurboQuant" post,
// sections 2.2-2.4 and 4.3): per query head, scores
//   s_t = sum_groups n_t ( <R q, c[idx_t]> + gamma rho_t <S R q, 2 z_t - 1> ),
// an exact softmax over the cached tokens, and the weighted sum of the
// reconstructed values n_t R_v^T c_v[idx_t], accumulated in the rotated domain.
//
// How it is computed. The codebook is mirror-symmetric (c_i = -c_{L-1-i}),
// so with s_p = 2 b_p - 1 for the code bit-planes b_p its Walsh expansion has
// only odd-order terms: c[idx] = sum_{|S| odd} alpha_S prod_{p in S} s_p, and
// prod_{p in S} s_p = 2 (xor_{p in S} b_p) - 1. Every score term and every
// value sum is therefore a dot product of real weights with a +-1 vector
// whose bits are the packed planes (xor-combined). Those products run on the
// fp8 x fp4 MFMA (v_mfma_f32_16x16x128_f8f6f4):
//  * the +-1 vectors are fp4 e2m1 (nibble 0x2 = +1, 0xA = -1): a 32-bit plane
//    word becomes the 4-register operand with one shift and one bfi per
//    register;
//  * the real operand (query coefficients, softmax weights) is split into
//    four fp8 e4m3 digits v = d0 + d1 + d2 + d3 (each digit the fp8 rounding
//    of what the previous ones left), carried as four MFMA rows, and summed
//    after the product: about 16 significant bits, fp32 accumulation.
// Rows of every MFMA are (query head, digit) = 4 x 4; columns are 16 tokens
// (scores) or 16 value coordinates (value sums).
//
// Operand layouts used (measured on gfx950 for the mixed fp8 x fp4 form):
// fp4 operand lane l, nibble p (register p/8) -> k = 32 (l/16) + p; fp8
// operand lane l, byte p -> k = 16 (l/16) + (p % 16) + 64 (p / 16); D lane l
// register i -> row 4 (l/16) + i, column l % 16.
//
// One workgroup (4 waves) owns (split of the sequence, head tile of 4 query
// heads, batch x KV head) and walks 256-token chunks: each wave scores 64
// tokens, the chunk maximum is exchanged through LDS, each wave writes the
// fp8 digits of its weights to LDS, and each wave then accumulates 32 value
// coordinates over all 256 tokens. Partials (max, sum, rotated accumulator)
// go to the workspace; the combine kernel merges splits and applies R_v^T.
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kChunk = 256;
constexpr int kHT = 4;          // query heads per tile
constexpr int kD = 128;         // head channels handled by this kernel
constexpr int kMaxSlots = 12;   // K operand slots (group x sign type)
constexpr int kMaxVTypes = 8;
constexpr int kMaxKG = 2;
constexpr int kMaxVG = 4;

struct KGroup {
  const uint32_t* packed;
  const uint16_t* norm;
  const uint16_t* rnorm;
  const float* R;
  const float* S;
  int64_t seq_stride;
  int ch, d, B, prod;
  float gamma;
};

struct VGroup {
  const uint32_t* packed;
  const uint16_t* norm;
  const float* R;
  int64_t seq_stride;
  int ch, d, B, ntypes;
  int mask[kMaxVTypes];
  float alpha[kMaxVTypes];
};

struct Slot {
  int group;
  int mask;   // planes xor-combined into the +-1 vector
  int qjl;    // 0: accumulates the codebook part, 1: the QJL part
  float alpha;
};

struct Args {
  int nk, nv, nslots;
  KGroup k[kMaxKG];
  VGroup v[kMaxVG];
  Slot slot[kMaxSlots];
  const void* q;
  int qbf16;
  int B, Hq, Hkv, G, HT, T_max;
  const int32_t* seq_lens;
  float scale_log2;
  int splits, split_len;
  float* scores_out;
  uint32_t* aops;    // [keys][nslots][64 lanes][8 dwords]
  float* ascale;     // [keys][4 heads][kMaxKG groups][2]
  float* partial;    // [B * Hq][splits][kD + 2]
  float* out;
};

__device__ __forceinline__ uint32_t fp8_of(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.f, 0, false) & 0xffu;
}
__device__ __forceinline__ float f32_of_fp8(uint32_t b) { return __builtin_amdgcn_cvt_f32_fp8((int)b, 0); }

// Digit m (0..3) of the fp8 expansion of v.
__device__ uint32_t fp8_digit(float v, int m) {
  float r = v;
  uint32_t d = 0;
  for (int i = 0; i <= m; ++i) {
    d = fp8_of(r);
    r -= f32_of_fp8(d);
  }
  return d;
}

// Coordinate (within a 128-wide K block) fed to k-index kappa of the fp4
// operand built by expand_pm1: register r = (kappa % 32) / 8, nibble i =
// kappa % 8 takes bit 4 i + r of word kappa / 32.
__device__ __forceinline__ int coord_of_kappa(int kappa) {
  const int g = kappa >> 5, r = (kappa >> 3) & 3, i = kappa & 7;
  return 32 * g + 4 * i + r;
}

// fp8 operand: byte p of lane group gp holds k-index kappa.
__device__ __forceinline__ int kappa_of_fp8(int gp, int p) { return 16 * gp + (p & 15) + 64 * (p >> 4); }

// 32 plane bits -> 32 fp4 values +-1 (bit 1 -> +1) in four registers.
__device__ __forceinline__ v8i expand_pm1(uint32_t w) {
  v8i r;
  const uint32_t A = 0x22222222u, Bm = 0xAAAAAAAAu;
  uint32_t x0 = w << 3, x1 = w << 2, x2 = w << 1, x3 = w;
  r[0] = (int)((x0 & A) | (~x0 & Bm));
  r[1] = (int)((x1 & A) | (~x1 & Bm));
  r[2] = (int)((x2 & A) | (~x2 & Bm));
  r[3] = (int)((x3 & A) | (~x3 & Bm));
  r[4] = r[5] = r[6] = r[7] = 0;
  return r;
}

__device__ __forceinline__ v4f mfma_fp8_fp4(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, 0, 0, 0);
}

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 8, 64));
  v = fmaxf(v, __shfl_xor(v, 4, 64));
  v = fmaxf(v, __shfl_xor(v, 2, 64));
  v = fmaxf(v, __shfl_xor(v, 1, 64));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += __shfl_xor(v, 8, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 1, 64);
  return v;
}

__device__ __forceinline__ int exponent_of(float x) {
  int e;
  frexpf(x, &e);
  return x > 0.f ? e : -60;
}

// ------------------------------------------------------------------ qprep
// One workgroup per (batch, KV head, head tile): q~ = R q and q^ = S q~ per key
// group, then the fp8 digit operands of every slot.
__global__ __launch_bounds__(kThreads) void qprep_kernel(Args a) {
  __shared__ float qin[kHT][kD], qt[kHT][kD], qh[kHT][kD];
  __shared__ float smse[kHT][kMaxKG], sqjl[kHT][kMaxKG];
  const int key = blockIdx.x;
  const int b = key / (a.Hkv * a.HT);
  const int g = (key / a.HT) % a.Hkv;
  const int ht = key % a.HT;
  const int h0 = g * a.G + ht * kHT;
  const int nh = min(kHT, a.G - ht * kHT);
  const int tid = threadIdx.x;
  for (int e = tid; e < kHT * kD; e += kThreads) {
    const int h = e / kD, c = e % kD;
    qin[h][c] = h < nh ? tqd::load_elem(a.q, ((int64_t)b * a.Hq + h0 + h) * kD + c, a.qbf16) : 0.f;
    qh[h][c] = 0.f;
  }
  __syncthreads();
  for (int gi = 0; gi < a.nk; ++gi) {
    const KGroup& kg = a.k[gi];
    for (int e = tid; e < kHT * kg.d; e += kThreads) {
      const int h = e / kg.d, i = e % kg.d;
      float s = 0.f;
      for (int j = 0; j < kg.d; ++j) s = fmaf(kg.R[(int64_t)i * kg.d + j], qin[h][kg.ch + j], s);
      qt[h][kg.ch + i] = s;
    }
  }
  __syncthreads();
  for (int gi = 0; gi < a.nk; ++gi) {
    const KGroup& kg = a.k[gi];
    if (!kg.prod) continue;
    for (int e = tid; e < kHT * kg.d; e += kThreads) {
      const int h = e / kg.d, i = e % kg.d;
      float s = 0.f;
      for (int j = 0; j < kg.d; ++j) s = fmaf(kg.S[(int64_t)i * kg.d + j], qt[h][kg.ch + j], s);
      qh[h][kg.ch + i] = s;
    }
  }
  __syncthreads();
  // power-of-two scales that bring each (head, group) operand to at most 128
  if (tid < kHT * kMaxKG) {
    const int h = tid / kMaxKG, gi = tid % kMaxKG;
    float smx = 1.f, qmx = 1.f;
    if (gi < a.nk) {
      float amax = 0.f;
      for (int s = 0; s < a.nslots; ++s)
        if (a.slot[s].group == gi && !a.slot[s].qjl) amax = fmaxf(amax, fabsf(a.slot[s].alpha));
      float mt = 0.f, mh = 0.f;
      for (int c = a.k[gi].ch; c < a.k[gi].ch + a.k[gi].d; ++c) {
        mt = fmaxf(mt, fabsf(qt[h][c]));
        mh = fmaxf(mh, fabsf(qh[h][c]));
      }
      const float vm = mt * amax;
      smx = vm > 0.f ? ldexpf(1.f, 7 - exponent_of(vm)) : 1.f;
      qmx = mh > 0.f ? ldexpf(1.f, 7 - exponent_of(mh)) : 1.f;
    }
    smse[h][gi] = smx;
    sqjl[h][gi] = qmx;
    a.ascale[(((int64_t)key * kHT + h) * kMaxKG + gi) * 2 + 0] = 1.f / smx;
    a.ascale[(((int64_t)key * kHT + h) * kMaxKG + gi) * 2 + 1] = 1.f / qmx;
  }
  __syncthreads();
  for (int e = tid; e < a.nslots * 64 * 8; e += kThreads) {
    const int s = e / 512, L = (e / 8) % 64, dw = e % 8;
    const int r = L % 16, h = r / 4, m = r % 4, gp = L / 16;
    const Slot sl = a.slot[s];
    const KGroup& kg = a.k[sl.group];
    uint32_t word = 0;
    for (int bb = 0; bb < 4; ++bb) {
      const int c = coord_of_kappa(kappa_of_fp8(gp, dw * 4 + bb));
      float v = 0.f;
      if (h < nh && c >= kg.ch && c < kg.ch + kg.d)
        v = sl.qjl ? qh[h][c] * sqjl[h][sl.group] : sl.alpha * qt[h][c] * smse[h][sl.group];
      word |= fp8_digit(v, m) << (8 * bb);
    }
    a.aops[(((int64_t)key * a.nslots + s) * 64 + L) * 8 + dw] = word;
  }
}

// ------------------------------------------------------------------ decode
template <int NS, int VT, int NKG>
__global__ __launch_bounds__(kThreads) void decode_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) uint8_t wbuf[2][kMaxVG][2][16][128];  // fp8 weight digits [buf][vgroup][k-step][row][kappa]
  __shared__ float red_m[4][kHT];
  __shared__ int red_e[4][kMaxVG];
  __shared__ float fin_l[4][kHT];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hl = lane >> 4, tl = lane & 15;
  const int split = blockIdx.x, ht = blockIdx.y, bg = blockIdx.z;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int key = (b * a.Hkv + g) * a.HT + ht;
  const int h0 = g * a.G + ht * kHT;
  const int nh = min(kHT, a.G - ht * kHT);
  const int len = a.seq_lens ? min(max(a.seq_lens[b], 0), a.T_max) : a.T_max;
  const int ts = split * a.split_len;
  const int te = min(ts + a.split_len, len);

  // query operands of this head tile
  v8i aop[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (s < a.nslots) {
      const v4i* src = reinterpret_cast<const v4i*>(a.aops + (((int64_t)key * a.nslots + s) * 64 + lane) * 8);
      const v4i lo = src[0], hi = src[1];
      aop[s] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      aop[s] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  float inv_mse[NKG], inv_qjl[NKG];
#pragma unroll
  for (int gi = 0; gi < NKG; ++gi) {
    inv_mse[gi] = a.ascale[(((int64_t)key * kHT + hl) * kMaxKG + gi) * 2 + 0];
    inv_qjl[gi] = a.ascale[(((int64_t)key * kHT + hl) * kMaxKG + gi) * 2 + 1];
  }
  // this lane's coordinate word of the key layout (K-score B operand)
  const int W = lane >> 4;
  int kgi = 0;
#pragma unroll
  for (int gi = 1; gi < NKG; ++gi)
    if (gi < a.nk && 32 * W >= a.k[gi].ch) kgi = gi;
  const KGroup& kme = a.k[kgi];
  const int kGw = kme.d / 32, kwg = W - kme.ch / 32, kP = kme.B + kme.prod;
  // this wave's value coordinates: 32 w .. 32 w + 31, one value group
  int vgi = 0;
  for (int gi = 1; gi < a.nv; ++gi)
    if (32 * w >= a.v[gi].ch) vgi = gi;
  const VGroup& vme = a.v[vgi];
  const int vjl0 = 32 * w - vme.ch;  // first group-local coordinate of this wave

  v4f vacc[2][VT];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int s = 0; s < VT; ++s) vacc[tt][s] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  int e_run[kMaxVG];
#pragma unroll
  for (int gv = 0; gv < kMaxVG; ++gv) e_run[gv] = -60;

  int buf = 0;
  for (int c0 = ts; c0 < te; c0 += kChunk, buf ^= 1) {
    // ---------------- scores for this wave's 64 tokens
    float lg[4];
    float nvv[4][kMaxVG];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = c0 + 64 * w + 16 * i + tl;
      const bool valid = tok < te;
      uint32_t wds[5] = {0u, 0u, 0u, 0u, 0u};
      {
        const int tokl = c0 + 64 * w + 16 * i + (lane & 15);
        if (tokl < te) {
          const int64_t vi = (int64_t)bg * kme.seq_stride + tokl;
          const uint32_t* p = kme.packed + (((vi >> 4) * kGw + kwg) * 16 + (vi & 15)) * kP;
#pragma unroll
          for (int pp = 0; pp < 5; ++pp)
            if (pp < kP) wds[pp] = p[pp];
        }
      }
      v4f dm[NKG], dq[NKG];
#pragma unroll
      for (int gi = 0; gi < NKG; ++gi) dm[gi] = dq[gi] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s < a.nslots) {
          const Slot sl = a.slot[s];
          uint32_t word = 0;
#pragma unroll
          for (int pp = 0; pp < 5; ++pp)
            if ((sl.mask >> pp) & 1) word ^= wds[pp];
          const v8i bop = expand_pm1(word);
#pragma unroll
          for (int gi = 0; gi < NKG; ++gi) {
            if (sl.group == gi) {
              if (sl.qjl)
                dq[gi] = mfma_fp8_fp4(aop[s], bop, dq[gi]);
              else
                dm[gi] = mfma_fp8_fp4(aop[s], bop, dm[gi]);
            }
          }
        }
      }
      float sc = 0.f;
#pragma unroll
      for (int gi = 0; gi < NKG; ++gi) {
        if (gi < a.nk && valid) {
          const KGroup& kg = a.k[gi];
          const int64_t vi = (int64_t)bg * kg.seq_stride + tok;
          const float n = tqd::half_bits_to_f32(kg.norm[vi]);
          const float mse = (dm[gi][0] + dm[gi][1] + dm[gi][2] + dm[gi][3]) * inv_mse[gi];
          float part = mse;
          if (kg.prod) {
            const float rho = tqd::half_bits_to_f32(kg.rnorm[vi]);
            const float qjl = (dq[gi][0] + dq[gi][1] + dq[gi][2] + dq[gi][3]) * inv_qjl[gi];
            part = fmaf(kg.gamma * rho, qjl, mse);
          }
          sc = fmaf(n, part, sc);
        }
      }
      if (valid && hl < nh && a.scores_out) a.scores_out[((int64_t)b * a.Hq + h0 + hl) * a.T_max + tok] = sc;
      lg[i] = (valid && hl < nh) ? sc * a.scale_log2 : -INFINITY;
#pragma unroll
      for (int gv = 0; gv < kMaxVG; ++gv) {
        float nv = 0.f;
        if (gv < a.nv && valid) nv = tqd::half_bits_to_f32(a.v[gv].norm[(int64_t)bg * a.v[gv].seq_stride + tok]);
        nvv[i][gv] = nv;
      }
    }
    // ---------------- chunk statistics shared by the four waves
    float mx = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    mx = row16_max(mx);
    if (tl == 0) red_m[w][hl] = mx;
#pragma unroll
    for (int gv = 0; gv < kMaxVG; ++gv) {
      float vm = fmaxf(fmaxf(nvv[0][gv], nvv[1][gv]), fmaxf(nvv[2][gv], nvv[3][gv]));
      vm = tqd::wave_max(vm);
      if (lane == 0) red_e[w][gv] = exponent_of(vm);
    }
    __syncthreads();
    const float cm = fmaxf(fmaxf(red_m[0][hl], red_m[1][hl]), fmaxf(red_m[2][hl], red_m[3][hl]));
    const float m_new = fmaxf(m_run, cm);
    const bool live = m_new != -INFINITY;
    const float corr = (live && m_run != -INFINITY) ? exp2f(m_run - m_new) : (live ? 0.f : 1.f);
    int e_new[kMaxVG];
#pragma unroll
    for (int gv = 0; gv < kMaxVG; ++gv)
      e_new[gv] = max(max(max(red_e[0][gv], red_e[1][gv]), max(red_e[2][gv], red_e[3][gv])), e_run[gv]);
    // rescale this wave's value accumulators (softmax shift and weight scale)
    int eshift = 0;
#pragma unroll
    for (int gv = 0; gv < kMaxVG; ++gv)
      if (gv == vgi) eshift = e_run[gv] - e_new[gv];
    const float vcorr = corr * ldexpf(1.f, eshift);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int s = 0; s < VT; ++s) vacc[tt][s] *= vcorr;
    l_run *= corr;
    m_run = m_new;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = live ? exp2f(lg[i] - m_new) : 0.f;
      l_run += p[i];
    }
    // weights -> fp8 digits in LDS
#pragma unroll
    for (int gv = 0; gv < kMaxVG; ++gv) {
      if (gv >= a.nv) continue;
      const float sv = ldexpf(1.f, 7 - e_new[gv]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tau = 64 * w + 16 * i + tl;
        const int ks = tau >> 7, tp = tau & 127;
        const int kappa = 32 * (tp >> 5) + 8 * (tp & 3) + ((tp & 31) >> 2);
        float r = p[i] * nvv[i][gv] * sv;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t d = fp8_of(r);
          r -= f32_of_fp8(d);
          wbuf[buf][gv][ks][4 * hl + m][kappa] = (uint8_t)d;
        }
      }
      e_run[gv] = e_new[gv];
    }
#pragma unroll
    for (int gv = 0; gv < kMaxVG; ++gv)
      if (gv >= a.nv) e_run[gv] = e_new[gv];
    __syncthreads();
    // ---------------- values: this wave's 32 coordinates over the 256 tokens
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int tok0 = c0 + 128 * ks;
      if (tok0 >= te) break;
      const uint8_t* wrow = &wbuf[buf][vgi][ks][lane & 15][0];
      const int gp = lane >> 4;
      const v4i lo = *reinterpret_cast<const v4i*>(wrow + 16 * gp);
      const v4i hi = *reinterpret_cast<const v4i*>(wrow + 64 + 16 * gp);
      const v8i aw = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const int vP = vme.B;
      const int tblk = tok0 + 32 * gp;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        uint32_t wds[4] = {0u, 0u, 0u, 0u};
        if (tblk < te) {
          const int64_t vt = ((int64_t)bg * vme.seq_stride + tblk) >> 5;
          const int jl = vjl0 + 16 * tt + (lane & 15);
          const uint32_t* pw = vme.packed + (vt * vme.d + jl) * vP;
#pragma unroll
          for (int pp = 0; pp < 4; ++pp)
            if (pp < vP) wds[pp] = pw[pp];
        }
#pragma unroll
        for (int s = 0; s < VT; ++s) {
          if (s < vme.ntypes) {
            uint32_t word = 0;
#pragma unroll
            for (int pp = 0; pp < 4; ++pp)
              if ((vme.mask[s] >> pp) & 1) word ^= wds[pp];
            vacc[tt][s] = mfma_fp8_fp4(aw, expand_pm1(word), vacc[tt][s]);
          }
        }
      }
    }
  }

  // ---------------- partial results of this split
  float lsum = row16_sum(l_run);
  if (tl == 0) fin_l[w][hl] = lsum;
  __syncthreads();
  if (hl < nh) {
    float* part = a.partial + (((int64_t)b * a.Hq + h0 + hl) * a.splits + split) * (kD + 2);
    int efin = 0;
#pragma unroll
    for (int gv = 0; gv < kMaxVG; ++gv)
      if (gv == vgi) efin = e_run[gv];
    const float unscale = ldexpf(1.f, efin - 7);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float v = 0.f;
#pragma unroll
      for (int s = 0; s < VT; ++s)
        if (s < vme.ntypes)
          v = fmaf(vme.alpha[s], vacc[tt][s][0] + vacc[tt][s][1] + vacc[tt][s][2] + vacc[tt][s][3], v);
      part[2 + 32 * w + 16 * tt + tl] = v * unscale;
    }
    if (w == 0 && tl == 0) {
      part[0] = m_run;
      part[1] = fin_l[0][hl] + fin_l[1][hl] + fin_l[2][hl] + fin_l[3][hl];
    }
  }
}

// ------------------------------------------------------------------ combine
// One workgroup per (batch, query head): merge the split partials (log2
// domain) and rotate the value accumulator back with R_v^T.
__global__ __launch_bounds__(kThreads) void combine_kernel(Args a) {
  __shared__ float acc[kD];
  __shared__ float tot, mmax;
  const int bh = blockIdx.x, tid = threadIdx.x;
  const float* part = a.partial + (int64_t)bh * a.splits * (kD + 2);
  if (tid == 0) {
    float M = -INFINITY;
    for (int s = 0; s < a.splits; ++s) M = fmaxf(M, part[(int64_t)s * (kD + 2)]);
    mmax = M;
  }
  __syncthreads();
  const float M = mmax;
  if (tid <= kD) {
    float v = 0.f;
    if (M != -INFINITY) {
      for (int s = 0; s < a.splits; ++s) {
        const float ms = part[(int64_t)s * (kD + 2)];
        if (ms == -INFINITY) continue;
        v = fmaf(exp2f(ms - M), part[(int64_t)s * (kD + 2) + 1 + tid], v);
      }
    }
    if (tid == 0)
      tot = v;
    else
      acc[tid - 1] = v;
  }
  __syncthreads();
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  for (int gv = 0; gv < a.nv; ++gv) {
    const VGroup& vg = a.v[gv];
    for (int i = tid; i < vg.d; i += kThreads) {
      float s = 0.f;
      for (int j = 0; j < vg.d; ++j) s = fmaf(vg.R[(int64_t)j * vg.d + i], acc[vg.ch + j], s);
      a.out[(int64_t)bh * kD + vg.ch + i] = s * inv;
    }
  }
}

// Walsh coefficients of a mirror-symmetric codebook: c[idx] =
// sum_{|S| odd} alpha_S prod_{p in S} (2 bit_p(idx) - 1).
int odd_walsh(const tq_quantizer& q, int* masks, float* alphas) {
  const int B = q.mse_bits, L = 1 << B;
  int n = 0;
  for (int S = 1; S < L; ++S) {
    if (!(__builtin_popcount(S) & 1)) continue;
    double acc = 0.0;
    for (int idx = 0; idx < L; ++idx) {
      double chi = 1.0;
      for (int p = 0; p < B; ++p)
        if ((S >> p) & 1) chi *= ((idx >> p) & 1) ? 1.0 : -1.0;
      acc += chi * (double)q.centroids[idx];
    }
    masks[n] = S;
    alphas[n] = (float)(acc / L);
    ++n;
  }
  return n;
}

template <int NS, int VT, int NKG>
void launch_kernel(const Args& a, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((decode_kernel<NS, VT, NKG>), grid, dim3(kThreads), 0, s, a);
}

}  // namespace

namespace tqk {

bool mfma_decode_supported(const tq_kv_desc& k, const tq_kv_desc& v) {
  int D = 0, Dv = 0, slots = 0, vt = 0;
  for (int i = 0; i < k.n_groups; ++i) {
    D += k.g[i].q.d;
    slots += (1 << (k.g[i].q.mse_bits - 1)) + (k.g[i].q.variant == TQ_PROD ? 1 : 0);
  }
  for (int i = 0; i < v.n_groups; ++i) {
    Dv += v.g[i].q.d;
    vt = vt > (1 << (v.g[i].q.mse_bits - 1)) ? vt : (1 << (v.g[i].q.mse_bits - 1));
  }
  return D == kD && Dv == kD && k.n_groups <= kMaxKG && v.n_groups <= kMaxVG && slots <= kMaxSlots &&
         vt <= kMaxVTypes;
}

DecodePlan plan_decode_mfma(const tq_kv_desc& k, const tq_kv_desc& v, int B, int Hq, int Hkv, int T_max) {
  DecodePlan p{};
  const int G = Hq / Hkv;
  const int HT = (G + kHT - 1) / kHT;
  int slots = 0;
  for (int i = 0; i < k.n_groups; ++i)
    slots += (1 << (k.g[i].q.mse_bits - 1)) + (k.g[i].q.variant == TQ_PROD ? 1 : 0);
  const int64_t wgs_per_split = (int64_t)B * Hkv * HT;
  int64_t splits = (1024 + wgs_per_split - 1) / wgs_per_split;
  int64_t sl = (T_max + splits - 1) / splits;
  sl = (sl + kChunk - 1) / kChunk * kChunk;
  p.split_len = (int)sl;
  p.splits = (int)((T_max + sl - 1) / sl);
  p.head_chunk = kHT;
  p.n_chunks = HT;
  p.D = kD;
  p.Dv = kD;
  const size_t keys = (size_t)B * Hkv * HT;
  p.qprep_floats = keys * slots * 64 * 8 + keys * kHT * kMaxKG * 2;
  p.partial_floats = (size_t)B * Hq * p.splits * (kD + 2);
  return p;
}

hipError_t launch_decode_mfma(const tq_kv_desc& k, const tq_kv_desc& v, const void* q, tq_dtype qdt, int B, int Hq,
                              int Hkv, int T_max, const int32_t* seq_lens, float scale, float* out,
                              float* scores_out, void* ws, const DecodePlan& plan, hipStream_t s) {
  Args a{};
  a.nk = k.n_groups;
  a.nv = v.n_groups;
  int ns = 0, vtmax = 0;
  for (int gi = 0; gi < a.nk; ++gi) {
    const tq_group& g = k.g[gi];
    KGroup& o = a.k[gi];
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
    int masks[kMaxVTypes];
    float alphas[kMaxVTypes];
    const int nt = odd_walsh(g.q, masks, alphas);
    for (int t = 0; t < nt; ++t) a.slot[ns++] = Slot{gi, masks[t], 0, alphas[t]};
    if (o.prod) a.slot[ns++] = Slot{gi, 1 << o.B, 1, 1.f};
  }
  a.nslots = ns;
  for (int gi = 0; gi < a.nv; ++gi) {
    const tq_group& g = v.g[gi];
    VGroup& o = a.v[gi];
    o.packed = static_cast<const uint32_t*>(g.packed);
    o.norm = g.norm;
    o.R = g.q.R;
    o.seq_stride = g.seq_stride;
    o.ch = g.ch_offset;
    o.d = g.q.d;
    o.B = g.q.mse_bits;
    o.ntypes = odd_walsh(g.q, o.mask, o.alpha);
    vtmax = vtmax > o.ntypes ? vtmax : o.ntypes;
  }
  a.q = q;
  a.qbf16 = qdt == TQ_BF16;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.HT = plan.n_chunks;
  a.T_max = T_max;
  a.seq_lens = seq_lens;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.splits = plan.splits;
  a.split_len = plan.split_len;
  a.scores_out = scores_out;
  const size_t keys = (size_t)B * Hkv * a.HT;
  a.aops = static_cast<uint32_t*>(ws);
  a.ascale = reinterpret_cast<float*>(a.aops + keys * ns * 64 * 8);
  a.partial = static_cast<float*>(ws) + plan.qprep_floats;
  a.out = out;
  hipLaunchKernelGGL(qprep_kernel, dim3((unsigned)keys), dim3(kThreads), 0, s, a);
  const dim3 grid(plan.splits, a.HT, B * Hkv);
  const bool two = a.nk > 1;
  if (ns <= 6) {
    if (vtmax <= 4) {
      if (two) launch_kernel<6, 4, 2>(a, grid, s); else launch_kernel<6, 4, 1>(a, grid, s);
    } else {
      if (two) launch_kernel<6, 8, 2>(a, grid, s); else launch_kernel<6, 8, 1>(a, grid, s);
    }
  } else {
    if (vtmax <= 4) {
      if (two) launch_kernel<12, 4, 2>(a, grid, s); else launch_kernel<12, 4, 1>(a, grid, s);
    } else {
      if (two) launch_kernel<12, 8, 2>(a, grid, s); else launch_kernel<12, 8, 1>(a, grid, s);
    }
  }
  hipLaunchKernelGGL(combine_kernel, dim3(B * Hq), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace tqk
