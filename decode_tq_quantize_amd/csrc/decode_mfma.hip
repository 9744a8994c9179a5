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
//  * a 32-bit plane word w becomes four fp4 registers, register r taking bit
//    4 i + r of w into nibble i with one bit operation: r = 3 gives +-1
//    (bit select), r = 2, 1, 0 give {0, 2}, {0, 1}, {0, 1/2} (masks), i.e.
//    u_r + v_r sigma with (u, v) = (0, 1), (1, 1), (1/2, 1/2), (1/4, 1/4);
//    the real operand is pre-multiplied by 1 / v_r (a power of two) and the
//    constant part sum a u_r is removed exactly with one more MFMA against
//    the constant operand 4 u_r;
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
// Kernels: qprep builds the query operands of every (batch, KV head, head
// tile) (q~ = R q, q^ = S q~, power-of-two scales, fp8 digits); decode runs
// one workgroup (4 waves) per (split of the sequence, head tile of 4 query
// heads, batch x KV head) over 256-token chunks: each wave scores 64 tokens,
// the chunk maximum is exchanged through LDS, each wave writes the fp8 digits
// of its weights to LDS, and each wave accumulates 32 value coordinates over
// the 256 tokens; the next chunk's key planes and norms are prefetched during
// the current chunk. Partials (max, sum, rotated accumulator) go to the
// workspace; combine merges the splits and applies R_v^T.
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
constexpr int kMaxSlots = 12;   // key operand slots (group x sign type)
constexpr int kMaxVTypes = 8;
constexpr int kMaxKG = 2;
constexpr int kMaxVG = 2;
constexpr int kMaxCombineSplits = 4096;
constexpr int kCombThreads = 256;

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
  float alpha[kMaxVTypes];
  float alpha_sum;
};

struct Slot {
  int group;
  int qjl;    // 0: codebook part, 1: QJL part
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
  uint32_t* aops;    // [keys][nslots][64 lanes][8 dwords] query operands
  float* ascale;     // [keys][4 heads][kMaxKG][2] inverse operand scales
  float* partial;    // [B * Hq][splits][kD + 2]
  float* out;
};

__device__ __forceinline__ uint32_t fp8_of(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.f, 0, false) & 0xffu;
}
__device__ __forceinline__ float f32_of_fp8(uint32_t b) { return __builtin_amdgcn_cvt_f32_fp8((int)b, 0); }

// 32 plane bits -> fp4 operand; register r, nibble i <- bit 4 i + r.
__device__ __forceinline__ v8i expand_bits(uint32_t w) {
  v8i r;
  r[0] = (int)(w & 0x11111111u);                               // {0, 1/2}
  r[1] = (int)(w & 0x22222222u);                               // {0, 1}
  r[2] = (int)(w & 0x44444444u);                               // {0, 2}
  r[3] = (int)((w & 0x22222222u) | (~w & 0xAAAAAAAAu));        // {-1, +1}
  r[4] = r[5] = r[6] = r[7] = 0;
  return r;
}

// The constant operand 4 u_r (nibble values 1, 2, 4, 0 in registers 0..3).
__device__ __forceinline__ v8i const_operand() {
  return v8i{0x22222222, 0x44444444, 0x66666666, 0, 0, 0, 0, 0};
}

// 1 / v_r for register r of the fp4 operand.
__device__ __forceinline__ float inv_v(int r) { return r == 0 ? 4.f : (r == 1 ? 2.f : 1.f); }

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

__device__ __forceinline__ float sum4(v4f x) { return (x[0] + x[1]) + (x[2] + x[3]); }

// Odd subsets of B code planes, in ascending bitmask order (the host orders
// the Walsh coefficients the same way).
__host__ __device__ constexpr int n_odd(int B) { return B > 0 ? 1 << (B - 1) : 0; }
__host__ __device__ constexpr int odd_mask(int B, int t) {
  int n = 0;
  for (int S = 1; S < (1 << B); ++S) {
    int pc = 0;
    for (int x = S; x; x >>= 1) pc += x & 1;
    if (pc & 1) {
      if (n == t) return S;
      ++n;
    }
  }
  return 0;
}

// ------------------------------------------------------------------ qprep
// One workgroup per (batch, KV head, head tile, slot). Every workgroup of a
// tile recomputes q~ = R q and q^ = S q~ for the tile's 4 heads (both
// matrices are read in one round of loads, before the query is needed) and
// writes the fp8 digit operand of its own slot; slot 0 also writes the
// inverse scales. Lane (row lane/4, quarter lane%4) of wave w owns rows
// 16 w + lane/4 and 64 + 16 w + lane/4 of a 128 x 128 matrix (d <= 128).
constexpr int kPrepThreads = 256;

__device__ __forceinline__ void load_rows(const float* __restrict__ M, int d, float4 (&reg)[2][8]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int rr = lane >> 2, qtr = lane & 3, span = d >> 2;
#pragma unroll
  for (int ps = 0; ps < 2; ++ps) {
    const int i = 64 * ps + 16 * wv + rr;
#pragma unroll
    for (int j4 = 0; j4 < 8; ++j4) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i < d && 4 * j4 < span) v = reinterpret_cast<const float4*>(M + (int64_t)i * d + qtr * span)[j4];
      reg[ps][j4] = v;
    }
  }
}

__device__ __forceinline__ void matvec_regs(const float4 (&reg)[2][8], int d, int ch, const float (*in)[kD],
                                            float (*out)[kD]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int rr = lane >> 2, qtr = lane & 3, span = d >> 2;
#pragma unroll
  for (int ps = 0; ps < 2; ++ps) {
    const int i = 64 * ps + 16 * wv + rr;
    float acc[kHT] = {0.f, 0.f, 0.f, 0.f};
    const int j0 = ch + qtr * span;
#pragma unroll
    for (int j4 = 0; j4 < 8; ++j4) {
      if (4 * j4 < span) {
        const float4 m4 = reg[ps][j4];
#pragma unroll
        for (int h = 0; h < kHT; ++h) {
          const float4 x = *reinterpret_cast<const float4*>(&in[h][j0 + 4 * j4]);
          acc[h] = fmaf(m4.x, x.x, acc[h]);
          acc[h] = fmaf(m4.y, x.y, acc[h]);
          acc[h] = fmaf(m4.z, x.z, acc[h]);
          acc[h] = fmaf(m4.w, x.w, acc[h]);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < kHT; ++h) {
      acc[h] += __shfl_xor(acc[h], 1, 64);
      acc[h] += __shfl_xor(acc[h], 2, 64);
    }
    if (i < d && qtr == 0) {
#pragma unroll
      for (int h = 0; h < kHT; ++h) out[h][ch + i] = acc[h];
    }
  }
}

__global__ __launch_bounds__(kPrepThreads) void qprep_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) float qin[kHT][kD];
  __shared__ __attribute__((aligned(16))) float qt[kHT][kD];
  __shared__ __attribute__((aligned(16))) float qh[kHT][kD];
  __shared__ float smse[kHT][kMaxKG], sqjl[kHT][kMaxKG];
  __shared__ __attribute__((aligned(16))) uint8_t opb[64][32];
  const int key = blockIdx.x, slot = blockIdx.y;
  const int b = key / (a.Hkv * a.HT);
  const int g = (key / a.HT) % a.Hkv;
  const int ht = key % a.HT;
  const int h0 = g * a.G + ht * kHT;
  const int nh = min(kHT, a.G - ht * kHT);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  float4 regR[kMaxKG][2][8], regS[kMaxKG][2][8];
#pragma unroll
  for (int gi = 0; gi < kMaxKG; ++gi) {
    if (gi < a.nk) {
      load_rows(a.k[gi].R, a.k[gi].d, regR[gi]);
      if (a.k[gi].prod) load_rows(a.k[gi].S, a.k[gi].d, regS[gi]);
    }
  }
  for (int e = tid; e < kHT * kD; e += kPrepThreads) {
    const int h = e / kD, c = e % kD;
    qin[h][c] = h < nh ? tqd::load_elem(a.q, ((int64_t)b * a.Hq + h0 + h) * kD + c, a.qbf16) : 0.f;
    qh[h][c] = 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int gi = 0; gi < kMaxKG; ++gi)
    if (gi < a.nk) matvec_regs(regR[gi], a.k[gi].d, a.k[gi].ch, qin, qt);
  __syncthreads();
#pragma unroll
  for (int gi = 0; gi < kMaxKG; ++gi)
    if (gi < a.nk && a.k[gi].prod) matvec_regs(regS[gi], a.k[gi].d, a.k[gi].ch, qt, qh);
  __syncthreads();
  // power-of-two scales bringing each (head, group) operand below 32 (the
  // fp4 encoding multiplies it by up to 4); wave w handles head w
  for (int gi = 0; gi < a.nk; ++gi) {
    float amax = 0.f;
    for (int s = 0; s < a.nslots; ++s)
      if (a.slot[s].group == gi && !a.slot[s].qjl) amax = fmaxf(amax, fabsf(a.slot[s].alpha));
    float mt = 0.f, mh = 0.f;
    for (int c = a.k[gi].ch + lane; c < a.k[gi].ch + a.k[gi].d; c += 64) {
      mt = fmaxf(mt, fabsf(qt[wv][c]));
      mh = fmaxf(mh, fabsf(qh[wv][c]));
    }
    mt = tqd::wave_max(mt) * amax;
    mh = tqd::wave_max(mh);
    if (lane == 0) {
      const float sm = mt > 0.f ? ldexpf(1.f, 5 - exponent_of(mt)) : 1.f;
      const float sq = mh > 0.f ? ldexpf(1.f, 5 - exponent_of(mh)) : 1.f;
      smse[wv][gi] = sm;
      sqjl[wv][gi] = sq;
      if (slot == 0) {
        a.ascale[(((int64_t)key * kHT + wv) * kMaxKG + gi) * 2 + 0] = 1.f / sm;
        a.ascale[(((int64_t)key * kHT + wv) * kMaxKG + gi) * 2 + 1] = 1.f / sq;
      }
    }
  }
  __syncthreads();
  // this slot's digits: one value per (head, coordinate), scattered to its operand bytes
  const Slot sl = a.slot[slot];
  const KGroup& kg = a.k[sl.group];
  for (int e = tid; e < kHT * kD; e += kPrepThreads) {
    const int h = e / kD, c = e % kD;
    float v = 0.f;
    if (h < nh && c >= kg.ch && c < kg.ch + kg.d)
      v = (sl.qjl ? qh[h][c] * sqjl[h][sl.group] : sl.alpha * qt[h][c] * smse[h][sl.group]) * inv_v(c & 3);
    const int cg = c >> 5, cw = c & 31;
    const int kappa = 32 * cg + 8 * (cw & 3) + (cw >> 2);
    const int gp = (kappa & 63) >> 4, byte = (kappa & 15) + 16 * (kappa >> 6);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t d8 = fp8_of(v);
      v -= f32_of_fp8(d8);
      opb[16 * gp + 4 * h + m][byte] = (uint8_t)d8;
    }
  }
  __syncthreads();
  const uint32_t* src = reinterpret_cast<const uint32_t*>(&opb[0][0]);
  uint32_t* dst = a.aops + ((int64_t)key * a.nslots + slot) * 512;
  for (int e = tid; e < 512; e += kPrepThreads) dst[e] = src[e];
}

// P consecutive 32-bit words with one vector load (P = 1..5).
template <int P>
__device__ __forceinline__ void load_words(const uint32_t* p, uint32_t* out) {
  if constexpr (P == 1) {
    out[0] = p[0];
  } else if constexpr (P == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    out[0] = v.x; out[1] = v.y;
  } else if constexpr (P == 3) {
    const uint3 v = *reinterpret_cast<const uint3*>(p);
    out[0] = v.x; out[1] = v.y; out[2] = v.z;
  } else if constexpr (P == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  } else {
    // 5-word records are only 4-byte aligned
    typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(4)));
    const u32x4a v = *reinterpret_cast<const u32x4a*>(p);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3]; out[4] = p[4];
  }
}

// Per-lane data of one chunk for the score phase: the key plane words of the
// lane's coordinate word for its 4 tokens, the key norms and the value norms.
// Norms are held one per lane (lane l holds token 64 w + l of the chunk) and
// handed to the score lanes with a cross-lane read.
template <int NK, int NV>
struct KChunk {
  uint32_t w[4][5];
  float n[NK], r[NK];
  float nv[NV];
};

template <int NK, int NV, int P0, int P1>
__device__ __forceinline__ void load_k(KChunk<NK, NV>& kc, const Args& a, int c0, int te, int bg, int w, int lane,
                                       int kgi, const uint32_t* kbase, int64_t kstep) {
  // kbase points at this lane's words of token lane % 16 of the sequence's
  // first 16-token tile; tiles are kstep words apart.
  const int tl = lane & 15;
  const int64_t tile0 = (c0 >> 4) + 4 * w;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tok = c0 + 64 * w + 16 * i + tl;
#pragma unroll
    for (int pp = 0; pp < 5; ++pp) kc.w[i][pp] = 0u;
    if (tok < te) {
      const uint32_t* p = kbase + (tile0 + i) * kstep;
      if (NK == 1 || kgi == 0)
        load_words<P0>(p, kc.w[i]);
      else
        load_words<P1>(p, kc.w[i]);
    }
  }
  const int tok = c0 + 64 * w + lane;
  const bool valid = tok < te;
#pragma unroll
  for (int gi = 0; gi < NK; ++gi) {
    float n = 0.f, r = 0.f;
    if (valid) {
      const int64_t vi = (int64_t)bg * a.k[gi].seq_stride + tok;
      n = tqd::half_bits_to_f32(a.k[gi].norm[vi]);
      if (a.k[gi].prod) r = tqd::half_bits_to_f32(a.k[gi].rnorm[vi]);
    }
    kc.n[gi] = n;
    kc.r[gi] = r;
  }
#pragma unroll
  for (int gv = 0; gv < NV; ++gv)
    kc.nv[gv] = valid ? tqd::half_bits_to_f32(a.v[gv].norm[(int64_t)bg * a.v[gv].seq_stride + tok]) : 0.f;
}

// Value plane words of this wave's 32 coordinates for a chunk's two 128-token steps.
struct VChunk {
  uint32_t w[2][2][4];
};

__device__ __forceinline__ void load_v(VChunk& vc, const VGroup& vme, int c0, int te, int bg, int lane, int vjl0) {
  const int gp = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int tblk = c0 + 128 * ks + 32 * gp;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) vc.w[ks][tt][pp] = 0u;
      if (tblk < te) {
        const int64_t vt = ((int64_t)bg * vme.seq_stride + tblk) >> 5;
        const int jl = vjl0 + 16 * tt + (lane & 15);
        const uint32_t* pw = vme.packed + (vt * vme.d + jl) * vme.B;
        switch (vme.B) {
          case 1: load_words<1>(pw, vc.w[ks][tt]); break;
          case 2: load_words<2>(pw, vc.w[ks][tt]); break;
          case 3: load_words<3>(pw, vc.w[ks][tt]); break;
          default: load_words<4>(pw, vc.w[ks][tt]); break;
        }
      }
    }
  }
}

// Value sums of one 128-token step for a value group of VB bits.
template <int VB, int VT>
__device__ __forceinline__ void value_step(v4f (&vacc)[2][VT], const v8i& aw, const uint32_t (&vw)[2][4]) {
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
    for (int t = 0; t < n_odd(VB); ++t) {
      uint32_t word = 0;
      const int m = odd_mask(VB, t);
#pragma unroll
      for (int p = 0; p < 4; ++p)
        if ((m >> p) & 1) word ^= vw[tt][p];
      vacc[tt][t] = mfma_fp8_fp4(aw, expand_bits(word), vacc[tt][t]);
    }
  }
}

template <int KB0, int KP0, int KB1, int KP1, int VT, int NV>
__global__ __launch_bounds__(kThreads, 2) void decode_kernel(Args a) {
  constexpr int NK = KB1 > 0 ? 2 : 1;
  constexpr int NS0 = n_odd(KB0) + KP0;
  constexpr int NS = NS0 + (KB1 > 0 ? n_odd(KB1) + KP1 : 0);
  __shared__ __attribute__((aligned(16))) uint8_t wbuf[2][NV][2][16][128];  // [buf][vgroup][step][row][kappa]
  __shared__ float red_m[4][kHT];
  __shared__ int red_e[4][NV];
  __shared__ float fin_l[4][kHT];

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 4, tl = lane & 15;
  const int split = blockIdx.x, ht = blockIdx.y, bg = blockIdx.z;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int h0 = g * a.G + ht * kHT;
  const int nh = min(kHT, a.G - ht * kHT);
  const int len = a.seq_lens ? min(max(a.seq_lens[b], 0), a.T_max) : a.T_max;
  const int ts = split * a.split_len;
  const int te = min(ts + a.split_len, len);

  // this lane's coordinate word of the key layout (score-phase B operand)
  const int W = lane >> 4;
  const int kgi = (NK == 2 && 32 * W >= a.k[NK - 1].ch) ? 1 : 0;
  const KGroup& kme = a.k[kgi];
  const int kP = kgi ? (KB1 + KP1) : (KB0 + KP0);
  const int kGw = kme.d >> 5;
  const int64_t kstep = (int64_t)kGw * 16 * kP;  // words per 16-token tile
  const uint32_t* kbase = kme.packed + (((int64_t)bg * kme.seq_stride) >> 4) * kstep +
                          ((W - (kme.ch >> 5)) * 16 + tl) * kP;
  // this wave's value coordinates 32 w .. 32 w + 31 belong to one value group
  const int vgi = (NV > 1 && 32 * w >= a.v[NV - 1].ch) ? 1 : 0;
  const VGroup& vme = a.v[vgi];
  const int vjl0 = 32 * w - vme.ch;

  // ---- issue the first chunk's loads, then build the query operands
  KChunk<NK, NV> kc;
  VChunk vc;
  if (ts < te) {
    load_k<NK, NV, KB0 + KP0, KB1 + KP1>(kc, a, ts, te, bg, w, lane, kgi, kbase, kstep);
    load_v(vc, vme, ts, te, bg, lane, vjl0);
  }
  const int key = (b * a.Hkv + g) * a.HT + ht;
  v8i aop[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const v4i* src = reinterpret_cast<const v4i*>(a.aops + (((int64_t)key * NS + s) * 64 + lane) * 8);
    const v4i lo = src[0], hi = src[1];
    aop[s] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  // constant parts of the fp4 encoding, per (group, class); scales of this lane's head
  float cm[NK], cq[NK], inv_mse[NK], inv_qjl[NK], gam[NK];
  {
    const v8i cop = const_operand();
#pragma unroll
    for (int gi = 0; gi < NK; ++gi) {
      cm[gi] = cq[gi] = 0.f;
      inv_mse[gi] = a.ascale[(((int64_t)key * kHT + hl) * kMaxKG + gi) * 2 + 0];
      inv_qjl[gi] = a.ascale[(((int64_t)key * kHT + hl) * kMaxKG + gi) * 2 + 1];
      gam[gi] = a.k[gi].gamma;
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const float c4 = 0.25f * sum4(mfma_fp8_fp4(aop[s], cop, v4f{0.f, 0.f, 0.f, 0.f}));
      const int gi = s < NS0 ? 0 : 1;
      const bool q = (gi == 0) ? (KP0 && s == NS0 - 1) : (KP1 && s == NS - 1);
      if (q)
        cq[gi] += c4;
      else
        cm[gi] += c4;
    }
  }
  const float tinv = inv_v(tl & 3);  // fp4 register of this lane's tokens in the value step

  v4f vacc[2][VT], vcon;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int s = 0; s < VT; ++s) vacc[tt][s] = v4f{0.f, 0.f, 0.f, 0.f};
  vcon = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  int e_run[NV];
#pragma unroll
  for (int gv = 0; gv < NV; ++gv) e_run[gv] = -60;

  int buf = 0;
  for (int c0 = ts; c0 < te; c0 += kChunk, buf ^= 1) {
    const bool more = c0 + kChunk < te;
    KChunk<NK, NV> kn;
    if (more) load_k<NK, NV, KB0 + KP0, KB1 + KP1>(kn, a, c0 + kChunk, te, bg, w, lane, kgi, kbase, kstep);

    // ---------------- scores for this wave's 64 tokens
    float lg[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t(&wd)[5] = kc.w[i];
      v4f dm[NK], dq[NK];
#pragma unroll
      for (int gi = 0; gi < NK; ++gi) dm[gi] = dq[gi] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < n_odd(KB0); ++t) {
        uint32_t word = 0;
        const int m = odd_mask(KB0, t);
#pragma unroll
        for (int p = 0; p < 5; ++p)
          if ((m >> p) & 1) word ^= wd[p];
        dm[0] = mfma_fp8_fp4(aop[t], expand_bits(word), dm[0]);
      }
      if constexpr (KP0) dq[0] = mfma_fp8_fp4(aop[NS0 - 1], expand_bits(wd[KB0]), dq[0]);
      if constexpr (KB1 > 0) {
#pragma unroll
        for (int t = 0; t < n_odd(KB1); ++t) {
          uint32_t word = 0;
          const int m = odd_mask(KB1, t);
#pragma unroll
          for (int p = 0; p < 5; ++p)
            if ((m >> p) & 1) word ^= wd[p];
          dm[NK - 1] = mfma_fp8_fp4(aop[NS0 + t], expand_bits(word), dm[NK - 1]);
        }
        if constexpr (KP1) dq[NK - 1] = mfma_fp8_fp4(aop[NS - 1], expand_bits(wd[KB1]), dq[NK - 1]);
      }
      float sc = 0.f;
#pragma unroll
      for (int gi = 0; gi < NK; ++gi) {
        float part = (sum4(dm[gi]) - cm[gi]) * inv_mse[gi];
        if ((gi == 0 && KP0) || (gi == 1 && KP1)) {
          const float qjl = (sum4(dq[gi]) - cq[gi]) * inv_qjl[gi];
          part = fmaf(gam[gi] * __shfl(kc.r[gi], 16 * i + tl, 64), qjl, part);
        }
        sc = fmaf(__shfl(kc.n[gi], 16 * i + tl, 64), part, sc);
      }
      const int tok = c0 + 64 * w + 16 * i + tl;
      const bool valid = tok < te && hl < nh;
      if (valid && a.scores_out) a.scores_out[((int64_t)b * a.Hq + h0 + hl) * a.T_max + tok] = sc;
      lg[i] = valid ? sc * a.scale_log2 : -INFINITY;
    }
    // ---------------- chunk statistics shared by the four waves
    float mx = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    mx = row16_max(mx);
    if (tl == 0) red_m[w][hl] = mx;
#pragma unroll
    for (int gv = 0; gv < NV; ++gv) {
      const float vm = tqd::wave_max(kc.nv[gv]);
      if (lane == 0) red_e[w][gv] = exponent_of(vm);
    }
    __syncthreads();
    const float cmax = fmaxf(fmaxf(red_m[0][hl], red_m[1][hl]), fmaxf(red_m[2][hl], red_m[3][hl]));
    const float m_new = fmaxf(m_run, cmax);
    const bool live = m_new != -INFINITY;
    const float corr = (live && m_run != -INFINITY) ? exp2f(m_run - m_new) : (live ? 0.f : 1.f);
    int e_new[NV];
#pragma unroll
    for (int gv = 0; gv < NV; ++gv)
      e_new[gv] = max(max(max(red_e[0][gv], red_e[1][gv]), max(red_e[2][gv], red_e[3][gv])), e_run[gv]);
    const int eshift = (NV > 1 && vgi) ? e_run[NV - 1] - e_new[NV - 1] : e_run[0] - e_new[0];
    const float vcorr = corr * ldexpf(1.f, eshift);
    if (vcorr != 1.f) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int s = 0; s < VT; ++s) vacc[tt][s] *= vcorr;
      vcon *= vcorr;
    }
    l_run *= corr;
    m_run = m_new;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = live ? exp2f(lg[i] - m_new) : 0.f;
      l_run += p[i];
    }
    // weights -> fp8 digits in LDS (pre-multiplied by 1 / v_r of their fp4 register)
#pragma unroll
    for (int gv = 0; gv < NV; ++gv) {
      const float sv = ldexpf(tinv, 5 - e_new[gv]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tau = 64 * w + 16 * i + tl;
        const int ks = tau >> 7, tp = tau & 127;
        const int kappa = 32 * (tp >> 5) + 8 * (tp & 3) + ((tp & 31) >> 2);
        float r = p[i] * __shfl(kc.nv[gv], 16 * i + tl, 64) * sv;
        uint8_t* dst = &wbuf[buf][gv][ks][4 * hl][kappa];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t d = fp8_of(r);
          r -= f32_of_fp8(d);
          dst[128 * m] = (uint8_t)d;
        }
      }
      e_run[gv] = e_new[gv];
    }
    __syncthreads();
    // ---------------- values: this wave's 32 coordinates over the 256 tokens
    const v8i cop = const_operand();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (c0 + 128 * ks >= te) break;
      const uint8_t* wrow = &wbuf[buf][vgi][ks][lane & 15][0];
      const int gp = lane >> 4;
      const v4i lo = *reinterpret_cast<const v4i*>(wrow + 16 * gp);
      const v4i hi = *reinterpret_cast<const v4i*>(wrow + 64 + 16 * gp);
      const v8i aw = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      vcon = mfma_fp8_fp4(aw, cop, vcon);
      switch (vme.B) {
        case 1: value_step<1, VT>(vacc, aw, vc.w[ks]); break;
        case 2: value_step<2, VT>(vacc, aw, vc.w[ks]); break;
        case 3: if constexpr (VT >= 4) value_step<3, VT>(vacc, aw, vc.w[ks]); break;
        default: if constexpr (VT >= 8) value_step<4, VT>(vacc, aw, vc.w[ks]); break;
      }
    }
    if (more) {
      kc = kn;
      load_v(vc, vme, c0 + kChunk, te, bg, lane, vjl0);
    }
  }

  // ---------------- partial results of this split
  float lsum = row16_sum(l_run);
  if (tl == 0) fin_l[w][hl] = lsum;
  __syncthreads();
  if (hl < nh) {
    float* part = a.partial + (((int64_t)b * a.Hq + h0 + hl) * a.splits + split) * (kD + 2);
    const int ef = (NV > 1 && vgi) ? e_run[NV - 1] : e_run[0];
    const float unscale = ldexpf(1.f, ef - 5);
    const float csub = 0.25f * sum4(vcon) * vme.alpha_sum;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float v = -csub;
#pragma unroll
      for (int s = 0; s < VT; ++s)
        if (s < vme.ntypes) v = fmaf(vme.alpha[s], sum4(vacc[tt][s]), v);
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
// domain) and rotate the value accumulator back with R_v^T. The split weights
// 2^(m_s - M) are tabulated once; each (column, half of the splits) sum
// streams independent loads sixteen at a time; R_v^T splits its rows over the
// two halves of the workgroup.
__global__ __launch_bounds__(kCombThreads) void combine_kernel(Args a) {
  __shared__ float wsp[kMaxCombineSplits];
  __shared__ float acc[kD + 1];
  __shared__ float part2[2][kD + 1];
  __shared__ float osum[2][kD];
  __shared__ float wred[kCombThreads / 64];
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float* part = a.partial + (int64_t)bh * a.splits * (kD + 2);
  const int S = a.splits;
  float mx = -INFINITY;
  for (int s = tid; s < S; s += kCombThreads) mx = fmaxf(mx, part[(int64_t)s * (kD + 2)]);
  mx = tqd::wave_max(mx);
  if (lane == 0) wred[wv] = mx;
  __syncthreads();
  float M = wred[0];
#pragma unroll
  for (int i = 1; i < kCombThreads / 64; ++i) M = fmaxf(M, wred[i]);
  for (int s = tid; s < S; s += kCombThreads) {
    const float ms = part[(int64_t)s * (kD + 2)];
    wsp[s] = (M == -INFINITY || ms == -INFINITY) ? 0.f : exp2f(ms - M);
  }
  __syncthreads();
  // columns 0..kD (0 = softmax sum) times two halves of the splits
  for (int job = tid; job < 2 * (kD + 1); job += kCombThreads) {
    const int col = job % (kD + 1), half = job / (kD + 1);
    const int sbeg = half ? S / 2 : 0, send = half ? S : S / 2;
    const float* pc = part + 1 + col;
    float v0 = 0.f, v1 = 0.f;
    int s = sbeg;
    for (; s + 16 <= send; s += 16) {
      float x[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) x[u] = pc[(int64_t)(s + u) * (kD + 2)];
#pragma unroll
      for (int u = 0; u < 16; u += 2) {
        v0 = fmaf(wsp[s + u], x[u], v0);
        v1 = fmaf(wsp[s + u + 1], x[u + 1], v1);
      }
    }
    for (; s < send; ++s) v0 = fmaf(wsp[s], pc[(int64_t)s * (kD + 2)], v0);
    part2[half][col] = v0 + v1;
  }
  __syncthreads();
  if (tid <= kD) acc[tid] = part2[0][tid] + part2[1][tid];
  __syncthreads();
  const float tot = acc[0];
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  const int half = tid >> 7, i = tid & 127;
  for (int gv = 0; gv < a.nv; ++gv) {
    const VGroup& vg = a.v[gv];
    if (i < vg.d) {
      const int jb = half ? vg.d / 2 : 0, je = half ? vg.d : vg.d / 2;  // multiples of 16
      float s8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const float* Rc = vg.R + i;
      for (int j = jb; j < je; j += 8) {
        float r8[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) r8[u] = Rc[(int64_t)(j + u) * vg.d];
#pragma unroll
        for (int u = 0; u < 8; ++u) s8[u] = fmaf(r8[u], acc[1 + vg.ch + j + u], s8[u]);
      }
      osum[half][vg.ch + i] = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
    }
  }
  __syncthreads();
  if (tid < kD) a.out[(int64_t)bh * kD + tid] = (osum[0][tid] + osum[1][tid]) * inv;
}

// Walsh coefficients of a mirror-symmetric codebook: c[idx] =
// sum_{|S| odd} alpha_S prod_{p in S} (2 bit_p(idx) - 1), subsets S in
// ascending bitmask order.
int odd_walsh(const tq_quantizer& q, float* alphas) {
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
    alphas[n++] = (float)(acc / L);
  }
  return n;
}

using KernelFn = void (*)(Args);

struct Spec {
  int kb0, kp0, kb1, kp1, vt, nv;
  KernelFn fn;
};

#define TQ_SPEC(a, b, c, d, e, f) Spec{a, b, c, d, e, f, decode_kernel<a, b, c, d, e, f>}
// Key group layouts compiled for the matrix-core decode: one group of 1-4
// bits with or without QJL (values in one group), and the 2.5 / 3.5 bit
// outlier splits (two key and two value groups).
const Spec kSpecs[] = {
    TQ_SPEC(1, 1, 0, 0, 4, 1), TQ_SPEC(2, 1, 0, 0, 4, 1), TQ_SPEC(3, 1, 0, 0, 4, 1), TQ_SPEC(4, 1, 0, 0, 4, 1),
    TQ_SPEC(1, 0, 0, 0, 4, 1), TQ_SPEC(2, 0, 0, 0, 4, 1), TQ_SPEC(3, 0, 0, 0, 4, 1), TQ_SPEC(4, 0, 0, 0, 4, 1),
    TQ_SPEC(3, 1, 0, 0, 8, 1), TQ_SPEC(4, 1, 0, 0, 8, 1), TQ_SPEC(3, 0, 0, 0, 8, 1), TQ_SPEC(4, 0, 0, 0, 8, 1),
    TQ_SPEC(2, 1, 1, 1, 4, 2), TQ_SPEC(3, 1, 2, 1, 4, 2),
};
#undef TQ_SPEC

const Spec* find_spec(const tq_kv_desc& k, const tq_kv_desc& v) {
  int vt = 0, Dv = 0, D = 0;
  for (int i = 0; i < v.n_groups; ++i) {
    const int t = n_odd(v.g[i].q.mse_bits);
    vt = vt > t ? vt : t;
    Dv += v.g[i].q.d;
  }
  for (int i = 0; i < k.n_groups; ++i) D += k.g[i].q.d;
  if (D != kD || Dv != kD || k.n_groups > kMaxKG || v.n_groups > kMaxVG) return nullptr;
  const int need_vt = vt <= 4 ? 4 : 8;
  const int kb0 = k.g[0].q.mse_bits, kp0 = k.g[0].q.variant == TQ_PROD;
  const int kb1 = k.n_groups > 1 ? k.g[1].q.mse_bits : 0;
  const int kp1 = k.n_groups > 1 ? (k.g[1].q.variant == TQ_PROD) : 0;
  for (const Spec& sp : kSpecs)
    if (sp.kb0 == kb0 && sp.kp0 == kp0 && sp.kb1 == kb1 && sp.kp1 == kp1 && sp.vt == need_vt &&
        sp.nv == v.n_groups)
      return &sp;
  return nullptr;
}

}  // namespace

namespace tqk {

bool mfma_decode_supported(const tq_kv_desc& k, const tq_kv_desc& v) { return find_spec(k, v) != nullptr; }

DecodePlan plan_decode_mfma(const tq_kv_desc& k, const tq_kv_desc& v, int B, int Hq, int Hkv, int T_max) {
  (void)v;
  DecodePlan p{};
  const int G = Hq / Hkv;
  const int HT = (G + kHT - 1) / kHT;
  const int64_t wgs_per_split = (int64_t)B * Hkv * HT;
  int64_t splits = (512 + wgs_per_split - 1) / wgs_per_split;
  int64_t sl = (T_max + splits - 1) / splits;
  const int64_t min_sl = (T_max + kMaxCombineSplits - 1) / kMaxCombineSplits;  // the combine's split table
  if (sl < min_sl) sl = min_sl;
  sl = (sl + kChunk - 1) / kChunk * kChunk;
  p.split_len = (int)sl;
  p.splits = (int)((T_max + sl - 1) / sl);
  p.head_chunk = kHT;
  p.n_chunks = HT;
  p.D = kD;
  p.Dv = kD;
  int slots = 0;
  for (int i = 0; i < k.n_groups; ++i) slots += n_odd(k.g[i].q.mse_bits) + (k.g[i].q.variant == TQ_PROD ? 1 : 0);
  const size_t keys = (size_t)B * Hkv * HT;
  p.qprep_floats = keys * slots * 512 + keys * kHT * kMaxKG * 2;
  p.partial_floats = (size_t)B * Hq * p.splits * (kD + 2);
  return p;
}

hipError_t launch_decode_mfma(const tq_kv_desc& k, const tq_kv_desc& v, const void* q, tq_dtype qdt, int B, int Hq,
                              int Hkv, int T_max, const int32_t* seq_lens, float scale, float* out,
                              float* scores_out, void* ws, const DecodePlan& plan, hipStream_t s) {
  const Spec* sp = find_spec(k, v);
  if (!sp) return hipErrorInvalidValue;
  Args a{};
  a.nk = k.n_groups;
  a.nv = v.n_groups;
  int ns = 0;
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
    float alphas[kMaxVTypes];
    const int nt = odd_walsh(g.q, alphas);
    for (int t = 0; t < nt; ++t) a.slot[ns++] = Slot{gi, 0, alphas[t]};
    if (o.prod) a.slot[ns++] = Slot{gi, 1, 1.f};
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
    o.ntypes = odd_walsh(g.q, o.alpha);
    o.alpha_sum = 0.f;
    for (int t = 0; t < o.ntypes; ++t) o.alpha_sum += o.alpha[t];
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
  a.ascale = reinterpret_cast<float*>(a.aops + keys * ns * 512);
  a.partial = static_cast<float*>(ws) + plan.qprep_floats;
  a.out = out;
  hipLaunchKernelGGL(qprep_kernel, dim3((unsigned)keys, ns), dim3(kPrepThreads), 0, s, a);
  const dim3 grid(plan.splits, a.HT, B * Hkv);
  hipLaunchKernelGGL(sp->fn, grid, dim3(kThreads), 0, s, a);
  hipLaunchKernelGGL(combine_kernel, dim3(B * Hq), dim3(kCombThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace tqk
