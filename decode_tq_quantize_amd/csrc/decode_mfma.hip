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
// fp8 / fp6 x fp4 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4):
//  * a 32-bit plane word w becomes four fp4 registers, register r taking bit
//    4 i + r of w into nibble i with one bit operation: r = 3 gives +-1
//    (bit select); for the value sums r = 2, 1, 0 give {0, 2}, {0, 1},
//    {0, 1/2} (masks), i.e. u_r + v_r sigma with (u, v) = (0, 1), (1, 1),
//    (1/2, 1/2), (1/4, 1/4), and the weights are pre-multiplied by 1 / v_r
//    (a power of two); for the scores r = 0, 1 also take fixed exponent bits
//    ({4, 6}, {2, 4}, {0, 2}: every plane bit weighs 2, expand_key_bits);
//    the constant part is removed exactly with MFMAs against constant
//    operands;
//  * the softmax weights are split into fp8 e4m3 digits v = d0 + d1/16 +
//    d2/256 (each the fp8 rounding of what the previous ones left, scaled up
//    by 16 so that it stays a normal fp8 number), about 12 significant bits;
//    the query coefficients into four fp6 e2m3 digits per 32-channel block
//    with a per-block E8M0 scale (write_block_operands), error at most 2^-20
//    of the block's largest; digits are MFMA rows, fp32 accumulation.
// Rows of every MFMA are (query head, digit) = 4 x 4; columns are 16 tokens
// (scores) or 16 value coordinates (value sums).
//
// Operand layouts used (measured on gfx950 for the mixed forms):
// fp4 operand lane l, nibble p (register p/8) -> k = 32 (l/16) + p; fp8
// operand lane l, byte p -> k = 16 (l/16) + (p % 16) + 64 (p / 16); fp6
// operand lane l, bits 6 p .. 6 p + 5 of 6 registers -> k = 32 (l/16) + p;
// D lane l register i -> row 4 (l/16) + i, column l % 16.
//
// Kernels: qprep builds the query operands of every (batch, KV head, head
// tile) (q~ = R q, q^ = S q~, per-block scales, fp6 digits); decode runs
// one workgroup (4 waves) per (split of the sequence, head tile of 4 query
// heads, batch x KV head) over 256-token chunks: each wave scores 64 tokens,
// the chunk maximum is exchanged through LDS, each wave writes the fp8 digits
// of its weights to LDS, and each wave accumulates 32 value coordinates over
// the 256 tokens; the next chunk's key planes and norms are prefetched during
// the current chunk. Partials (max, sum, rotated accumulator) go to the
// workspace; combine merges the splits and applies R_v^T.
#include <math.h>
#include <stdlib.h>

#include <algorithm>

#include "device_common.h"
#include "internal.h"
#include "quantize_tile.h"

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
constexpr int kJSlice = 16;                // value channels per combine workgroup
constexpr int kJSlices = kD / kJSlice;
constexpr int kRowSlice = 32;              // query-transform rows per workgroup (one K block of the score products)

struct KGroup {
  const uint32_t* packed;
  const uint16_t* norm;
  const uint16_t* rnorm;
  const float* R;
  const float* S;
  const float* SR;  // S R followed by its largest row norm, or null
  int64_t seq_stride;
  int ch, d, B, prod;
  float gamma;
  float amax;  // largest |Walsh coefficient| of the codebook
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
  int slot_group;             // bit s: slot s belongs to key group 1
  int slot_qjl;               // bit s: slot s is the QJL part of its group
  float slot_alpha[kMaxSlots];  // Walsh coefficient of codebook slot s (1 for QJL)
  const void* q;
  int qbf16;
  int B, Hq, Hkv, G, HT, T_max;
  const int32_t* seq_lens;
  float scale_log2;
  int splits, split_len;
  float* scores_out;
  float* qt;         // [keys][4 heads][kD] q~ = R q per key group
  float* qh;         // [keys][4 heads][kD] q^ = S q~ (PROD groups, else 0)
  uint32_t* aops;    // [keys][nslots][64 lanes][8 dwords] query operands of every slot
  float* partial;    // [B * Hq][splits][kD + 2] (max, sum, rotated accumulator)
  float* out;
  // paged cache (null table: contiguous sequences): row of (sequence b, KV
  // head g, token t) = (block_table[b][t / block_tokens] * Hkv + g) *
  // block_tokens + t % block_tokens
  const int32_t* block_table;
  int max_blocks, block_tokens;
  int64_t num_blocks;
};

// Slot s of the operand table for a per-lane s: the coefficients are read
// as uniform values and selected, so no per-lane access to the argument
// memory is made.
__device__ __forceinline__ Slot slot_of(const Args& a, int s) {
  float al = a.slot_alpha[0];
#pragma unroll
  for (int t = 1; t < kMaxSlots; ++t) al = s == t ? a.slot_alpha[t] : al;
  return Slot{(a.slot_group >> s) & 1, (a.slot_qjl >> s) & 1, al};
}

__device__ __forceinline__ uint32_t fp8_of(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.f, 0, false) & 0xffu;
}
__device__ __forceinline__ float f32_of_fp8(uint32_t b) { return __builtin_amdgcn_cvt_f32_fp8((int)b, 0); }
// The leading four significant bits of x (truncated toward zero): a value
// that e4m3 holds exactly whenever it lies in e4m3's normal range, and
// x - head4(x) is exact.
__device__ __forceinline__ float head4(float x) { return __uint_as_float(__float_as_uint(x) & 0xfff00000u); }
// e4m3 byte (in bits 0..7) of a value with at most four significant bits;
// the register's other bytes are left undefined.
__device__ __forceinline__ uint32_t fp8_exact(float x) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x, x, (int)__float_as_uint(x), false);
}


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

// Key planes for the score products: every plane register carries 2 b plus
// an offset o_r = 4, 2, 0 (fp4 pairs {4, 6}, {2, 4}, {0, 2}: an OR of fixed
// exponent bits, no shift), register 3 the sign +-1 as in expand_bits. With
// the same weight 2 in every register the query operand needs no per-register
// factor, so the 32 entries of a block share one magnitude range.
// (w & m) | c in one VALU instruction (the VOP3 form takes one scalar and
// one vector constant: the compiler otherwise splits it in two)
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(m), "v"(c));
  return r;
}
__device__ __forceinline__ v8i expand_key_bits(uint32_t w) {
  v8i r;
  r[0] = (int)and_or(w, 0x11111111u, 0x66666666u);
  r[1] = (int)and_or(w, 0x22222222u, 0x44444444u);
  r[2] = (int)(w & 0x44444444u);
  r[3] = (int)((w & 0x22222222u) | (~w & 0xAAAAAAAAu));
  r[4] = r[5] = r[6] = r[7] = 0;
  return r;
}
// What expand_key_bits adds beyond 2 b - 1 in registers 0..2, 1 + o_r =
// 5, 3, 1, as two fp4 operands (4, 2, 1, 0) + (1, 1, 0, 0): 5 has no fp4 code.
__device__ __forceinline__ v8i key_const_hi() { return v8i{0x66666666, 0x44444444, 0x22222222, 0, 0, 0, 0, 0}; }
__device__ __forceinline__ v8i key_const_lo() { return v8i{0x22222222, 0x22222222, 0, 0, 0, 0, 0, 0}; }

// 1 / v_r for register r of the fp4 operand.
__device__ __forceinline__ float inv_v(int r) { return r == 0 ? 4.f : (r == 1 ? 2.f : 1.f); }

__device__ __forceinline__ v4f mfma_fp8_fp4(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, 0, 0, 0);
}
// The same with a per-lane E8M0 scale (2^(sa - 127)) on the A operand: the
// scale of lane l multiplies row l % 16 over the 32 consecutive K positions
// 32 (l / 16) .. + 31 (measured on gfx950: not the bytes lane l holds, which
// are K 16 (l / 16) + 0..15 and 64 + 16 (l / 16) + 0..15); B is unscaled
// (127).
__device__ __forceinline__ v4f mfma_fp8_fp4_sa(v8i a, v8i b, v4f c, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, sa, 0, 127);
}
// The same with an fp6 e2m3 A operand (six registers: lane l holds K
// positions 32 (l / 16) + f in bits 6 f .. 6 f + 5, measured on gfx950), at
// twice the fp8 rate.
__device__ __forceinline__ v4f mfma_fp6_fp4_sa(v8i a, v8i b, v4f c, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 2, 4, 0, sa, 0, 127);
}
// Sum of the four digit rows of a result already weighted by the scales.
__device__ __forceinline__ float sum4(v4f x) { return (x[0] + x[1]) + (x[2] + x[3]); }

// Reductions over the 16 lanes of a DPP row by row rotations (every lane
// of the row ends with the result); no LDS traffic.
template <int N>
__device__ __forceinline__ float row_ror(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x120 + N, 0xf, 0xf, true));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, row_ror<8>(v));
  v = fmaxf(v, row_ror<4>(v));
  v = fmaxf(v, row_ror<2>(v));
  v = fmaxf(v, row_ror<1>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += row_ror<8>(v);
  v += row_ror<4>(v);
  v += row_ror<2>(v);
  v += row_ror<1>(v);
  return v;
}
// Largest of unsigned values over the wave: row maxima by row rotations,
// then the four rows' values read as uniform values. (Raw bits of
// non-negative IEEE halves order like the values they encode.)
template <int N>
__device__ __forceinline__ uint32_t row_ror_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x120 + N, 0xf, 0xf, true);
}
__device__ __forceinline__ uint32_t wave_max64_u(uint32_t v) {
  v = max(v, row_ror_u<8>(v));
  v = max(v, row_ror_u<4>(v));
  v = max(v, row_ror_u<2>(v));
  v = max(v, row_ror_u<1>(v));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}

__device__ __forceinline__ int exponent_of(float x) {
  int e;
  frexpf(x, &e);
  return x > 0.f ? e : -60;
}

// fp6 e2m3 (OCP MX: sign, two exponent bits of bias 1, three mantissa bits;
// magnitudes 0.125 .. 7.5, subnormals below 1) of x, rounded to nearest
// even, saturating; and the value of such a code.
__device__ __forceinline__ uint32_t e2m3_of(float x) {
  const float ax = fabsf(x);
  const int ep = ax < 2.f ? 1 : (ax < 4.f ? 2 : 3);  // max(exponent field, 1)
  const int code = min((int)rintf(ldexpf(ax, 4 - ep)) + 8 * (ep - 1), 31);
  return (uint32_t)code | (x < 0.f ? 32u : 0u);
}
__device__ __forceinline__ float e2m3_value(uint32_t c) {
  const int ef = (int)((c >> 3) & 3), m = (int)(c & 7);
  const float v = ef == 0 ? 0.125f * (float)m : ldexpf(1.f + 0.125f * (float)m, ef - 1);
  return (c & 32u) ? -v : v;
}

// Digits of a real operand: v = d0 + d1 / 16 + d2 / 256 + d3 / 4096, each
// d_m the fp8 e4m3 rounding of the residual left by the previous digits,
// scaled by 16 per digit so that every digit stays in the normal fp8 range
// (relative precision about 2^-16; no absolute floor). The four digits are
// four rows of the MFMA; wsum4 recombines them. The softmax weights take
// three digits: the first two by truncation (d_m the leading four
// significant bits of the residual, cut by a mask, so each carries at least
// four new bits), the third rounded to nearest, relative precision about
// 2^-12 with no bias; their fourth row is zero.
constexpr float kDigitStep = 16.f;
// The score operands' fp6 digits step by 32 (write_block_operands).
constexpr float kScoreDigitStep = 32.f;
__device__ __forceinline__ float wsum4(v4f x) {
  return (x[0] + x[1] * (1.f / 16.f)) + (x[2] * (1.f / 256.f) + x[3] * (1.f / 4096.f));
}

template <int N>
struct IntC {
  static constexpr int value = N;
};

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

// ------------------------------------------------------------------ query transforms
// q~ = R q (rotate) and q^ = S q~ (project) of every (batch, KV head, head
// tile), one workgroup per 16 rows of the stacked key groups so that the
// matrices are read by many compute units at once. Thread t handles row
// t / 16 of the slice and columns 8 (t % 16) .. 8 (t % 16) + 7 of it for the
// tile's 4 heads; the 16 partial sums of a row meet by lane exchanges.
constexpr int kQtThreads = 256;

// The score operands of every slot over one 32-channel block kb (K
// positions 32 kb .. 32 kb + 31 of the score products), from the block's
// q~ (tq[h * tstride + c]) and q^ (hq[h * hstride + c]), c = channel within
// the block. K position f of a block holds channel 4 (f % 8) + f / 8 (the
// key operand's bit order, expand_key_bits). Per (slot, head) the block's
// values are scaled by a power of two that puts the largest in [1, 2) and
// split into four fp6 e2m3 digits, each carrying the rounding of the ones
// before it times 32 (a digit below 2 is exact to 1/16 in the subnormal and
// first binades, so every digit stays at most 2 and adds 5 bits; error at
// most 2^-20 of the block's largest); lane 16 kb + 4 h + m of the slot's
// 64 x 8 dwords holds digit m of head h (bits 6 f .. 6 f + 5 of dwords 0..5)
// and, in dword 6, the E8M0 scale that undoes both (the slot's other lanes
// are written by the other blocks' workgroups).
__device__ __forceinline__ void write_block_operands(const Args& a, int key, int kb, int gsl, const float* tq, int tstride,
                                                     const float* hq, int hstride,
                                                     uint8_t (&codes)[kMaxSlots][kHT][4][32], int (&escl)[kMaxSlots][kHT]) {
  const int tid = threadIdx.x, nslots = a.nslots;
  // unit (slot, head, f): the 32 positions of a (slot, head) are 32
  // consecutive lanes of one wave
  for (int unit = tid; unit < nslots * kHT * 32; unit += kQtThreads) {
    const int f = unit & 31, h = (unit >> 5) & 3, s2 = unit >> 7;
    const Slot sl = slot_of(a, s2);
    const int c = 4 * (f & 7) + (f >> 3);
    float v = 0.f;
    if (sl.group == gsl) v = sl.qjl ? hq[h * hstride + c] : sl.alpha * tq[h * tstride + c];
    float mx = row16_max(fabsf(v));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 32));
    const int e = exponent_of(mx);  // the largest lies in [2^(e-1), 2^e)
    float x = ldexpf(v, 1 - e);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t code = e2m3_of(x);
      codes[s2][h][m][f] = (uint8_t)code;
      x = (x - e2m3_value(code)) * kScoreDigitStep;
    }
    if (f == 0) escl[s2][h] = e;
  }
  __syncthreads();
  // unit (slot, head, digit): the row's 32 codes packed into dwords 0..5,
  // its scale into dword 6
  for (int unit = tid; unit < nslots * kHT * 4; unit += kQtThreads) {
    const int m = unit & 3, h = (unit >> 2) & 3, s2 = unit >> 4;
    const uint4* src = reinterpret_cast<const uint4*>(&codes[s2][h][m][0]);
    const uint4 c0 = src[0], c1 = src[1];
    const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    uint32_t w[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
    for (int f = 0; f < 32; ++f) {
      const uint32_t code = (cw[f >> 2] >> (8 * (f & 3))) & 63u;
      const int bit = 6 * f;
      w[bit >> 5] |= code << (bit & 31);
      if ((bit & 31) > 26) w[(bit >> 5) + 1] |= code >> (32 - (bit & 31));
    }
    // a digit whose scale would fall below E8M0's 2^-127 (blocks whose
    // largest magnitude is under about 2^-110) is left out rather than
    // weighted wrongly
    const int sc = 127 + escl[s2][h] - 1 - 5 * m;
    if (sc < 0) {
#pragma unroll
      for (int i = 0; i < 6; ++i) w[i] = 0u;
    }
    w[6] = (uint32_t)max(sc, 0);
    uint4* dst = reinterpret_cast<uint4*>(a.aops + ((int64_t)key * nslots + s2) * 512 + (16 * kb + 4 * h + m) * 8);
    dst[0] = uint4{w[0], w[1], w[2], w[3]};
    dst[1] = uint4{w[4], w[5], w[6], w[7]};
  }
}

// Both transforms in one pass when S R is available: workgroup (key, 32-row
// slice) forms rows of q~ = R q and q^ = (S R) q, the slice being one
// 32-channel block of the score products, and writes the fp6 digit
// operands of every slot for its block (write_block_operands).
__device__ __forceinline__ void qfused_body(const Args& a, const int key, const int slice) {
  __shared__ float qts[kHT][kRowSlice], qhs[kHT][kRowSlice];
  __shared__ __attribute__((aligned(16))) uint8_t codes[kMaxSlots][kHT][4][32];
  __shared__ int escl[kMaxSlots][kHT];
  const int nk = a.nk, Hkv = a.Hkv, HT = a.HT, G = a.G, Hq = a.Hq, qbf16 = a.qbf16;
  const int k1ch = a.k[1].ch, k0d = a.k[0].d, k1d = a.k[1].d, k0p = a.k[0].prod, k1p = a.k[1].prod;
  const float* R0 = a.k[0].R;
  const float* R1 = a.k[1].R;
  const float* F0 = a.k[0].SR;
  const float* F1 = a.k[1].SR;
  const int b = key / (Hkv * HT);
  const int g = (key / HT) % Hkv;
  const int ht = key % HT;
  const int h0 = g * G + ht * kHT;
  const int nh = min(kHT, G - ht * kHT);
  const int tid = threadIdx.x, cb = tid & 15;
  const int gsl = ((nk > 1) & (slice * kRowSlice >= k1ch)) ? 1 : 0;
  const bool g1 = gsl == 1;
  const int d = g1 ? k1d : k0d, ch = g1 ? k1ch : 0;
  const int prod = g1 ? k1p : k0p;
  const float* Rm = g1 ? R1 : R0;
  const float* Fm = g1 ? F1 : F0;
  const bool on = 8 * cb < d;
  const int col = ch + min(8 * cb, d - 8);

  // every load unconditional and of one shape (a group without a sketch
  // reads R in place of S R and ignores it), so that none waits on another;
  // thread t takes rows 16 half + t / 16 of the slice
  const float* Fsrc = prod ? Fm : Rm;
  float4 m0[2], m1[2], f0[2], f1[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int r = slice * kRowSlice + 16 * hf + (tid >> 4) - ch;
    const float4* rr = reinterpret_cast<const float4*>(Rm + (int64_t)r * d + (col - ch));
    const float4* fr = reinterpret_cast<const float4*>(Fsrc + (int64_t)r * d + (col - ch));
    m0[hf] = rr[0];
    m1[hf] = rr[1];
    f0[hf] = fr[0];
    f1[hf] = fr[1];
  }
  float x[kHT][8];
  if (qbf16) {
#pragma unroll
    for (int h = 0; h < kHT; ++h) {
      const int64_t qo = ((int64_t)b * Hq + h0 + min(h, nh - 1)) * kD + col;
      const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + qo);
      const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[h][2 * k] = __uint_as_float(wd[k] << 16);
        x[h][2 * k + 1] = __uint_as_float(wd[k] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < kHT; ++h) {
      const int64_t qo = ((int64_t)b * Hq + h0 + min(h, nh - 1)) * kD + col;
      const float4* xr = reinterpret_cast<const float4*>(static_cast<const float*>(a.q) + qo);
      const float4 u = xr[0], v = xr[1];
      x[h][0] = u.x; x[h][1] = u.y; x[h][2] = u.z; x[h][3] = u.w;
      x[h][4] = v.x; x[h][5] = v.y; x[h][6] = v.z; x[h][7] = v.w;
    }
  }
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    float ot = 0.f, oh = 0.f;
    const float mv[8] = {m0[hf].x, m0[hf].y, m0[hf].z, m0[hf].w, m1[hf].x, m1[hf].y, m1[hf].z, m1[hf].w};
    const float fv[8] = {f0[hf].x, f0[hf].y, f0[hf].z, f0[hf].w, f1[hf].x, f1[hf].y, f1[hf].z, f1[hf].w};
#pragma unroll
    for (int h = 0; h < kHT; ++h) {
      float t = 0.f, u = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        t = fmaf(mv[k], x[h][k], t);
        u = fmaf(fv[k], x[h][k], u);
      }
      const bool use = on && h < nh;
      // the 16 lanes of a row hold the 16 column blocks: row rotations sum them
      t = row16_sum(use ? t : 0.f);
      u = row16_sum(use && prod ? u : 0.f);
      if (cb == h) {
        ot = t;
        oh = u;
      }
    }
    if (cb < kHT) {
      qts[cb][16 * hf + (tid >> 4)] = ot;
      qhs[cb][16 * hf + (tid >> 4)] = oh;
    }
  }
  __syncthreads();
  write_block_operands(a, key, slice, gsl, &qts[0][0], kRowSlice, &qhs[0][0], kRowSlice, codes, escl);
}

__global__ __launch_bounds__(kQtThreads) void qfused_kernel(Args a) { qfused_body(a, blockIdx.x, blockIdx.y); }

// The appends of a decode step (riverfrot sections 2.2-2.3 and 4.1-4.3: the
// new token's key and value are compressed into the cache before the query
// attends to them), carried by the query-transform launch: workgroups past
// the transform's take 2-vector tiles of one group's appends each.
struct StepAppend {
  tqq::QArgs q[2 * TQ_MAX_GROUPS];
  int n;             // argument sets
  int tiles;         // 2-vector tiles per set
  int key_columns;   // transform workgroups along x (the rest are appends)
};
// (tiles of 2 vectors, the matrices staged through LDS 32 columns at a time:
// about 19 KB of LDS, so the transform's workgroups keep their occupancy;
// staging 128 columns at once measured no faster)
constexpr int kStepTV = 2, kStepJC = 32;
static_assert(sizeof(Args) + sizeof(StepAppend) <= 4096, "kernel arguments of the step launch");

template <bool DIRECT>
__global__ __launch_bounds__(kQtThreads) void qfused_step_kernel(Args a, StepAppend st) {
  static_assert(kQtThreads == tqq::kQThreads, "the append tiles assume the quantiser's workgroup size");
  if ((int)blockIdx.x < st.key_columns) {
    qfused_body(a, blockIdx.x, blockIdx.y);
    return;
  }
  const int t = ((int)blockIdx.x - st.key_columns) * (int)gridDim.y + (int)blockIdx.y;
  const int e = t / st.tiles;
  if (e >= st.n) return;
  extern __shared__ float smem[];
  tqq::quantize_tile<kStepTV, kStepJC, DIRECT>(st.q[e], t - e * st.tiles, smem);
}

template <bool PROJECT>
__global__ __launch_bounds__(kQtThreads) void qtransform_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) float qts[kHT][kD];  // q~ of the key (project)
  __shared__ float qhs[kHT][kRowSlice];
  __shared__ __attribute__((aligned(16))) uint8_t codes[kMaxSlots][kHT][4][32];
  __shared__ int escl[kMaxSlots][kHT];
  // every argument field this kernel needs is read up front and
  // unconditionally (both groups), so the reads overlap instead of chaining
  const int nk = a.nk, Hkv = a.Hkv, HT = a.HT, G = a.G, Hq = a.Hq, qbf16 = a.qbf16;
  const int k1ch = a.k[1].ch, k0d = a.k[0].d, k1d = a.k[1].d;
  const int k0p = a.k[0].prod, k1p = a.k[1].prod;
  const float* R0 = a.k[0].R;
  const float* R1 = a.k[1].R;
  const float* S0 = a.k[0].S;
  const float* S1 = a.k[1].S;
  const void* qsrc = a.q;
  float* qt = a.qt;
  float* qh = a.qh;
  const int key = blockIdx.x, slice = blockIdx.y;
  const int b = key / (Hkv * HT);
  const int g = (key / HT) % Hkv;
  const int ht = key % HT;
  const int h0 = g * G + ht * kHT;
  const int nh = min(kHT, G - ht * kHT);
  const int tid = threadIdx.x, cb = tid & 15;
  // the slice lies in one key group (group sizes are multiples of 32)
  const int gsl = ((nk > 1) & (slice * kRowSlice >= k1ch)) ? 1 : 0;
  const bool g1 = gsl == 1;
  const int d = g1 ? k1d : k0d, ch = g1 ? k1ch : 0;
  const int prod = g1 ? k1p : k0p;
  const float* Rm = g1 ? R1 : R0;
  const float* Sm = g1 ? S1 : S0;
  const bool on = 8 * cb < d;
  const int col = ch + min(8 * cb, d - 8);  // clamped so that every load is in range

  // this thread's 8 entries of rows 16 half + t / 16 of the slice of R
  // (rotate) or S (project)
  float4 m0[2], m1[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    m0[hf] = m1[hf] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!PROJECT || prod) {
      const int r = slice * kRowSlice + 16 * hf + (tid >> 4) - ch;
      const float4* mr = reinterpret_cast<const float4*>((PROJECT ? Sm : Rm) + (int64_t)r * d + (col - ch));
      m0[hf] = mr[0];
      m1[hf] = mr[1];
    }
  }
  float x[kHT][8];
  if (PROJECT) {
#pragma unroll
    for (int h = 0; h < kHT; ++h) {
      const float4* xr = reinterpret_cast<const float4*>(qt + ((int64_t)key * kHT + h) * kD + col);
      const float4 u = xr[0], v = xr[1];
      x[h][0] = u.x; x[h][1] = u.y; x[h][2] = u.z; x[h][3] = u.w;
      x[h][4] = v.x; x[h][5] = v.y; x[h][6] = v.z; x[h][7] = v.w;
    }
  } else if (qbf16) {
#pragma unroll
    for (int h = 0; h < kHT; ++h) {
      const int hr = min(h, nh - 1);
      const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(qsrc) +
                                                      ((int64_t)b * Hq + h0 + hr) * kD + col);
      const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[h][2 * k] = __uint_as_float(wd[k] << 16);
        x[h][2 * k + 1] = __uint_as_float(wd[k] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < kHT; ++h) {
      const int hr = min(h, nh - 1);
      const float4* xr =
          reinterpret_cast<const float4*>(static_cast<const float*>(qsrc) + ((int64_t)b * Hq + h0 + hr) * kD + col);
      const float4 u = xr[0], v = xr[1];
      x[h][0] = u.x; x[h][1] = u.y; x[h][2] = u.z; x[h][3] = u.w;
      x[h][4] = v.x; x[h][5] = v.y; x[h][6] = v.z; x[h][7] = v.w;
    }
  }
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int i = slice * kRowSlice + 16 * hf + (tid >> 4);  // output channel (stacked row)
    float acc[kHT];
#pragma unroll
    for (int h = 0; h < kHT; ++h) {
      float s0 = m0[hf].x * x[h][0], s1 = m0[hf].y * x[h][1];
      s0 = fmaf(m0[hf].z, x[h][2], s0);
      s1 = fmaf(m0[hf].w, x[h][3], s1);
      s0 = fmaf(m1[hf].x, x[h][4], s0);
      s1 = fmaf(m1[hf].y, x[h][5], s1);
      s0 = fmaf(m1[hf].z, x[h][6], s0);
      s1 = fmaf(m1[hf].w, x[h][7], s1);
      float v = on && h < nh ? s0 + s1 : 0.f;
      v += __shfl_xor(v, 8, 16);
      v += __shfl_xor(v, 4, 16);
      v += __shfl_xor(v, 2, 16);
      v += __shfl_xor(v, 1, 16);
      acc[h] = v;
    }
    float out = acc[0];
#pragma unroll
    for (int h = 1; h < kHT; ++h)
      if (cb == h) out = acc[h];
    if (!PROJECT) {
      if (cb < kHT) qt[((int64_t)key * kHT + cb) * kD + i] = out;
    } else if (cb < kHT) {
      qh[((int64_t)key * kHT + cb) * kD + i] = prod ? out : 0.f;
      qhs[cb][16 * hf + (tid >> 4)] = prod ? out : 0.f;
    }
  }
  if (!PROJECT) return;

  // ---- project only: the fp6 operands of every slot over this slice's
  // block, from q~ (all of the key's channels, staged here) and the
  // slice's rows of q^
  if ((tid >> 4) == 0 && on) {
#pragma unroll
    for (int h = 0; h < kHT; ++h)
#pragma unroll
      for (int k = 0; k < 8; ++k) qts[h][col + k] = x[h][k];
  }
  __syncthreads();
  write_block_operands(a, key, slice, gsl, &qts[0][slice * kRowSlice], kD, &qhs[0][0], kRowSlice, codes, escl);
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
//
// Every load below is unconditional and of one fixed shape: tokens past the
// split's end re-read its last valid tile or token and are masked where they
// are used (their logits are -inf, so their softmax weights are 0). A load
// under a per-lane or data-dependent condition would make the compiler wait
// for it at the join, serialising the prefetch.
template <int NK, int NV>
struct KChunk {
  uint32_t w[4][5];
  // IEEE half bits, two to a register, converted where used: key norm (low
  // half) and residual norm (high half) of token 16 i + lane % 16; value
  // norms of tokens 32 j + lane % 16 (low) and 32 j + 16 + lane % 16 (high)
  uint32_t nr[NK][4];
  uint32_t nv[NV][2];
};

__device__ __forceinline__ float hbits(uint32_t h) { return tqd::half_bits_to_f32((uint16_t)h); }
__device__ __forceinline__ float hbits_hi(uint32_t h) { return tqd::half_bits_to_f32((uint16_t)(h >> 16)); }
// Half i (0: low, 1: high) of a register of two halves.
__device__ __forceinline__ float hbits_at(uint32_t h, int i) { return i ? hbits_hi(h) : hbits(h); }

// Load at a 32-bit unsigned byte offset from a base pointer.
template <class T>
__device__ __forceinline__ const T* at_bytes(const T* base, uint32_t byte_off) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + byte_off);
}

// Raw buffer resource over [base, base + bytes): loads use a per-lane byte
// offset (vector register, fixed for the kernel) plus a wave-uniform byte
// offset (scalar register, advanced per chunk), and read 0 past `bytes`.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
template <int P>
__device__ __forceinline__ void buf_words(rsrc_t r, uint32_t voff, uint32_t soff, uint32_t* out) {
  typedef uint32_t u2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u3 __attribute__((ext_vector_type(3)));
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  if constexpr (P == 1) {
    out[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
  } else if constexpr (P == 2) {
    const u2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    out[0] = v[0]; out[1] = v[1];
  } else if constexpr (P == 3) {
    const u3 v = __builtin_amdgcn_raw_buffer_load_b96(r, voff, soff, 0);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2];
  } else {
    const u4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
    if constexpr (P == 5) out[4] = __builtin_amdgcn_raw_buffer_load_b32(r, voff + 16u, soff, 0);
  }
}
__device__ __forceinline__ uint32_t buf_half(rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

// Addressing of one wave's loads. One key group: buffer resources over the
// sequence's key planes and norms. Two key groups (lanes of different
// groups read different arrays): plain per-lane pointers.
// Key planes: one resource per key group over the sequence's planes. A lane
// reads its own group's planes at its offset in a tile; its offset into the
// other group's resource lies outside that resource, so the same load reads
// 0 there without touching memory, and the two results are merged by OR.
constexpr uint32_t kOutside = 0x80000000u;
struct KAddr {
  rsrc_t res[kMaxKG];     // key planes of the sequence, per group
  uint32_t step[kMaxKG];  // bytes per 16-token tile, per group
  uint32_t voff[kMaxKG];  // this lane's byte offset within a tile, per group
};
struct NAddr {
  rsrc_t n[kMaxKG], r[kMaxKG], nv[kMaxVG];  // norms of the sequence
};
struct VAddr {
  rsrc_t res;           // value planes of the sequence (this wave's value group)
  uint32_t tile_bytes;  // bytes per 32-token tile
  uint32_t lane_off;    // this lane's byte offset (its 32-token block and first coordinate)
  int vB;
};

template <int NK, int NV, int P0, int P1, int KP0, int KP1, int PART = 3>
__device__ __forceinline__ void load_k(KChunk<NK, NV>& kc, const KAddr& ka, const NAddr& na, int c0, int tlast,
                                       int w, int lane) {
  // tiles past the split's end re-read its last tile (their tokens are
  // masked where used; the tile lies inside the sequence's stride)
  const int last_tile = tlast >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (!(PART & 1)) break;
    const uint32_t tile = (uint32_t)min((c0 >> 4) + 4 * w + i, last_tile);
    if constexpr (NK == 1) {
      buf_words<P0>(ka.res[0], ka.voff[0], tile * ka.step[0], kc.w[i]);
    } else {
      // lanes of the two groups hold P0 or P1 words; the extra words of the
      // smaller group are 0 and never weighted (its query digits are zero)
      uint32_t w0[5] = {0u, 0u, 0u, 0u, 0u}, w1[5] = {0u, 0u, 0u, 0u, 0u};
      buf_words<P0>(ka.res[0], ka.voff[0], tile * ka.step[0], w0);
      buf_words<P1>(ka.res[1], ka.voff[1], tile * ka.step[1], w1);
#pragma unroll
      for (int pp = 0; pp < 5; ++pp) kc.w[i][pp] = w0[pp] | w1[pp];
    }
  }
  const uint32_t tl2 = 2u * (lane & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t tok0 = 16u * (uint32_t)min((c0 >> 4) + 4 * w + i, last_tile);
#pragma unroll
    for (int gi = 0; gi < NK; ++gi) {
      if constexpr (!(PART & 1)) break;
      const uint32_t nn = buf_half(na.n[gi], tl2, 2u * tok0);
      const uint32_t rn = ((gi == 0 && KP0) || (gi == 1 && KP1)) ? buf_half(na.r[gi], tl2, 2u * tok0) : 0u;
      kc.nr[gi][i] = nn | (rn << 16);
    }
#pragma unroll
    for (int gv = 0; gv < NV; ++gv) {
      if constexpr (!(PART & 2)) break;
      const uint32_t h = buf_half(na.nv[gv], tl2, 2u * tok0);
      kc.nv[gv][i >> 1] = (i & 1) ? (kc.nv[gv][i >> 1] | (h << 16)) : h;
    }
  }
}

// Value plane words of this wave's 32 coordinates for a chunk's two 128-token
// steps (steps wholly past the split's end are skipped where they are used;
// blocks past the sequence read 0).
struct VChunk {
  uint32_t w[2][2][4];
};

template <int NV, int VB0, int VB1>
__device__ __forceinline__ void load_v(VChunk& vc, const VAddr& va, int c0, int lane) {
  (void)lane;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const uint32_t soff = (uint32_t)((c0 >> 5) + 4 * ks) * va.tile_bytes;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint32_t voff = va.lane_off + 64u * tt * va.vB;
      if constexpr (NV == 1) {
        buf_words<VB0>(va.res, voff, soff, vc.w[ks][tt]);
#pragma unroll
        for (int pp = VB0; pp < 4; ++pp) vc.w[ks][tt][pp] = 0u;
      } else {
        constexpr int PM = VB0 > VB1 ? VB0 : VB1;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp)
          vc.w[ks][tt][pp] = pp < PM ? __builtin_amdgcn_raw_buffer_load_b32(va.res, voff + 4u * min(pp, va.vB - 1), soff, 0) : 0u;
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

template <int KB0, int KP0, int KB1, int KP1, int VB0, int VB1>
__global__ __launch_bounds__(kThreads, (KB0 >= 4 && VB0 >= 4) ? 1 : 2) void decode_kernel(Args a) {
  constexpr int NK = KB1 > 0 ? 2 : 1;
  constexpr int NV = VB1 > 0 ? 2 : 1;
  constexpr int VT = n_odd(VB0) > n_odd(VB1) ? n_odd(VB0) : n_odd(VB1);
  constexpr int NS0 = n_odd(KB0) + KP0;
  constexpr int NS = NS0 + (KB1 > 0 ? n_odd(KB1) + KP1 : 0);
  // two key groups hold more per-lane state: their keys are single-buffered
  // (refilled once a chunk's weights are formed) to stay within 2 waves/SIMD
  constexpr bool kOneK = NK == 2;
  __shared__ __attribute__((aligned(16))) uint8_t wbuf[2][NV][2][16][128];  // [buf][vgroup][step][row][kappa]
  __shared__ float red_m[4][kHT];
  __shared__ int red_e[4][NV];
  __shared__ float fin_l[4][kHT];

  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 4, tl = lane & 15;
  const int split = blockIdx.x, ht = blockIdx.y, bg = blockIdx.z;
  // the argument fields that the first loads depend on, fetched in one batch
  // (left to itself the compiler fetches them in several dependent rounds)
  asm volatile("" ::"s"(a.Hkv), "s"(a.HT), "s"(a.split_len), "s"(a.T_max), "s"(a.aops),
               "s"(a.k[0].packed), "s"(a.k[0].norm), "s"(a.k[0].rnorm), "s"(a.k[0].seq_stride), "s"(a.k[0].d),
               "s"(a.k[0].ch), "s"(a.v[0].packed), "s"(a.v[0].norm), "s"(a.v[0].seq_stride), "s"(a.v[0].d),
               "s"(a.v[0].B), "s"(a.v[0].ch), "s"(a.seq_lens), "s"(a.B), "s"(a.G), "s"(a.block_table));
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int h0 = g * a.G + ht * kHT;
  const int nh = min(kHT, a.G - ht * kHT);
  const int ts = split * a.split_len;
  // A paged cache: the split lies in one block of the sequence's block
  // table; that block's rows stand where a contiguous sequence's would
  // (pbg), token offsets count from the block's first token (tok_base), and
  // a block id outside the pool reads as empty (zero-sized resources).
  int64_t pbg = bg;
  int tok_base = 0, rel_first_last = a.T_max - 1;
  uint32_t live = 1u;
  if (a.block_table) {
    const int bi = ts / a.block_tokens;
    const int blk = a.block_table[(int64_t)b * a.max_blocks + bi];
    const bool ok = blk >= 0 && blk < a.num_blocks;
    pbg = (int64_t)(ok ? blk : 0) * a.Hkv + g;
    tok_base = bi * a.block_tokens;
    rel_first_last = a.block_tokens - 1;
    live = ok ? 1u : 0u;
  }

  // this lane's coordinate word of the key layout (score-phase B operand)
  // (group fields are selected from uniform values, never indexed per lane)
  const int W = lane >> 4;
  const bool kg1 = NK == 2 && 32 * W >= a.k[NK - 1].ch;
  KAddr ka;
#pragma unroll
  for (int gi = 0; gi < NK; ++gi) {
    const int P = gi ? (KB1 + KP1) : (KB0 + KP0);
    const int kd = a.k[gi].d, kch = a.k[gi].ch;
    const int64_t kss = a.k[gi].seq_stride;
    ka.step[gi] = (uint32_t)((kd >> 5) * 16 * P * 4);
    const uint32_t* seq = a.k[gi].packed + ((pbg * kss) >> 4) * ((kd >> 5) * 16 * P);
    ka.res[gi] = make_rsrc(seq, (uint32_t)(kss >> 4) * ka.step[gi] * live);
    const bool own = NK == 1 || (gi == 1) == kg1;
    ka.voff[gi] = own ? (uint32_t)(((W - (kch >> 5)) * 16 + tl) * P * 4) : kOutside;
  }
  NAddr na;
#pragma unroll
  for (int gi = 0; gi < NK; ++gi) {
    const uint32_t nb = (uint32_t)(2 * a.k[gi].seq_stride) * live;
    na.n[gi] = make_rsrc(a.k[gi].norm + pbg * a.k[gi].seq_stride, nb);
    na.r[gi] = make_rsrc(((gi == 0 && KP0) || (gi == 1 && KP1)) ? a.k[gi].rnorm + pbg * a.k[gi].seq_stride
                                                                 : a.k[gi].norm,
                         ((gi == 0 && KP0) || (gi == 1 && KP1)) ? nb : 0u);
  }
#pragma unroll
  for (int gv = 0; gv < NV; ++gv)
    na.nv[gv] = make_rsrc(a.v[gv].norm + pbg * a.v[gv].seq_stride, (uint32_t)(2 * a.v[gv].seq_stride) * live);
  // this wave's value coordinates 32 w .. 32 w + 31 belong to one value group
  const int vgi = (NV > 1 && 32 * w >= a.v[NV - 1].ch) ? 1 : 0;
  const VGroup& vme = a.v[vgi];
  const int vjl0 = 32 * w - vme.ch;
  VAddr va;
  va.vB = vme.B;
  va.tile_bytes = (uint32_t)(vme.d * vme.B * 4);
  va.res = make_rsrc(vme.packed + ((pbg * vme.seq_stride) >> 5) * (vme.d * vme.B),
                     (uint32_t)(vme.seq_stride >> 5) * va.tile_bytes * live);
  va.lane_off = (uint32_t)((lane >> 4) * va.tile_bytes + (vjl0 + (lane & 15)) * vme.B * 4);

  // ---- query operands of every slot and their inverse scales (built by the
  // query-transform kernels); issued before the first chunk's loads, so
  // they complete first
  const int key = bg * a.HT + ht;
  v8i aop[NS];
  int esc[NS];  // E8M0 scale of this lane's operand row and K block, per slot
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const v4i* src = reinterpret_cast<const v4i*>(a.aops + (((int64_t)key * NS + s) * 64 + lane) * 8);
    const v4i lo = src[0], hi = src[1];
    aop[s] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], 0, 0};
    esc[s] = hi[2];
  }
  // ---- the first chunk's loads: clamped to the cache's extent (T_max) rather
  // than to the sequence's length, so that they need no value read from
  // memory; tokens at or past the length are masked where they are used
  KChunk<NK, NV> kA, kB;
  VChunk vv;
  load_k<NK, NV, KB0 + KP0, KB1 + KP1, KP0, KP1>(kA, ka, na, ts - tok_base, rel_first_last, w, lane);
  load_v<NV, VB0, VB1>(vv, va, ts - tok_base, lane);
  // the sequence length, read through a buffer resource that is empty when
  // no lengths are given (the read then returns 0 without touching memory),
  // so that no branch holds the loads above behind it
  const uint32_t lraw = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
      make_rsrc(a.seq_lens, a.seq_lens ? (uint32_t)(4 * a.B) : 0u), 4u * (uint32_t)b, 0u, 0);
  // nothing below is moved above the loads
  __builtin_amdgcn_sched_barrier(0);
  const int len = max(min(max(__builtin_amdgcn_readfirstlane((int)lraw), 0), a.T_max), a.seq_lens ? 0 : a.T_max);
  const int te = min(ts + a.split_len, len);
  const int tlast = max(te, 1) - 1;
  // (loads take token offsets within the block of a paged cache)
  const int rel_last = max(tlast - tok_base, 0);
  // constant parts of the fp4 encoding, per (group, class); scales of this lane's head
  float cm[NK], cq[NK], gam[NK];
  {
    const v8i khi = key_const_hi(), klo = key_const_lo();
#pragma unroll
    for (int gi = 0; gi < NK; ++gi) {
      cm[gi] = cq[gi] = 0.f;
      gam[gi] = a.k[gi].gamma;
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int gi = s < NS0 ? 0 : 1;
      const bool q = (gi == 0) ? (KP0 && s == NS0 - 1) : (KP1 && s == NS - 1);
      const float c4 = sum4(mfma_fp6_fp4_sa(aop[s], khi, mfma_fp6_fp4_sa(aop[s], klo, v4f{0.f, 0.f, 0.f, 0.f}, esc[s]), esc[s]));
      if (q)
        cq[gi] += c4;
      else
        cm[gi] += c4;
    }
  }
  // fp4 register of this lane's tokens in the value step: token t of a
  // 64-token block sits in register (t mod 8) / 2 of its tile's expansion,
  // and this lane's tokens 64 w + 16 i + tl all have t mod 8 = tl mod 8
  const float tinv = inv_v((tl & 7) >> 1);

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
  // the weights' fourth digit rows stay zero (three digits are written)
  for (int e = tid; e < 2 * NV * 2 * 4 * 8; e += kThreads) {
    const int q16 = e & 7, rowq = (e >> 3) & 3, bsg = e >> 5;  // 16-byte piece, head, (buffer, group, step)
    *reinterpret_cast<uint4*>(&wbuf[0][0][0][0][0] + (size_t)bsg * 16 * 128 + (4 * rowq + 3) * 128 + 16 * q16) =
        make_uint4(0u, 0u, 0u, 0u);
  }
  // one 256-token chunk: kc, vc hold its data; the next chunk is prefetched
  // into kn, vn (the last chunk re-reads its own, cached, addresses so that
  // the loads stay unconditional). Called with the two buffers swapped on
  // alternate chunks, so nothing is copied.
  auto chunk = [&](auto vbt, const int c0, KChunk<NK, NV>& kc, KChunk<NK, NV>& kn, VChunk& vc)
                   __attribute__((always_inline)) {
    constexpr int VB = decltype(vbt)::value;  // value bits of this wave's coordinates
    const int cn = c0 + kChunk < te ? c0 + kChunk : c0;
    if constexpr (!kOneK) load_k<NK, NV, KB0 + KP0, KB1 + KP1, KP0, KP1>(kn, ka, na, cn - tok_base, rel_last, w, lane);

    // ---------------- scores for this wave's 64 tokens
    float lg[4], raw[4];
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
        dm[0] = mfma_fp6_fp4_sa(aop[t], expand_key_bits(word), dm[0], esc[t]);
      }
      if constexpr (KP0) dq[0] = mfma_fp6_fp4_sa(aop[NS0 - 1], expand_key_bits(wd[KB0]), dq[0], esc[NS0 - 1]);
      if constexpr (KB1 > 0) {
#pragma unroll
        for (int t = 0; t < n_odd(KB1); ++t) {
          uint32_t word = 0;
          const int m = odd_mask(KB1, t);
#pragma unroll
          for (int p = 0; p < 5; ++p)
            if ((m >> p) & 1) word ^= wd[p];
          dm[NK - 1] = mfma_fp6_fp4_sa(aop[NS0 + t], expand_key_bits(word), dm[NK - 1], esc[NS0 + t]);
        }
        if constexpr (KP1) dq[NK - 1] = mfma_fp6_fp4_sa(aop[NS - 1], expand_key_bits(wd[KB1]), dq[NK - 1], esc[NS - 1]);
      }
      float sc = 0.f;
#pragma unroll
      for (int gi = 0; gi < NK; ++gi) {
        float part = sum4(dm[gi]) - cm[gi];
        if ((gi == 0 && KP0) || (gi == 1 && KP1)) {
          const float qjl = sum4(dq[gi]) - cq[gi];
          part = fmaf(gam[gi] * hbits_hi(kc.nr[gi][i]), qjl, part);
        }
        sc = fmaf(hbits(kc.nr[gi][i]), part, sc);
      }
      const int tok = c0 + 64 * w + 16 * i + tl;
      const bool valid = tok < te && hl < nh;
      raw[i] = sc;
      lg[i] = valid ? sc * a.scale_log2 : -INFINITY;
    }
    if (a.scores_out) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = c0 + 64 * w + 16 * i + tl;
        if (tok < te && hl < nh) a.scores_out[((int64_t)b * a.Hq + h0 + hl) * a.T_max + tok] = raw[i];
      }
    }
    // (one key buffer: its plane words and key norms are used up; refill them)
    if constexpr (kOneK) load_k<NK, NV, KB0 + KP0, KB1 + KP1, KP0, KP1, 1>(kc, ka, na, cn - tok_base, rel_last, w, lane);
    // value norms of tokens at or past the split's end (rows the loads
    // re-read or the cache never wrote) are cleared before they are used:
    // token c0 + 64 w + 16 i + tl is in range iff 16 i < rem
    {
      const int rem = te - (c0 + 64 * w + tl);
      const uint32_t mk0 = (rem > 0 ? 0xffffu : 0u) | (rem > 16 ? 0xffff0000u : 0u);
      const uint32_t mk1 = (rem > 32 ? 0xffffu : 0u) | (rem > 48 ? 0xffff0000u : 0u);
#pragma unroll
      for (int gv = 0; gv < NV; ++gv) {
        kc.nv[gv][0] &= mk0;
        kc.nv[gv][1] &= mk1;
      }
    }
    // ---------------- chunk statistics shared by the four waves
    float mx = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
    mx = row16_max(mx);
    if (tl == 0) red_m[w][hl] = mx;
#pragma unroll
    for (int gv = 0; gv < NV; ++gv) {
      const uint32_t m2 = max(kc.nv[gv][0] & 0xffffu, kc.nv[gv][1] & 0xffffu);
      const uint32_t vm = wave_max64_u(max(m2, max(kc.nv[gv][0] >> 16, kc.nv[gv][1] >> 16)));
      if (lane == 0) red_e[w][gv] = exponent_of(hbits(vm));
    }
    __syncthreads();
    const float cmax = fmaxf(fmaxf(red_m[0][hl], red_m[1][hl]), fmaxf(red_m[2][hl], red_m[3][hl]));
    const float m_new = fmaxf(m_run, cmax);
    const bool live = m_new != -INFINITY;
    // (v_exp_f32 directly: arguments here are at most 0, and results below
    // the normal range are negligible beside the chunk's largest weight 1)
    const float corr = (live && m_run != -INFINITY) ? __builtin_amdgcn_exp2f(m_run - m_new) : (live ? 0.f : 1.f);
    int e_new[NV];
#pragma unroll
    for (int gv = 0; gv < NV; ++gv)
      e_new[gv] = max(max(max(red_e[0][gv], red_e[1][gv]), max(red_e[2][gv], red_e[3][gv])), e_run[gv]);
    const int eshift = (NV > 1 && vgi) ? e_run[NV - 1] - e_new[NV - 1] : e_run[0] - e_new[0];
    const float vcorr = corr * ldexpf(1.f, eshift);
    // (the first chunk of a split has nothing to rescale)
    if (c0 != ts && vcorr != 1.f) {
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
      p[i] = live ? __builtin_amdgcn_exp2f(lg[i] - m_new) : 0.f;
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
        // operand position of the token: the fp4 expansion of the words of
        // value tile s puts token t = 16 q + 8 s + 2 r + e of its block
        // (e = 0, 1) at K position 32 s + 8 r + q + 4 e of the block's 64,
        // i.e. token 16 i + tl at 4 tl + i
        const int kappa = 64 * (tp >> 6) + 4 * (tp & 15) + ((tp >> 4) & 3);
        float r = p[i] * hbits_at(kc.nv[gv][i >> 1], i & 1) * sv;
        uint8_t* dst = &wbuf[buf][gv][ks][4 * hl][kappa];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          // the residual is taken from the digit as stored: below e4m3's
          // normal range the conversion rounds the leading bits, and that
          // rounding must pass on to the next digit
          const uint32_t d8 = fp8_exact(head4(r)) & 0xffu;
          dst[128 * m] = (uint8_t)d8;
          r = (r - f32_of_fp8(d8)) * kDigitStep;
        }
        dst[256] = (uint8_t)fp8_of(r);  // the third and last digit, rounded to nearest
      }
      e_run[gv] = e_new[gv];
    }
    // (one key buffer: it is used up; refill it with the next chunk's keys)
    if constexpr (kOneK) load_k<NK, NV, KB0 + KP0, KB1 + KP1, KP0, KP1, 2>(kc, ka, na, cn - tok_base, rel_last, w, lane);
    __syncthreads();
    // ---------------- values: this wave's 32 coordinates over the 256 tokens
    // (a step past the split's end has all weights 0 and adds nothing)
    const v8i cop = const_operand();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint8_t* wrow = &wbuf[buf][vgi][ks][lane & 15][0];
      const int gp = lane >> 4;
      const v4i lo = *reinterpret_cast<const v4i*>(wrow + 16 * gp);
      const v4i hi = *reinterpret_cast<const v4i*>(wrow + 64 + 16 * gp);
      const v8i aw = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      vcon = mfma_fp8_fp4(aw, cop, vcon);
      value_step<VB, VT>(vacc, aw, vc.w[ks]);
    }
    // the value words are used: refill them with the next chunk's (they
    // arrive while its scores and weights are formed)
    load_v<NV, VB0, VB1>(vc, va, cn - tok_base, lane);
  };
  // The first chunk always runs (an empty split runs it fully masked: no
  // weight, no change to the running state), so that its loads and the
  // query-operand loads above are issued together, ahead of any branch.
  // The loop is instantiated once per value width and chosen per wave, so
  // that no branch inside it touches the value accumulators.
  auto run = [&](auto vbt) __attribute__((always_inline)) {
    int c0 = ts;
    do {
      chunk(vbt, c0, kA, kB, vv);
      c0 += kChunk;
      buf ^= 1;
      if (c0 >= te) break;
      if constexpr (kOneK)
        chunk(vbt, c0, kA, kA, vv);
      else
        chunk(vbt, c0, kB, kA, vv);
      c0 += kChunk;
      buf ^= 1;
    } while (c0 < te);
  };
  if (NV == 1 || vgi == 0)
    run(IntC<VB0>{});
  else
    run(IntC<(VB1 > 0 ? VB1 : 1)>{});

  // ---------------- partial results of this split
  float lsum = row16_sum(l_run);
  if (tl == 0) fin_l[w][hl] = lsum;
  __syncthreads();
  if (hl < nh) {
    float* part = a.partial + (((int64_t)b * a.Hq + h0 + hl) * a.splits + split) * (kD + 2);
    const int ef = (NV > 1 && vgi) ? e_run[NV - 1] : e_run[0];
    const float unscale = ldexpf(1.f, ef - 5);
    const float csub = 0.25f * wsum4(vcon) * vme.alpha_sum;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float v = -csub;
#pragma unroll
      for (int s = 0; s < VT; ++s)
        if (s < vme.ntypes) v = fmaf(vme.alpha[s], wsum4(vacc[tt][s]), v);
      // a split with no token in range leaves zeros (its weight in the merge is 0)
      part[2 + 32 * w + 16 * tt + tl] = m_run == -INFINITY ? 0.f : v * unscale;
    }
    if (w == 0 && tl == 0) {
      part[0] = m_run;
      part[1] = fin_l[0][hl] + fin_l[1][hl] + fin_l[2][hl] + fin_l[3][hl];
    }
  }
}

// ------------------------------------------------------------------ combine
// Merge the split partials (log2 domain) and rotate back with R_v^T. One
// workgroup per (batch, query head, slice of 16 output channels): it merges
// the whole rotated accumulator over the splits (the partials are re-read
// by the head's 8 workgroups, from L2) and multiplies it by the 16 columns
// of R_v it owns. All loads of the common case (up to 64 splits) are issued
// before the first result is used; indices are clamped in range and masked
// where used, so nothing waits between them.
constexpr int kCombCols = kD / 4;                    // float4 columns of a partial row
constexpr int kCombRows = kCombThreads / kCombCols;  // split rows per round of loads (8)
constexpr int kCombBatch = 8;                        // rounds held at once (64 splits)

__global__ __launch_bounds__(kCombThreads) void combine_kernel(Args a) {
  __shared__ float wsp[kMaxCombineSplits];
  __shared__ __attribute__((aligned(16))) float accp[kCombRows][kD];
  __shared__ __attribute__((aligned(16))) float acc[kD];
  __shared__ float opart[kCombThreads / kJSlice][kJSlice];
  __shared__ float wred[kCombThreads / 64], lred[kCombThreads / 64];
  const int bh = blockIdx.x, is = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float* part = a.partial + (int64_t)bh * a.splits * (kD + 2);
  const int S = a.splits;
  const int i0 = is * kJSlice;
  // the output slice lies in one value group (group sizes are multiples of 32)
  const bool g1 = a.nv > 1 && i0 >= a.v[1].ch;
  const float* Rv = g1 ? a.v[1].R : a.v[0].R;
  const int vd = g1 ? a.v[1].d : a.v[0].d, vch = g1 ? a.v[1].ch : a.v[0].ch;

  // R_v rows j (of the group) at this slice's 16 columns: thread t takes row
  // t / 16 + 16 k (k < vd / 16) and column t % 16
  const int ic = tid & (kJSlice - 1), jr = tid >> 4;
  float rcol[kD / 16];
#pragma unroll
  for (int k = 0; k < kD / 16; ++k)
    rcol[k] = Rv[(int64_t)min(jr + 16 * k, vd - 1) * vd + (i0 - vch) + ic];
  // split maxima and sums
  const int sm = min(tid, S - 1);
  const float ms0 = part[(int64_t)sm * (kD + 2)], ls0 = part[(int64_t)sm * (kD + 2) + 1];
  // accumulator rows: thread t takes float4 column t % 32 of split rows t / 32 + 8 k
  const int c4 = tid & (kCombCols - 1), sr = tid / kCombCols;
  float4 x[kCombBatch];
#pragma unroll
  for (int k = 0; k < kCombBatch; ++k) {
    const float* row = part + (int64_t)min(sr + kCombRows * k, S - 1) * (kD + 2) + 2;
    // rows are kD + 2 floats apart, so only 8-byte aligned: two 8-byte loads
    const float2 lo = *reinterpret_cast<const float2*>(row + 4 * c4);
    const float2 hi = *reinterpret_cast<const float2*>(row + 4 * c4 + 2);
    x[k] = make_float4(lo.x, lo.y, hi.x, hi.y);
  }

  float mx = tid < S ? ms0 : -INFINITY;
  for (int s2 = tid + kCombThreads; s2 < S; s2 += kCombThreads) mx = fmaxf(mx, part[(int64_t)s2 * (kD + 2)]);
  mx = tqd::wave_max(mx);
  if (lane == 0) wred[wv] = mx;
  __syncthreads();
  float M = wred[0];
#pragma unroll
  for (int k = 1; k < kCombThreads / 64; ++k) M = fmaxf(M, wred[k]);
  float lsum = 0.f;
  for (int s2 = tid; s2 < S; s2 += kCombThreads) {
    const float m = s2 == tid ? ms0 : part[(int64_t)s2 * (kD + 2)];
    const float l = s2 == tid ? ls0 : part[(int64_t)s2 * (kD + 2) + 1];
    const float wgt = (M == -INFINITY || m == -INFINITY) ? 0.f : exp2f(m - M);
    wsp[s2] = wgt;
    lsum = fmaf(wgt, l, lsum);
  }
  lsum = tqd::wave_sum(lsum);
  if (lane == 0) lred[wv] = lsum;
  __syncthreads();
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0;; s0 += kCombRows * kCombBatch) {
#pragma unroll
    for (int k = 0; k < kCombBatch; ++k) {
      const int sk = s0 + sr + kCombRows * k;
      const float wk = sk < S ? wsp[sk] : 0.f;
      v.x = fmaf(wk, x[k].x, v.x);
      v.y = fmaf(wk, x[k].y, v.y);
      v.z = fmaf(wk, x[k].z, v.z);
      v.w = fmaf(wk, x[k].w, v.w);
    }
    const int nxt = s0 + kCombRows * kCombBatch;
    if (nxt >= S) break;
#pragma unroll
    for (int k = 0; k < kCombBatch; ++k) {
      const float* row = part + (int64_t)min(nxt + sr + kCombRows * k, S - 1) * (kD + 2) + 2;
      const float2 lo = *reinterpret_cast<const float2*>(row + 4 * c4);
      const float2 hi = *reinterpret_cast<const float2*>(row + 4 * c4 + 2);
      x[k] = make_float4(lo.x, lo.y, hi.x, hi.y);
    }
  }
  *reinterpret_cast<float4*>(&accp[sr][4 * c4]) = v;
  __syncthreads();
  if (tid < kD) {
    float t = 0.f;
#pragma unroll
    for (int r = 0; r < kCombRows; ++r) t += accp[r][tid];
    acc[tid] = t;
  }
  __syncthreads();
  // out[i0 + ic] = sum_j R_v[j][i0 + ic - vch] acc[vch + j]
  float o = 0.f;
#pragma unroll
  for (int k = 0; k < kD / 16; ++k)
    if (jr + 16 * k < vd) o = fmaf(rcol[k], acc[vch + jr + 16 * k], o);
  opart[jr][ic] = o;
  __syncthreads();
  if (tid < kJSlice) {
    float t = 0.f;
#pragma unroll
    for (int r = 0; r < kCombThreads / kJSlice; ++r) t += opart[r][tid];
    const float tot = (lred[0] + lred[1]) + (lred[2] + lred[3]);
    a.out[(int64_t)bh * kD + i0 + tid] = tot > 0.f ? t / tot : 0.f;
  }
}

// Few splits (large batches): the same merge and rotation with kHeadsPerComb
// query heads per workgroup, so that R_v is read once per workgroup (into
// LDS) instead of once per head and channel slice. Thread t of head
// t / 32 merges channels 4 (t % 32) .. + 3 over the splits, then forms the
// same 4 output channels from the merged accumulator and R_v's columns.
constexpr int kHeadsPerComb = kCombThreads / 32;
constexpr int kFewSplits = 8;

__global__ __launch_bounds__(kCombThreads) void combine_heads_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) float rv[kD * kD];  // the value groups' R_v, one after the other
  __shared__ __attribute__((aligned(16))) float accs[kHeadsPerComb][kD];
  __shared__ float tots[kHeadsPerComb];
  const int tid = threadIdx.x, hh = tid >> 5, c = tid & 31;
  const int S = a.splits;
  const int64_t bh = (int64_t)blockIdx.x * kHeadsPerComb + hh;
  const bool live = bh < (int64_t)a.B * a.Hq;
  // R_v of every value group into LDS
  int off[kMaxVG];
  {
    int o = 0;
#pragma unroll
    for (int g = 0; g < kMaxVG; ++g) {
      off[g] = o;
      if (g < a.nv) {
        const int dg = a.v[g].d;
        const float4* src = reinterpret_cast<const float4*>(a.v[g].R);
        for (int e = tid; e < dg * dg / 4; e += kCombThreads) *reinterpret_cast<float4*>(&rv[o + 4 * e]) = src[e];
        o += dg * dg;
      }
    }
  }
  // merge this head's splits (channels 4 c .. 4 c + 3)
  const float* part = a.partial + (live ? bh : 0) * S * (kD + 2);
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, part[(int64_t)s * (kD + 2)]);
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  float tot = 0.f;
  for (int s = 0; s < S; ++s) {
    const float* row = part + (int64_t)s * (kD + 2);
    const float m = row[0];
    const float wgt = (M == -INFINITY || m == -INFINITY) ? 0.f : exp2f(m - M);
    tot = fmaf(wgt, row[1], tot);
    const float2 lo = *reinterpret_cast<const float2*>(row + 2 + 4 * c);
    const float2 hi = *reinterpret_cast<const float2*>(row + 4 + 4 * c);
    v.x = fmaf(wgt, lo.x, v.x);
    v.y = fmaf(wgt, lo.y, v.y);
    v.z = fmaf(wgt, hi.x, v.z);
    v.w = fmaf(wgt, hi.y, v.w);
  }
  *reinterpret_cast<float4*>(&accs[hh][4 * c]) = v;
  if (c == 0) tots[hh] = tot;
  __syncthreads();
  // out[i] = sum_j R_v[j][i - ch] acc[ch + j] over i's value group
  const int i0 = 4 * c;
  const int g = (a.nv > 1 && i0 >= a.v[1].ch) ? 1 : 0;
  const int dg = g ? a.v[1].d : a.v[0].d, ch = g ? a.v[1].ch : 0, og = g ? off[1] : off[0];
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < dg; ++j) {
    const float4 r = *reinterpret_cast<const float4*>(&rv[og + j * dg + (i0 - ch)]);
    const float x = accs[hh][ch + j];
    o.x = fmaf(r.x, x, o.x);
    o.y = fmaf(r.y, x, o.y);
    o.z = fmaf(r.z, x, o.z);
    o.w = fmaf(r.w, x, o.w);
  }
  const float t = tots[hh];
  if (live) {
    const float inv = t > 0.f ? 1.f / t : 0.f;
    *reinterpret_cast<float4*>(a.out + bh * kD + i0) = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  }
}

// ------------------------------------------------------------------ two-wave decode
// A workgroup of two waves walks 128-token chunks of its split. Per chunk:
//  * wave w scores 4 of the chunk's 8 key tiles (16 tokens each) on the
//    fp8 x fp4 matrix cores as above: tiles 4 w .. 4 w + 3, the 64-token
//    block w of the chunk, whose tokens fill the value operand's K blocks
//    2 w and 2 w + 1 (32 positions each, the unit of its per-lane scale);
//    lane (h, c) = (lane / 16, lane % 16) ends with the scores of tokens
//    64 w + 16 j + c (j = 0..3) for head h;
//  * each wave turns its softmax weights times the value norm into three
//    fp8 digits per token (each the rounding of 16 times what the previous
//    ones left), four tokens per conversion pair: the value layout puts
//    token 16 j + c of a 64-token block at K position 4 c + j of the
//    block's 64 (the two tiles of a block interleave its tokens), so a
//    lane's four tokens are one digit row's 4 consecutive operand bytes,
//    stored with one 32-bit LDS write per digit;
//  * one barrier; each wave reads the whole weight operand (two 16-byte LDS
//    reads per value group) and accumulates the value sums of its 64 value
//    coordinates (4 tiles of 16) over the chunk's 128 tokens.
// Each wave keeps its own weight reference per head: its running maximum of
// the logits (log2 domain) rounded up to an integer, and per value group the
// running maximum exponent of the value norms. The value accumulators keep
// the references both waves reported at the first chunk; a wave's later
// weights enter the matrix cores with the difference as a power-of-two
// (E8M0) operand scale per lane, so the accumulators are never rescaled in
// the loop (only if a reference ran more than kMaxShift above them).
constexpr int kPChunk = 128;
constexpr int kPThreads = 128;
constexpr int kWRow = 144;    // bytes per digit row of the weight operand in LDS (conflict-free, 16-byte aligned)
constexpr int kWScale = 6;    // weight (<= 1) x value norm x 2^(kWScale - its exponent) x fp4 pre-scale (<= 4) < 256
constexpr int kMaxShift = 60;  // largest reference difference carried by the operand scale

// Three fp8 digits of two non-negative values a, b into half HI of the
// dwords x[0..2]: digit m of a and b in bytes 2 HI and 2 HI + 1 of x[m],
// digit m the e4m3 rounding (to nearest) of 16^m times what the digits
// before it left (taken from the digits as stored). The low half clears
// the dwords' high half.
template <bool HI>
__device__ __forceinline__ void digits3(float a, float b, uint32_t (&x)[3]) {
  typedef float f2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    x[m] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, HI ? (int)x[m] : 0, HI);
    if (m < 2) {
      const f2 f = __builtin_amdgcn_cvt_pk_f32_fp8((int)x[m], HI);
      a = (a - f[0]) * kDigitStep;
      b = (b - f[1]) * kDigitStep;
    }
  }
}

// Chunk tile j (0..3) of wave w: 4 w + j.
__device__ __forceinline__ int ptile(int w, int j) { return 4 * w + j; }

template <int NK>
struct PKeys {
  uint32_t kw[4][5];  // key plane words of the lane's coordinate word, token c of each of the wave's tiles
  // (norms are kept as loaded, one half per register: packing or widening
  // them right after the load would wait for the loads in flight)
  uint16_t nn[NK][4];  // key norm (half bits), token c of each of the wave's tiles
  uint16_t rn[NK][4];  // residual norm (half bits; groups with the sketch)
};
template <int NV>
struct PVals {
  uint16_t nv[NV][4];  // value norms (half bits), token c of each of the wave's tiles
  uint32_t vw[4][3];  // value plane words of the wave's 4 coordinate tiles
};

template <int NK, int P0, int P1, int KP0, int KP1>
__device__ __forceinline__ void pload_keys(PKeys<NK>& dt, const KAddr& ka, const NAddr& na, int c0, int tlast,
                                           int w, int lane, bool g1) {
  const int last_tile = tlast >> 4;
  const uint32_t tl2 = 2u * (lane & 15);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t tile = (uint32_t)min((c0 >> 4) + ptile(w, j), last_tile);
    if constexpr (NK == 1) {
      buf_words<P0>(ka.res[0], ka.voff[0], tile * ka.step[0], dt.kw[j]);
    } else {
      // each lane loads its own group's words (two loads under complementary
      // lane masks into the same registers: nothing merges the groups' words
      // after the loads)
      uint32_t wv[5];
      if (g1) {
        buf_words<P1>(ka.res[1], ka.voff[1], tile * ka.step[1], wv);
#pragma unroll
        for (int pp = P1; pp < 5; ++pp) wv[pp] = 0u;
      } else {
        buf_words<P0>(ka.res[0], ka.voff[0], tile * ka.step[0], wv);
#pragma unroll
        for (int pp = P0; pp < 5; ++pp) wv[pp] = 0u;
      }
#pragma unroll
      for (int pp = 0; pp < 5; ++pp) dt.kw[j][pp] = wv[pp];
    }
#pragma unroll
    for (int gi = 0; gi < NK; ++gi) {
      dt.nn[gi][j] = __builtin_amdgcn_raw_buffer_load_b16(na.n[gi], tl2, 32u * tile, 0);
      dt.rn[gi][j] = ((gi == 0 && KP0) || (gi == 1 && KP1)) ? __builtin_amdgcn_raw_buffer_load_b16(na.r[gi], tl2, 32u * tile, 0)
                                                             : (uint16_t)0;
    }
  }
}

template <int NV>
__device__ __forceinline__ void pload_vnorms(PVals<NV>& dt, const NAddr& na, int c0, int tlast, int w, int lane) {
  const int last_tile = tlast >> 4;
  const uint32_t tl2 = 2u * (lane & 15);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t tile = (uint32_t)min((c0 >> 4) + ptile(w, j), last_tile);
#pragma unroll
    for (int gv = 0; gv < NV; ++gv) {
      dt.nv[gv][j] = __builtin_amdgcn_raw_buffer_load_b16(na.nv[gv], tl2, 32u * tile, 0);
    }
  }
}

// Value words of the wave's coordinate tiles (global tiles 4 W + j, value
// group G[j] with B[j] planes): this lane's coordinate (lane % 16) and
// 32-token block (lane / 16) of the chunk.
template <int NV, int W, int G0, int G1, int G2, int G3, int B0, int B1, int B2, int B3>
__device__ __forceinline__ void pload_values(PVals<NV>& dt, const rsrc_t (&vres)[2], const uint32_t (&vtile_bytes)[2],
                                             const uint32_t (&voff)[4], int c0) {
  constexpr int Gs[4] = {G0, G1, G2, G3}, Bs[4] = {B0, B1, B2, B3};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t soff = (uint32_t)(c0 >> 5) * vtile_bytes[Gs[j]];
    if (Bs[j] == 3) {  // (constant once the loop is unrolled)
      buf_words<3>(vres[Gs[j]], voff[j], soff, dt.vw[j]);
    } else if (Bs[j] == 2) {
      buf_words<2>(vres[Gs[j]], voff[j], soff, dt.vw[j]);
      dt.vw[j][2] = 0u;
    } else {
      buf_words<1>(vres[Gs[j]], voff[j], soff, dt.vw[j]);
      dt.vw[j][1] = dt.vw[j][2] = 0u;
    }
  }
}

// CT1: first 16-coordinate tile of value group 1 (8 with one value group);
// two key groups split at a channel that is a multiple of 32.
template <int KB0, int KP0, int KB1, int KP1, int VB0, int VB1, int CT1>
__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void pair_decode_kernel(Args a) {
  constexpr int NK = KB1 > 0 ? 2 : 1;
  constexpr int NV = VB1 > 0 ? 2 : 1;
  constexpr int NS0 = n_odd(KB0) + KP0;
  constexpr int NS = NS0 + (KB1 > 0 ? n_odd(KB1) + KP1 : 0);
  constexpr int P0 = KB0 + KP0, P1 = KB1 + KP1;
  __shared__ __attribute__((aligned(16))) uint8_t wbuf[2][NV][16 * kWRow];
  __shared__ float xm[2][2][kHT];  // [parity][wave][head] weight references (log2, integer-valued)
  __shared__ int xe[2][2][2];      // [parity][wave][value group] value-norm exponents
  __shared__ float xl[2][kHT];     // [wave][head] final sums

  const int tid = threadIdx.x, lane = tid & 63;
  // The two roles differ in value work (with the outlier split, role 0 sums
  // the 3-bit tiles); alternating them between neighbouring workgroups puts
  // both roles on each SIMD (about 1% faster than a fixed assignment).
  const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6) ^ (lin & 1);
  const int hl = lane >> 4, tl = lane & 15;
  const int split = blockIdx.x, ht = blockIdx.y, bg = blockIdx.z;
  asm volatile("" ::"s"(a.Hkv), "s"(a.HT), "s"(a.split_len), "s"(a.T_max), "s"(a.aops),
               "s"(a.k[0].packed), "s"(a.k[0].norm), "s"(a.k[0].rnorm), "s"(a.k[0].seq_stride), "s"(a.k[0].d),
               "s"(a.k[0].ch), "s"(a.v[0].packed), "s"(a.v[0].norm), "s"(a.v[0].seq_stride), "s"(a.v[0].d),
               "s"(a.v[0].B), "s"(a.v[0].ch), "s"(a.seq_lens), "s"(a.B), "s"(a.G), "s"(a.block_table));
  const int b = bg / a.Hkv, g = bg - b * a.Hkv;
  const int h0 = g * a.G + ht * kHT;
  const int nh = min(kHT, a.G - ht * kHT);
  const int ts = split * a.split_len;
  int64_t pbg = bg;
  int tok_base = 0, rel_first_last = a.T_max - 1;
  uint32_t live_blk = 1u;
  if (a.block_table) {
    const int bi = ts / a.block_tokens;
    const int blk = a.block_table[(int64_t)b * a.max_blocks + bi];
    const bool ok = blk >= 0 && blk < a.num_blocks;
    pbg = (int64_t)(ok ? blk : 0) * a.Hkv + g;
    tok_base = bi * a.block_tokens;
    rel_first_last = a.block_tokens - 1;
    live_blk = ok ? 1u : 0u;
  }
  // key words: lane group W = lane / 16 reads coordinate word W
  const int W = lane >> 4;
  const bool kg1 = NK == 2 && 32 * W >= a.k[NK - 1].ch;
  KAddr ka;
#pragma unroll
  for (int gi = 0; gi < NK; ++gi) {
    const int P = gi ? P1 : P0;
    const int kd = a.k[gi].d, kch = a.k[gi].ch;
    const int64_t kss = a.k[gi].seq_stride;
    ka.step[gi] = (uint32_t)((kd >> 5) * 16 * P * 4);
    const uint32_t* seq = a.k[gi].packed + ((pbg * kss) >> 4) * ((kd >> 5) * 16 * P);
    ka.res[gi] = make_rsrc(seq, (uint32_t)(kss >> 4) * ka.step[gi] * live_blk);
    const bool own = NK == 1 || (gi == 1) == kg1;
    ka.voff[gi] = own ? (uint32_t)(((W - (kch >> 5)) * 16 + tl) * P * 4) : kOutside;
  }
  NAddr na;
#pragma unroll
  for (int gi = 0; gi < NK; ++gi) {
    const uint32_t nb = (uint32_t)(2 * a.k[gi].seq_stride) * live_blk;
    na.n[gi] = make_rsrc(a.k[gi].norm + pbg * a.k[gi].seq_stride, nb);
    const bool pr = (gi == 0 && KP0) || (gi == 1 && KP1);
    na.r[gi] = make_rsrc(pr ? a.k[gi].rnorm + pbg * a.k[gi].seq_stride : a.k[gi].norm, pr ? nb : 0u);
  }
  rsrc_t vres[2];
  uint32_t vtile_bytes[2];
#pragma unroll
  for (int gv = 0; gv < 2; ++gv) {
    const VGroup& vg = a.v[NV > 1 ? gv : 0];
    na.nv[gv < NV ? gv : 0] = make_rsrc(vg.norm + pbg * vg.seq_stride, (uint32_t)(2 * vg.seq_stride) * live_blk);
    vtile_bytes[gv] = (uint32_t)(vg.d * vg.B * 4);
    vres[gv] = make_rsrc(vg.packed + ((pbg * vg.seq_stride) >> 5) * (vg.d * vg.B),
                         (uint32_t)(vg.seq_stride >> 5) * vtile_bytes[gv] * live_blk);
  }

  // query operands of every slot and their scales (from the query transform)
  const int key = bg * a.HT + ht;
  v8i aop[NS];
  int esc[NS];  // E8M0 scale of this lane's operand row and K block, per slot
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const v4i* src = reinterpret_cast<const v4i*>(a.aops + (((int64_t)key * NS + s) * 64 + lane) * 8);
    const v4i lo = src[0], hi = src[1];
    aop[s] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], 0, 0};
    esc[s] = hi[2];
  }
  PKeys<NK> kA;
  PVals<NV> vd;
  pload_keys<NK, P0, P1, KP0, KP1>(kA, ka, na, ts - tok_base, rel_first_last, w, lane, kg1);
  pload_vnorms<NV>(vd, na, ts - tok_base, rel_first_last, w, lane);
  const uint32_t lraw = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
      make_rsrc(a.seq_lens, a.seq_lens ? (uint32_t)(4 * a.B) : 0u), 4u * (uint32_t)b, 0u, 0);
  __builtin_amdgcn_sched_barrier(0);
  const int len = max(min(max(__builtin_amdgcn_readfirstlane((int)lraw), 0), a.T_max), a.seq_lens ? 0 : a.T_max);
  const int te = min(ts + a.split_len, len);
  const int tlast = max(te, 1) - 1;
  const int rel_last = max(tlast - tok_base, 0);

  // constant part of the fp4 encoding per (group, class), as the initial
  // value of each score accumulator (its four digit rows sum to -constant)
  v4f cinit_m[NK], cinit_q[NK];
  float gam[NK];
  {
    const v8i khi = key_const_hi(), klo = key_const_lo();
#pragma unroll
    for (int gi = 0; gi < NK; ++gi) {
      cinit_m[gi] = cinit_q[gi] = v4f{0.f, 0.f, 0.f, 0.f};
      gam[gi] = a.k[gi].gamma;
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int gi = s < NS0 ? 0 : 1;
      const bool q = (gi == 0) ? (KP0 && s == NS0 - 1) : (KP1 && s == NS - 1);
      const v4f c = mfma_fp6_fp4_sa(aop[s], khi, mfma_fp6_fp4_sa(aop[s], klo, v4f{0.f, 0.f, 0.f, 0.f}, esc[s]), esc[s]);
      if (q)
        cinit_q[gi] -= c;
      else
        cinit_m[gi] -= c;
    }
  }
  // fp4 register of this lane's tokens in the value step: token t of a
  // 64-token block lies in register (t mod 8) / 2 of its tile's expansion,
  // and the lane's tokens 16 j + tl all have t mod 8 = tl mod 8
  const float tinv = inv_v((tl & 7) >> 1);
  const int dg_row = lane & 3;             // digit of this lane's row of the weight operand (row lane % 16)
  const int h_row = (lane & 15) >> 2;      // head of that row
  // The E8M0 scale a lane gives the A operand covers the 32 consecutive K
  // positions of block lane / 16 (measured on gfx950), here K blocks of the
  // chunk's 64-token block lane / 32: written by wave lane / 32
  const int src_w = (lane >> 5) & 1;
  // digit row 3 of every head stays zero (three digits per weight)
  // (thread tid: head tid / 32, dword tid % 32 of the row, in each buffer)
  static_assert(kPThreads == kHT * kPChunk / 4, "one dword of a zero row per thread");
#pragma unroll
  for (int k = 0; k < 2 * NV; ++k)
    *reinterpret_cast<uint32_t*>(&wbuf[k / NV][k % NV][(4 * (tid >> 5) + 3) * kWRow + 4 * (tid & 31)]) = 0u;

  // ---- the wave's loop, instantiated per wave (its value tiles' groups and
  // widths are compile-time)
  auto run = [&](auto wt) __attribute__((always_inline)) {
    constexpr int WW = decltype(wt)::value;
    constexpr int G0 = (NV > 1 && 4 * WW + 0 >= CT1) ? 1 : 0, G1 = (NV > 1 && 4 * WW + 1 >= CT1) ? 1 : 0;
    constexpr int G2 = (NV > 1 && 4 * WW + 2 >= CT1) ? 1 : 0, G3 = (NV > 1 && 4 * WW + 3 >= CT1) ? 1 : 0;
    constexpr int Gs[4] = {G0, G1, G2, G3};
    constexpr int B0 = G0 ? VB1 : VB0, B1 = G1 ? VB1 : VB0, B2 = G2 ? VB1 : VB0, B3 = G3 ? VB1 : VB0;
    constexpr int Bs[4] = {B0, B1, B2, B3};
    constexpr int T0 = n_odd(B0), T1 = n_odd(B1), T2 = n_odd(B2), T3 = n_odd(B3);
    constexpr int Ts[4] = {T0, T1, T2, T3};
    constexpr int TM = n_odd(VB0 > VB1 ? VB0 : VB1);
    uint32_t voff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const VGroup& vg = a.v[Gs[j]];
      voff[j] = (uint32_t)((lane >> 4) * vtile_bytes[Gs[j]] + (16 * (4 * WW + j) - vg.ch + (lane & 15)) * Bs[j] * 4);
    }
    pload_values<NV, WW, G0, G1, G2, G3, B0, B1, B2, B3>(vd, vres, vtile_bytes, voff, ts - tok_base);
    // value accumulators [tile][Walsh term]: rows (head, digit), columns the
    // tile's 16 coordinates; constant parts per value group
    v4f vacc[4][TM], vcon[NV];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < TM; ++t) vacc[j][t] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gv = 0; gv < NV; ++gv) vcon[gv] = v4f{0.f, 0.f, 0.f, 0.f};
    // this wave's weight references (per lane: head hl), sum of its weights
    float m_w = -INFINITY, l_w = 0.f;
    int e_w[NV];
#pragma unroll
    for (int gv = 0; gv < NV; ++gv) e_w[gv] = -60;
    // the accumulators' references (the same in both waves): per head, and
    // per value group
    // (per lane: the reference of the head of its operand row, h_row, and of
    // its accumulator rows, hl)
    float macc_row = -INFINITY, macc_out = -INFINITY;
    int e_acc[NV];
#pragma unroll
    for (int gv = 0; gv < NV; ++gv) e_acc[gv] = -60;
    int par = 0;

    auto chunk = [&](const int c0, PKeys<NK>& dc) __attribute__((always_inline)) {
      // (wave-uniform) the chunk holds tokens at or past the split's end, or
      // the group has fewer than kHT heads: only then is anything masked
      const bool tail = c0 + kPChunk > te || nh < kHT;
      const int cn = c0 + kPChunk < te ? c0 + kPChunk : c0;
      // ---------------- scores of the wave's 4 tiles
      float lg[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t(&wd)[5] = dc.kw[j];
        v4f dm[NK], dq[NK];
#pragma unroll
        for (int gi = 0; gi < NK; ++gi) {
          dm[gi] = cinit_m[gi];
          dq[gi] = cinit_q[gi];
        }
#pragma unroll
        for (int t = 0; t < n_odd(KB0); ++t) {
          uint32_t word = 0;
          const int m = odd_mask(KB0, t);
#pragma unroll
          for (int p = 0; p < 5; ++p)
            if ((m >> p) & 1) word ^= wd[p];
          dm[0] = mfma_fp6_fp4_sa(aop[t], expand_key_bits(word), dm[0], esc[t]);
        }
        if constexpr (KP0) dq[0] = mfma_fp6_fp4_sa(aop[NS0 - 1], expand_key_bits(wd[KB0]), dq[0], esc[NS0 - 1]);
        if constexpr (KB1 > 0) {
#pragma unroll
          for (int t = 0; t < n_odd(KB1); ++t) {
            uint32_t word = 0;
            const int m = odd_mask(KB1, t);
#pragma unroll
            for (int p = 0; p < 5; ++p)
              if ((m >> p) & 1) word ^= wd[p];
            dm[NK - 1] = mfma_fp6_fp4_sa(aop[NS0 + t], expand_key_bits(word), dm[NK - 1], esc[NS0 + t]);
          }
          if constexpr (KP1)
            dq[NK - 1] = mfma_fp6_fp4_sa(aop[NS - 1], expand_key_bits(wd[KB1]), dq[NK - 1], esc[NS - 1]);
        }
        float sc = 0.f;
#pragma unroll
        for (int gi = 0; gi < NK; ++gi) {
          float part = sum4(dm[gi]);
          if ((gi == 0 && KP0) || (gi == 1 && KP1)) part = fmaf(gam[gi] * hbits(dc.rn[gi][j]), sum4(dq[gi]), part);
          sc = fmaf(hbits(dc.nn[gi][j]), part, sc);
        }
        lg[j] = sc;
      }
      if (a.scores_out) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int tok = c0 + 16 * ptile(WW, j) + tl;
          if (tok < te && hl < nh) a.scores_out[((int64_t)b * a.Hq + h0 + hl) * a.T_max + tok] = lg[j];
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) lg[j] *= a.scale_log2;
      if (tail) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int tok = c0 + 16 * ptile(WW, j) + tl;
          if (!(tok < te && hl < nh)) lg[j] = -INFINITY;
        }
      }
      // the key words and norms are used up: the next chunk's go to the same
      // registers, arriving while this chunk's weights and value sums run
      pload_keys<NK, P0, P1, KP0, KP1>(dc, ka, na, cn - tok_base, rel_last, WW, lane, kg1);
      // value norms of tokens at or past the split's end are cleared
      if (tail) {
        const int rem = te - (c0 + tl);  // token c0 + 16 T + tl is in range iff 16 T < rem
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool in = rem > 16 * ptile(WW, j);
#pragma unroll
          for (int gv = 0; gv < NV; ++gv) vd.nv[gv][j] = in ? vd.nv[gv][j] : (uint16_t)0;
        }
      }
      // ---------------- this wave's references: running maximum (rounded up
      // to an integer) and value-norm exponents
      float mx = fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3]));
      mx = row16_max(mx);
      if (mx > m_w) {
        const float mn = ceilf(mx);
        l_w = m_w == -INFINITY ? 0.f : l_w * __builtin_amdgcn_exp2f(m_w - mn);
        m_w = mn;
      }
#pragma unroll
      for (int gv = 0; gv < NV; ++gv) {
        // (every 16-lane row holds the same 16 tokens of each tile: a row
        // maximum is the wave's)
        uint32_t vm = max(max(vd.nv[gv][0], vd.nv[gv][1]), max(vd.nv[gv][2], vd.nv[gv][3]));  // (16-bit maxima)
        vm = max(vm, row_ror_u<8>(vm));
        vm = max(vm, row_ror_u<4>(vm));
        vm = max(vm, row_ror_u<2>(vm));
        vm = max(vm, row_ror_u<1>(vm));
        e_w[gv] = max(e_w[gv], exponent_of(hbits(vm)));
      }
      const bool live = m_w != -INFINITY;
      // ---------------- weights -> fp8 digits -> the operand rows in LDS
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = live ? __builtin_amdgcn_exp2f(lg[j] - m_w) : 0.f;
        l_w += p[j];
      }
      // this lane's operand bytes in the rows of head hl. With one value
      // group they are recomputed in every chunk from the lane index: the
      // compiler otherwise holds the offset through the loop, spills it
      // (those layouts have the widest key and value codes) and reloads it
      // behind the loads in flight.
      int wofs = 4 * hl * kWRow + 4 * tl + 64 * WW;
      if constexpr (NV == 1) {
        uint32_t ones = ~0u;
        asm volatile("" : "+s"(ones));
        const int wl = (int)__builtin_amdgcn_mbcnt_hi(ones, __builtin_amdgcn_mbcnt_lo(ones, 0u));
        wofs = (wl >> 4) * (4 * kWRow) + 4 * (wl & 15) + 64 * WW;
      }
#pragma unroll
      for (int gv = 0; gv < NV; ++gv) {
        // value-norm scale times the fp4 pre-scale; tokens in pairs, the
        // second pair's digits into the dwords' high halves
        const float st = ldexpf(tinv, kWScale - e_w[gv]);
        uint32_t x[3];
        digits3<false>((p[0] * st) * hbits(vd.nv[gv][0]), (p[1] * st) * hbits(vd.nv[gv][1]), x);
        digits3<true>((p[2] * st) * hbits(vd.nv[gv][2]), (p[3] * st) * hbits(vd.nv[gv][3]), x);
        // rows (head hl, digit m), operand bytes 64 WW + 4 tl .. + 3
#pragma unroll
        for (int m = 0; m < 3; ++m) *reinterpret_cast<uint32_t*>(&wbuf[par][gv][wofs + m * kWRow]) = x[m];
      }
      if (tl == 0) xm[par][WW][hl] = m_w;
      if (lane == 0) {
#pragma unroll
        for (int gv = 0; gv < NV; ++gv) xe[par][WW][gv] = e_w[gv];
      }
      pload_vnorms<NV>(vd, na, cn - tok_base, rel_last, WW, lane);  // the value norms are used up
      __syncthreads();
      // ---------------- the weight operand and its per-lane scales
      v8i aw[NV];
#pragma unroll
      for (int gv = 0; gv < NV; ++gv) {
        const uint8_t* row = &wbuf[par][gv][(lane & 15) * kWRow];
        const v4i lo = *reinterpret_cast<const v4i*>(row + 16 * (lane >> 4));
        const v4i hi = *reinterpret_cast<const v4i*>(row + 64 + 16 * (lane >> 4));
        aw[gv] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      // the two waves' references, each lane reading those of its operand
      // row's head and of its accumulator rows' head (the value-norm
      // exponents are per group)
      const float mr0 = xm[par][0][h_row], mr1 = xm[par][1][h_row];
      const float mo0 = xm[par][0][hl], mo1 = xm[par][1][hl];
      int es[2][NV];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int gv = 0; gv < NV; ++gv) es[s][gv] = xe[par][s][gv];
      // the accumulators' references: set at a head's first reported maximum
      // (its accumulator rows are still zero then); raised, with a rescale,
      // only when a wave's reference runs more than kMaxShift above them
      const float mh_row = fmaxf(mr0, mr1), mh_out = fmaxf(mo0, mo1);
      if (macc_row == -INFINITY) macc_row = mh_row;
      if (macc_out == -INFINITY) macc_out = mh_out;
      bool over = mh_row - macc_row > (float)kMaxShift;  // (every head is some lane's operand-row head)
#pragma unroll
      for (int gv = 0; gv < NV; ++gv) {
        const int eh = max(es[0][gv], es[1][gv]);
        if (e_acc[gv] == -60) e_acc[gv] = eh;
        over |= eh - e_acc[gv] > kMaxShift;
      }
      if (__builtin_amdgcn_ballot_w64(over) != 0) {  // (wave-uniform) move the references up to the reported ones
        const float fl = macc_out == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(macc_out - fmaxf(mh_out, macc_out));
        macc_out = fmaxf(mh_out, macc_out);
        macc_row = fmaxf(mh_row, macc_row);
        float fe[NV];
#pragma unroll
        for (int gv = 0; gv < NV; ++gv) {
          const int eh = max(max(es[0][gv], es[1][gv]), e_acc[gv]);
          fe[gv] = ldexpf(1.f, e_acc[gv] - eh);
          e_acc[gv] = eh;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int t = 0; t < TM; ++t)
            if (t < Ts[j]) vacc[j][t] *= fl * fe[Gs[j]];
#pragma unroll
        for (int gv = 0; gv < NV; ++gv) vcon[gv] *= fl * fe[gv];
      }
      // this lane's operand scale: digit 16^-dg times 2^(reference shift) of
      // the wave that wrote its columns
      int sa[NV];
      {
        const float msrc = src_w ? mr1 : mr0;
        // (a source without any weight yet, or a masked head, has all-zero
        // digits: any scale will do; one far below the reference has
        // negligible weights, and its scale is clamped into E8M0's range)
        const int dm = (msrc == -INFINITY || macc_row == -INFINITY) ? 0 : (int)(msrc - macc_row);
#pragma unroll
        for (int gv = 0; gv < NV; ++gv)
          sa[gv] = min(max(127 - 4 * dg_row + dm + (src_w ? es[1][gv] : es[0][gv]) - e_acc[gv], 1), 254);
      }
      // ---------------- value sums of the wave's 4 coordinate tiles
      const v8i cop = const_operand();
#pragma unroll
      for (int gv = 0; gv < NV; ++gv) vcon[gv] = mfma_fp8_fp4_sa(aw[gv], cop, vcon[gv], sa[gv]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int t = 0; t < Ts[j]; ++t) {
          uint32_t word = 0;
          const int m = odd_mask(Bs[j], t);
#pragma unroll
          for (int p = 0; p < 3; ++p)
            if ((m >> p) & 1) word ^= vd.vw[j][p];
          vacc[j][t] = mfma_fp8_fp4_sa(aw[Gs[j]], expand_bits(word), vacc[j][t], sa[Gs[j]]);
        }
      }
      pload_values<NV, WW, G0, G1, G2, G3, B0, B1, B2, B3>(vd, vres, vtile_bytes, voff, cn - tok_base);
      par ^= 1;
    };
    int c0 = ts;
    // Wave priority falls by one step per quarter of the split. The SIMD
    // issues the older of two ready waves first, so the workgroups that a
    // compute unit received first ran ahead and the last ones set the
    // kernel's end (measured: equal work ended over 1105-1450 us); a wave
    // that is ahead now yields to those behind it. Only issue order
    // changes, never the results.
    const int qsh = 31 - __builtin_clz(max((te - ts) / (4 * kPChunk), 1));  // a quarter, as a shift
    int pr = 3;
    __builtin_amdgcn_s_setprio(3);
    do {  // (an empty split still runs one chunk, all of it masked)
      const int want = 3 - min(((c0 - ts) / kPChunk) >> qsh, 3);
      if (want != pr) {
        pr = want;
        if (pr == 2)
          __builtin_amdgcn_s_setprio(2);
        else if (pr == 1)
          __builtin_amdgcn_s_setprio(1);
        else
          __builtin_amdgcn_s_setprio(0);
      }
      chunk(c0, kA);
      c0 += kPChunk;
    } while (c0 < te);

    // ---------------- this split's partial results: the sum of weights of
    // both waves relative to the accumulators' reference
    const float lsum = row16_sum(l_w);
    if (tl == 0) {
      xl[WW][hl] = lsum;
      xm[par][WW][hl] = m_w;
    }
    __syncthreads();
    if (hl < nh) {
      const float macc = macc_out;
      float* part = a.partial + (((int64_t)b * a.Hq + h0 + hl) * a.splits + split) * (kD + 2);
      const bool none = macc == -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const VGroup& vg = a.v[Gs[j]];
        const float csub = 0.25f * sum4(vcon[Gs[j]]) * vg.alpha_sum;
        float v = -csub;
#pragma unroll
        for (int t = 0; t < Ts[j]; ++t) v = fmaf(vg.alpha[t], sum4(vacc[j][t]), v);
        part[2 + 16 * (4 * WW + j) + tl] = none ? 0.f : v * ldexpf(1.f, e_acc[Gs[j]] - kWScale);
      }
      if (WW == 0 && tl == 0) {
        float l = 0.f;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const float msw = xm[par][s][hl];
          if (msw != -INFINITY && !none) l += xl[s][hl] * __builtin_amdgcn_exp2f(msw - macc);
        }
        part[0] = macc;
        part[1] = l;
      }
    }
  };
  if (w == 0)
    run(IntC<0>{});
  else
    run(IntC<1>{});
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
  int kb0, kp0, kb1, kp1, vb0, vb1;
  KernelFn fn;
};

#define TQ_SPEC(a, b, c, d, e, f) Spec{a, b, c, d, e, f, decode_kernel<a, b, c, d, e, f>}
// Layouts compiled for the matrix-core decode: keys in one group of 1-4 bits
// with or without QJL and values of 2-4 bits (including MSE-only keys at 2-4
// bits and asymmetric key/value widths), plus the 2.5-bit outlier-channel
// split (32 + 96 channels). Other layouts of 128-channel heads run on the
// general kernel.
const Spec kSpecs[] = {
    TQ_SPEC(1, 1, 0, 0, 1, 0), TQ_SPEC(1, 1, 0, 0, 2, 0), TQ_SPEC(2, 1, 0, 0, 2, 0), TQ_SPEC(3, 1, 0, 0, 2, 0),
    TQ_SPEC(1, 1, 0, 0, 3, 0), TQ_SPEC(2, 1, 0, 0, 3, 0), TQ_SPEC(3, 1, 0, 0, 3, 0),
    TQ_SPEC(1, 1, 0, 0, 4, 0), TQ_SPEC(2, 1, 0, 0, 4, 0), TQ_SPEC(3, 1, 0, 0, 4, 0),
    TQ_SPEC(4, 1, 0, 0, 4, 0), TQ_SPEC(4, 0, 0, 0, 4, 0), TQ_SPEC(4, 0, 0, 0, 3, 0), TQ_SPEC(3, 0, 0, 0, 3, 0),
    TQ_SPEC(2, 0, 0, 0, 2, 0), TQ_SPEC(3, 0, 0, 0, 2, 0), TQ_SPEC(4, 0, 0, 0, 2, 0),
    TQ_SPEC(2, 1, 1, 1, 3, 2),
};
#undef TQ_SPEC

// Layouts of the two-wave kernel: value codes of up to 3 bits (each wave's
// value accumulators, 64 coordinates, then stay within the registers of two
// waves per SIMD; 4-bit MSE-only keys with 3-bit values would not), one key
// and one value group, or the 2.5-bit outlier split at channel 32 (CT1 = 2).
#define TQ_WSPEC(a, b, c, d, e, f, ct) Spec{a, b, c, d, e, f, pair_decode_kernel<a, b, c, d, e, f, ct>}
const Spec kWSpecs[] = {
    TQ_WSPEC(1, 1, 0, 0, 1, 0, 8), TQ_WSPEC(1, 1, 0, 0, 2, 0, 8), TQ_WSPEC(2, 1, 0, 0, 2, 0, 8),
    TQ_WSPEC(3, 1, 0, 0, 2, 0, 8), TQ_WSPEC(1, 1, 0, 0, 3, 0, 8), TQ_WSPEC(2, 1, 0, 0, 3, 0, 8),
    TQ_WSPEC(3, 1, 0, 0, 3, 0, 8), TQ_WSPEC(3, 0, 0, 0, 3, 0, 8),
    TQ_WSPEC(2, 0, 0, 0, 2, 0, 8), TQ_WSPEC(3, 0, 0, 0, 2, 0, 8), TQ_WSPEC(4, 0, 0, 0, 2, 0, 8),
    TQ_WSPEC(2, 1, 1, 1, 3, 2, 2),
};
#undef TQ_WSPEC

const Spec* find_wspec(const tq_kv_desc& k, const tq_kv_desc& v) {
  int Dv = 0, D = 0;
  for (int i = 0; i < v.n_groups; ++i) Dv += v.g[i].q.d;
  for (int i = 0; i < k.n_groups; ++i) D += k.g[i].q.d;
  if (D != kD || Dv != kD || k.n_groups > kMaxKG || v.n_groups > kMaxVG) return nullptr;
  if (k.n_groups > 1 && k.g[1].ch_offset != 32) return nullptr;
  if (v.n_groups > 1 && v.g[1].ch_offset != 32) return nullptr;
  const int kb0 = k.g[0].q.mse_bits, kp0 = k.g[0].q.variant == TQ_PROD;
  const int kb1 = k.n_groups > 1 ? k.g[1].q.mse_bits : 0;
  const int kp1 = k.n_groups > 1 ? (k.g[1].q.variant == TQ_PROD) : 0;
  const int vb0 = v.g[0].q.mse_bits, vb1 = v.n_groups > 1 ? v.g[1].q.mse_bits : 0;
  for (const Spec& sp : kWSpecs)
    if (sp.kb0 == kb0 && sp.kp0 == kp0 && sp.kb1 == kb1 && sp.kp1 == kp1 && sp.vb0 == vb0 && sp.vb1 == vb1)
      return &sp;
  return nullptr;
}

const Spec* find_spec(const tq_kv_desc& k, const tq_kv_desc& v) {
  int Dv = 0, D = 0;
  for (int i = 0; i < v.n_groups; ++i) Dv += v.g[i].q.d;
  for (int i = 0; i < k.n_groups; ++i) D += k.g[i].q.d;
  if (D != kD || Dv != kD || k.n_groups > kMaxKG || v.n_groups > kMaxVG) return nullptr;
  // a wave's 32 value coordinates must lie in one value group
  for (int i = 0; i < v.n_groups; ++i)
    if (v.g[i].q.d % 32) return nullptr;
  const int kb0 = k.g[0].q.mse_bits, kp0 = k.g[0].q.variant == TQ_PROD;
  const int kb1 = k.n_groups > 1 ? k.g[1].q.mse_bits : 0;
  const int kp1 = k.n_groups > 1 ? (k.g[1].q.variant == TQ_PROD) : 0;
  const int vb0 = v.g[0].q.mse_bits, vb1 = v.n_groups > 1 ? v.g[1].q.mse_bits : 0;
  for (const Spec& sp : kSpecs)
    if (sp.kb0 == kb0 && sp.kp0 == kp0 && sp.kb1 == kb1 && sp.kp1 == kp1 && sp.vb0 == vb0 && sp.vb1 == vb1)
      return &sp;
  return nullptr;
}

}  // namespace

namespace tqk {

bool mfma_decode_supported(const tq_kv_desc& k, const tq_kv_desc& v) {
  return find_wspec(k, v) != nullptr || find_spec(k, v) != nullptr;
}

int mfma_decode_max_splits() { return kMaxCombineSplits; }

DecodePlan plan_decode_mfma(const tq_kv_desc& k, const tq_kv_desc& v, int B, int Hq, int Hkv, int T_max,
                            int block_tokens) {
  DecodePlan p{};
  const int G = Hq / Hkv;
  const int HT = (G + kHT - 1) / kHT;
  const int64_t wgs_per_split = (int64_t)B * Hkv * HT;
  // the two-wave kernel: two waves per SIMD, i.e. four two-wave workgroups
  // per compute unit, chunks of 128 tokens; otherwise two four-wave
  // workgroups per compute unit and chunks of 256 tokens (the kernels'
  // launch bounds)
  const bool wave = find_wspec(k, v) != nullptr;
  const int chunk = wave ? kPChunk : kChunk;
  const int64_t target = (wave ? 4 : 2) * (int64_t)device_cus();
  int64_t splits = (target + wgs_per_split - 1) / wgs_per_split;
  int64_t sl = (T_max + splits - 1) / splits;
  // test hook: TQ_DECODE_SPLIT_TOKENS (a positive multiple of 256) fixes the
  // split length instead, so that tests can compare results across split
  // counts; read at every plan, so a size query and the decode it sizes
  // agree as long as the variable does not change between them
  if (const char* ev = getenv("TQ_DECODE_SPLIT_TOKENS")) {
    const long ov = strtol(ev, nullptr, 10);
    if (ov > 0 && ov % kChunk == 0) sl = ov;
  }
  const int64_t min_sl = (T_max + kMaxCombineSplits - 1) / kMaxCombineSplits;  // the combine's split table
  if (sl < min_sl) sl = min_sl;
  sl = (sl + chunk - 1) / chunk * chunk;
  if (block_tokens > 0) {  // a split must not leave its block: a divisor of it
    sl = std::min<int64_t>(sl, block_tokens);
    while (block_tokens % sl) sl -= chunk;
  }
  p.split_len = (int)sl;
  p.splits = (int)((T_max + sl - 1) / sl);
  p.head_chunk = kHT;
  p.n_chunks = HT;
  p.D = kD;
  p.Dv = kD;
  int slots = 0;
  for (int i = 0; i < k.n_groups; ++i) slots += n_odd(k.g[i].q.mse_bits) + (k.g[i].q.variant == TQ_PROD ? 1 : 0);
  const size_t keys = (size_t)B * Hkv * HT;
  // q~, q^ [keys][4][kD]; operands [keys][slots][512]; then the split
  // partials
  p.qprep_floats = 2 * keys * kHT * kD + keys * slots * 512;
  p.qprep_floats = (p.qprep_floats + 3) / 4 * 4;
  p.partial_floats = (size_t)B * Hq * p.splits * (kD + 2);
  return p;
}

hipError_t launch_decode_mfma(const tq_kv_desc& k, const tq_kv_desc& v, const void* q, tq_dtype qdt, int B, int Hq,
                              int Hkv, int T_max, const int32_t* seq_lens, float scale, float* out,
                              float* scores_out, void* ws, const DecodePlan& plan, hipStream_t s,
                              const PageTable* pages, const StepRows* step) {
  const Spec* wsp = find_wspec(k, v);
  const Spec* sp = wsp ? wsp : find_spec(k, v);
  if (!sp) return hipErrorInvalidValue;
  Args a{};
  if (pages) {
    a.block_table = pages->table;
    a.max_blocks = pages->max_blocks;
    a.block_tokens = pages->block_tokens;
    a.num_blocks = pages->num_blocks;
  }
  bool folded = true;  // every PROD key group carries S R: one query-transform pass
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
    o.SR = g.q.SR;
    o.seq_stride = g.seq_stride;
    o.ch = g.ch_offset;
    o.d = g.q.d;
    o.B = g.q.mse_bits;
    o.prod = g.q.variant == TQ_PROD;
    if (o.prod && !o.SR) folded = false;
    o.gamma = (float)(sqrt(M_PI / 2.0) / g.q.d);
    float alphas[kMaxVTypes];
    const int nt = odd_walsh(g.q, alphas);
    o.amax = 0.f;
    for (int t = 0; t < nt; ++t) {
      a.slot_group |= gi << ns;
      a.slot_alpha[ns++] = alphas[t];
      o.amax = fmaxf(o.amax, fabsf(alphas[t]));
    }
    if (o.prod) {
      a.slot_group |= gi << ns;
      a.slot_qjl |= 1 << ns;
      a.slot_alpha[ns++] = 1.f;
    }
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
  float* wsf = static_cast<float*>(ws);
  a.qt = wsf;
  a.qh = a.qt + keys * kHT * kD;
  a.aops = reinterpret_cast<uint32_t*>(a.qh + keys * kHT * kD);
  a.partial = wsf + plan.qprep_floats;
  a.out = out;
  const dim3 qgrid((unsigned)keys, kD / kRowSlice);
  if (step && !folded) {  // (without S R the appends take launches of their own)
    const hipError_t e = launch_append_step(k, v, *step, B, Hkv, s);
    if (e != hipSuccess) return e;
  }
  if (step && folded) {
    StepAppend st{};
    st.n = tqq::step_args(k, v, *step, B, Hkv, st.q);
    st.tiles = (B * Hkv + kStepTV - 1) / kStepTV;
    st.key_columns = (int)keys;
    int dmax = 32;
    for (int i = 0; i < st.n; ++i) dmax = std::max(dmax, st.q[i].d);
    const int extra = (st.n * st.tiles + (int)qgrid.y - 1) / (int)qgrid.y;
    const size_t lds = tqq::lds_bytes(dmax, kStepTV, kStepJC);
    // direct products for a handful of new rows (latency first); staged ones
    // otherwise, whose smaller register footprint keeps the transform's
    // workgroups at full occupancy
    const bool direct = B * Hkv <= 64;
    const void* fn = direct ? (const void*)qfused_step_kernel<true> : (const void*)qfused_step_kernel<false>;
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const dim3 sgrid(qgrid.x + extra, qgrid.y);
    if (direct)
      hipLaunchKernelGGL(qfused_step_kernel<true>, sgrid, dim3(kQtThreads), lds, s, a, st);
    else
      hipLaunchKernelGGL(qfused_step_kernel<false>, sgrid, dim3(kQtThreads), lds, s, a, st);
  } else if (folded) {
    hipLaunchKernelGGL(qfused_kernel, qgrid, dim3(kQtThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(qtransform_kernel<false>, qgrid, dim3(kQtThreads), 0, s, a);
    hipLaunchKernelGGL(qtransform_kernel<true>, qgrid, dim3(kQtThreads), 0, s, a);
  }
  const dim3 grid(plan.splits, a.HT, B * Hkv);
  hipLaunchKernelGGL(sp->fn, grid, dim3(wsp ? kPThreads : kThreads), 0, s, a);
  if (plan.splits <= kFewSplits)
    hipLaunchKernelGGL(combine_heads_kernel, dim3((B * Hq + kHeadsPerComb - 1) / kHeadsPerComb), dim3(kCombThreads),
                       0, s, a);
  else
    hipLaunchKernelGGL(combine_kernel, dim3(B * Hq, kJSlices), dim3(kCombThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace tqk
