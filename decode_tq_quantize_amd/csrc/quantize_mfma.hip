// Online TurboQuant compression of KV vectors of d = 32, 64, 96 or 128
// channels on the gfx950 matrix cores (riverfrot "TurboQuant" post, section
// 4.1: x~ = R x / |x|; section 4.2: Lloyd-Max interval index per coordinate;
// section 4.3: the residual r~ = x~ - c[idx] projected with S, signs kept,
// plus |r~|).
//
// A persistent workgroup of d / 32 waves streams tiles of 32 vectors; wave w
// owns output coordinates 32 w .. 32 w + 31. bf16 inputs are exact in bf16, so R
// is held in registers as bf16 high and low parts (MFMA A operands) and R x
// runs on v_mfma_f32_16x16x32_bf16 with both products accumulated in place;
// one more MFMA with the input as both operands gives the vectors' Gram
// matrix, whose diagonal is |x|^2. fp32 inputs use v_mfma_f32_16x16x4_f32
// with R in fp32. The rotated vector comes out with lane l holding
// coordinates 32 w + 16 m + 4 (l / 16) + r (m = 0, 1; r = 0..3) of vector
// l % 16 of a 16-vector half. The rotation's contraction over the d input
// coordinates runs in d / 32 steps of 32, lane group q (= lane / 16)
// supplying coordinates 32 k + 8 q .. + 7 at step k on both operands (fp32:
// steps of 4, coordinate 16 j + 4 q + e at step 4 j + e), so the four lanes
// of a vector row load one contiguous 64-byte segment per instruction. The
// interval index is found there by binary
// search over the thresholds, the residual's bf16 parts go through LDS to
// the operand layout of S r~ (bf16 matrix cores, S in LDS), and the code
// and sign bits are packed straight from wave ballots of the compares into
// the library's bit-plane layouts.
#include <mutex>
#include <utility>
#include <vector>

#include "device_common.h"
#include "internal.h"

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kTile = 32;  // vectors per iteration (one values tile, two keys tiles)

// 16-byte chunks per LDS row of a d-wide bf16 matrix (S, and the residuals):
// 128-wide rows are swizzled (chunk c of row r at c ^ (r % 16)), narrower
// rows padded to an odd number of chunks, so the 16 rows that a step reads
// at once hit 16 different bank groups either way.
template <int D>
constexpr int row_chunks() {
  return D == 128 ? 16 : D / 8 + 1;
}
template <int D>
__device__ __forceinline__ int swz(int row, int c) {
  return D == 128 ? c ^ (row & 15) : c;
}

struct QmArgs {
  const void* x;
  int64_t n;
  int64_t stride;
  int bf16;
  const float* R;
  const float* S;
  int B;
  int prod;
  int layout;
  int64_t ntiles;
  float cent[TQ_MAX_LEVELS];
  float thr[TQ_MAX_LEVELS - 1];
  uint32_t* packed;
  uint16_t* norm;
  uint16_t* rnorm;
};

// 2 x + (this lane's bit of the wave mask): one add with the mask as the
// carry in. The masks passed here are formed by the scalar unit.
__device__ __forceinline__ uint32_t shift_in(uint32_t x, uint64_t mask) {
  uint32_t r;
  uint64_t co;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=&s"(co) : "v"(x), "s"(mask));
  return r;
}

// v_writelane_b32 as the compiler's own intrinsic (its hazard checks then
// see the instruction; inline asm would be fenced with wait states)
extern "C" __device__ int tq_writelane_i32(int x, int lane, int old) __asm("llvm.amdgcn.writelane.i32");
// Lane `l` of v takes the uniform value x.
__device__ __forceinline__ void write_lane(uint32_t& v, uint32_t x, int l) {
  v = (uint32_t)tq_writelane_i32((int)x, l, (int)v);
}

__device__ __forceinline__ v4f mfma_f32(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ v4f mfma_bf16(bf16x8 a, bf16x8 b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// bf16 rounding (nearest even) of a finite float, as raw bits.
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// bf16 high and low parts (round to nearest even, v_cvt_pk_bf16_f32) of
// two floats, packed two to a register: x = hi + lo + O(2^-17 |x|).
__device__ __forceinline__ void split_bf16(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{x0, x1}, bf16x2));
  const float r0 = x0 - __uint_as_float(hi << 16), r1 = x1 - __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{r0, r1}, bf16x2));
}

// Rows 32 w + 16 m + (lane % 16) of the D x D matrix M, at the columns that
// lane group q = lane / 16 supplies to the contraction: A[m][8 k + e] =
// column 32 k + 8 q + e (bf16 inputs), A[m][4 j + e] = column 16 j + 4 q + e
// (fp32 inputs).
template <int D, bool BF16IN>
__device__ __forceinline__ void load_rows(const float* __restrict__ M, int w, int lane, float (&A)[2][D / 4]) {
  const int q = lane >> 4;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const float4* p = reinterpret_cast<const float4*>(M + (int64_t)(32 * w + 16 * m + (lane & 15)) * D);
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const float4 v = p[BF16IN ? 8 * (i >> 1) + 2 * q + (i & 1) : 4 * i + q];
      A[m][4 * i] = v.x;
      A[m][4 * i + 1] = v.y;
      A[m][4 * i + 2] = v.z;
      A[m][4 * i + 3] = v.w;
    }
  }
}

// Raw input of one lane, lane group q, from one vector row: coordinates
// 32 k + 8 q .. + 7 in w[k] (bf16), 16 j + 4 q .. + 3 in f[j] (fp32).
template <int D, bool BF16IN>
struct XIn;
template <int D>
struct XIn<D, true> {
  uint4 w[D / 32];
};
template <int D>
struct XIn<D, false> {
  float4 f[D / 16];
};
template <int D>
__device__ __forceinline__ void load_in(XIn<D, true>& r, const QmArgs& a, int64_t v, int q) {
  const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + v * a.stride) + q;
#pragma unroll
  for (int k = 0; k < D / 32; ++k) r.w[k] = p[4 * k];
}
template <int D>
__device__ __forceinline__ void load_in(XIn<D, false>& r, const QmArgs& a, int64_t v, int q) {
  const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + v * a.stride) + q;
#pragma unroll
  for (int k = 0; k < D / 16; ++k) r.f[k] = p[4 * k];
}

// Lane exchanges with lane l ^ 16 and l ^ 32 (v_permlane16/32_swap: with
// both operands the same value, the two results are this lane's value and
// its partner's, in some order), so combining them is symmetric.
__device__ __forceinline__ uint32_t or_q(uint32_t v) {
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = a[0] | a[1];
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return b[0] | b[1];
}
// Sum over the 4 lanes that hold the same vector (lanes l, l ^ 16, l ^ 32, l ^ 48).
__device__ __forceinline__ float sum_q(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Threshold th[LO + k STRIDE], k = 0 .. N - 1, chosen by the bits found so
// far (bits[0] the most significant): a tree of N - 1 selects over values
// (constant indices only, so the thresholds stay in registers).
template <int N, int LO, int STRIDE, int NT>
__device__ __forceinline__ float pick(const float (&th)[NT], const bool* bits) {
  if constexpr (N == 1) {
    return th[LO];
  } else {
    const float hi = pick<N / 2, LO + (N / 2) * STRIDE, STRIDE>(th, bits + 1);
    const float lo = pick<N / 2, LO, STRIDE>(th, bits + 1);
    return bits[0] ? hi : lo;
  }
}

// Bit j of the interval index and the bits below it: the compare against
// the middle threshold th[k 2^(j+1) + 2^j - 1] of the interval k that the
// higher bits (bits[0 .. B-2-j]) leave.
template <int B, int J>
__device__ __forceinline__ void interval_bits(float u, const float (&th)[(1 << B) - 1], bool (&bits)[B]) {
  bits[B - 1 - J] = u >= pick<(1 << (B - 1 - J)), (1 << J) - 1, (2 << J)>(th, bits);
  if constexpr (J > 0) interval_bits<B, J - 1>(u, th, bits);
}

// Interval index #{t : u >= th[t]} of the sorted thresholds by binary
// search (B compares instead of 2^B - 1).
template <int B>
__device__ __forceinline__ int interval(float u, const float (&th)[(1 << B) - 1]) {
  bool bits[B];
  interval_bits<B, B - 1>(u, th, bits);
  int idx = 0;
#pragma unroll
  for (int j = 0; j < B; ++j) idx |= bits[j] ? (1 << (B - 1 - j)) : 0;
  return idx;
}

// (registers sized for two waves per SIMD)
template <int D, bool BF16IN, int B, bool PROD, bool KEYS>
__global__ __launch_bounds__(2 * D, 2) void quantize_mfma_kernel(QmArgs a) {
  constexpr int NG = D / 32;  // waves (32-coordinate groups), and 32-coordinate steps of a contraction
  constexpr int kThreads = 64 * NG;
  constexpr int RC = row_chunks<D>();
  // The QJL projection S r~ runs on the bf16 matrix cores with both operands
  // split into bf16 high and low parts: S r~ = S_hi r_hi + S_hi r_lo +
  // S_lo r_hi up to about 2^-17 |S| |r~| per term. S (PROD) stays in LDS as
  // the two parts (for d = 128 two workgroups fit a compute unit); so does
  // the residual of the current 16 vectors. Rows are d / 8 chunks of 8
  // values (placed by swz within row_chunks<D>() slots).
  __shared__ uint4 Sq[2][PROD ? D : 1][RC];
  // residual parts of both 16-vector halves ([half][hi / lo][vector][chunk]);
  // once the projection has read them, the same space takes the residual
  // norms' partial sums (for d = 128, S and this fill the 160 KB of two
  // workgroups)
  __shared__ uint4 rq[PROD ? 2 : 1][2][PROD ? 16 : 1][RC];
  static_assert(!PROD || sizeof(rq) >= sizeof(float) * NG * kTile, "norm partials must fit the residual space");
  float(&rho_part)[NG][kTile] = *reinterpret_cast<float(*)[NG][kTile]>(&rq[0][0][0][0]);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, nl = lane & 15;
  constexpr int L = 1 << B;
  constexpr int P = B + (PROD ? 1 : 0);
  // thresholds as uniform values (the compares below are unrolled)
  float th[L - 1];
#pragma unroll
  for (int t = 0; t < L - 1; ++t) {
    th[t] = a.thr[t];
    asm volatile("" : "+v"(th[t]));  // held in a VGPR: the selects below take one SGPR operand at most
  }

  // R as A operands: fp32 (fp32 input), or bf16 high and low parts (bf16
  // input, which is exact in bf16: R x = R_hi x + R_lo x, |R - R_hi - R_lo|
  // <= 2^-18 |R| elementwise)
  float AR[2][D / 4];
  bf16x8 RH[2][NG], RL[2][NG];
  load_rows<D, BF16IN>(a.R, w, lane, AR);
  if constexpr (BF16IN) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int kk = 0; kk < NG; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float r = AR[m][8 * kk + e];
          const uint32_t hb = bf16_bits(r);
          const float hf = __uint_as_float(hb << 16);
          RH[m][kk][e] = __builtin_bit_cast(__bf16, (uint16_t)hb);
          RL[m][kk][e] = __builtin_bit_cast(__bf16, (uint16_t)bf16_bits(r - hf));
        }
  }
  if constexpr (PROD) {
    for (int e = tid; e < D * D / 8; e += kThreads) {
      const int row = e / (D / 8), c = e % (D / 8);
      const float4 u0 = reinterpret_cast<const float4*>(a.S)[2 * e];
      const float4 u1 = reinterpret_cast<const float4*>(a.S)[2 * e + 1];
      uint32_t h[4], l[4];
      split_bf16(u0.x, u0.y, h[0], l[0]);
      split_bf16(u0.z, u0.w, h[1], l[1]);
      split_bf16(u1.x, u1.y, h[2], l[2]);
      split_bf16(u1.z, u1.w, h[3], l[3]);
      Sq[0][row][swz<D>(row, c)] = make_uint4(h[0], h[1], h[2], h[3]);
      Sq[1][row][swz<D>(row, c)] = make_uint4(l[0], l[1], l[2], l[3]);
    }
  }
  // centroids as values (the residual picks one by the index bits)
  float cv[L];
#pragma unroll
  for (int t = 0; t < L; ++t) {
    cv[t] = a.cent[t];
    if constexpr (PROD) asm volatile("" : "+v"(cv[t]));
  }
  __syncthreads();

  // The vector that MFMA column c of half nt of tile t carries: for keys
  // vector 32 t + 16 nt + c; for values the vector whose bit in the words of
  // value tile t is 16 nt + c (the two tiles of a 64-vector block interleave
  // its vectors), so that the halves' ballots are the words' halves as they
  // stand
  auto col_vec = [&](int64_t t, int nt, int c) __attribute__((always_inline)) -> int64_t {
    return KEYS ? t * kTile + 16 * nt + c
                : (t >> 1) * tqk::kValuesBlock + tqk::value_tok((int)(t & 1), 16 * nt + c);
  };
  // a tile's inputs (rows past n re-read row n - 1 and are masked)
  auto load_tile = [&](XIn<D, BF16IN>(&dst)[2], int64_t t) __attribute__((always_inline)) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) load_in<D>(dst[nt], a, min(col_vec(t, nt, nl), a.n - 1), q);
  };
  // (value layout) word offset of this lane's pair word within the wave's
  // 32 P words, and the byte selector of the join (sources y, x)
  int woff[KEYS ? 1 : (16 * P + 31) / 32];
  uint32_t wsel = 0u;
  if constexpr (!KEYS) {
#pragma unroll
    for (int i = 0; i < (16 * P + 31) / 32; ++i) {
      const int k = 32 * i + (lane & 31), p = k % P, t = k / P;
      const int r = t & 3, h = (t >> 2) & 1, m = t >> 3;
      woff[i] = (16 * m + 4 * (2 * h + (lane >> 5)) + r) * P + p;
    }
    wsel = lane < 32 ? 0x05040100u : 0x07060302u;
  }
  const int64_t nround = (a.n + tqk::kKeysTile - 1) / tqk::kKeysTile * tqk::kKeysTile;
  // one tile, whose inputs are in cur; once the rotation has read them, cur
  // takes the inputs of tile tnext
  auto body = [&](int64_t tile, XIn<D, BF16IN>(&cur)[2], int64_t tnext) __attribute__((always_inline)) {
    const int64_t v0 = tile * kTile;
    // 1. rotated coordinates 32 w + 16 m + 4 q + r of vector 16 nt + nl, and
    // the vector norms
    v4f acc[2][2];
    float nrm[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      if constexpr (BF16IN) {
        const uint4(&xw)[NG] = cur[nt].w;
        // one accumulator per 16 rows: the matrix cores accumulate in place
        // back to back, so the hi and lo products need no separate sums
        v4f ah[2], gram = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 2; ++m) ah[m] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NG; ++kk) {
          const bf16x8 xb = __builtin_bit_cast(bf16x8, xw[kk]);
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            ah[m] = mfma_bf16(RH[m][kk], xb, ah[m]);
            ah[m] = mfma_bf16(RL[m][kk], xb, ah[m]);
          }
          // the 16 vectors' Gram matrix: the same register is the A operand
          // (row = vector) and the B operand (column = vector); products of
          // bf16 values are exact in the fp32 accumulation
          gram = mfma_bf16(xb, xb, gram);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) acc[nt][m] = ah[m];
        // |x|^2 of vector nl is the diagonal entry (nl, nl), held by lane
        // 16 (nl / 4) + nl as its element nl % 4
        const float dsel = (nl & 2) ? ((nl & 1) ? gram[3] : gram[2]) : ((nl & 1) ? gram[1] : gram[0]);
        nrm[nt] = __builtin_amdgcn_sqrtf(__shfl(dsel, 16 * (nl >> 2) + nl, 64));
      } else {
        float s2 = 0.f;
        float x[D / 4];
#pragma unroll
        for (int k = 0; k < D / 16; ++k) {
          x[4 * k] = cur[nt].f[k].x;
          x[4 * k + 1] = cur[nt].f[k].y;
          x[4 * k + 2] = cur[nt].f[k].z;
          x[4 * k + 3] = cur[nt].f[k].w;
        }
#pragma unroll
        for (int k = 0; k < D / 4; ++k) s2 = fmaf(x[k], x[k], s2);
        v4f ac[2][4];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int c = 0; c < 4; ++c) ac[m][c] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D / 4; ++kk) {
          ac[0][kk & 3] = mfma_f32(AR[0][kk], x[kk], ac[0][kk & 3]);
          ac[1][kk & 3] = mfma_f32(AR[1][kk], x[kk], ac[1][kk & 3]);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) acc[nt][m] = (ac[m][0] + ac[m][1]) + (ac[m][2] + ac[m][3]);
        nrm[nt] = __builtin_amdgcn_sqrtf(sum_q(s2));
      }
    }
    load_tile(cur, tnext);
    // 2. code bits (index bits by binary search, most significant first),
    // residuals and their norms. A vector of norm 0 gets index L / 2 and
    // residual 0; padding vectors keep all-zero bits. Wave ballots of the
    // bits have bit 16 q + nl = coordinate 32 w + 16 m + 4 q + r of vector
    // 16 nt + nl.
    bool valid[2], live[2];
    float inv[2], bias[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      valid[nt] = col_vec(tile, nt, nl) < a.n;
      live[nt] = valid[nt] & (nrm[nt] > 0.f);
      inv[nt] = live[nt] ? __builtin_amdgcn_rcpf(nrm[nt]) : 0.f;
      bias[nt] = valid[nt] ? (live[nt] ? 0.f : th[L / 2 - 1]) : -INFINITY;
      if (w == 0 && q == 0 && valid[nt]) a.norm[col_vec(tile, nt, nl)] = tqd::f32_to_half_bits(nrm[nt]);
    }
    float res[2][2][4];
    float r2[2] = {0.f, 0.f};
    // the search bits of one coordinate (most significant first), and the
    // residual. u = acc / |x| + bias: bias 0 for live vectors; for a vector
    // of norm 0 (inv 0) the threshold below the middle, which lands on
    // index L / 2; for padding (inv 0) -inf, index 0 (all bits clear). So
    // the code ballots need no masks; the residuals of those vectors are
    // not used (their signs are masked, their residual norm written as 0).
    auto code_bits = [&](int nt, int m, int r, bool (&bt)[B]) __attribute__((always_inline)) {
      const float u = fmaf(acc[nt][m][r], inv[nt], bias[nt]);
      interval_bits<B, B - 1>(u, th, bt);
      if constexpr (PROD) {
        const float rr = u - pick<L, 0, 1>(cv, bt);
        res[nt][m][r] = rr;
        r2[nt] = fmaf(rr, rr, r2[nt]);
      }
    };
    // word (vector t of key tile nt, group w, plane p) of the key layout:
    // bit i = coordinate 32 w + i. Each lane shifts its 8 bits of the plane
    // into an accumulator straight from the plane's ballots (coordinates
    // (m, r) in descending order, one add-with-carry per bit), spreads them
    // to bits 16 m + 4 q + r, and the 4 lanes of a vector combine theirs.
    uint32_t kw[2][P];
    auto key_word = [&](uint32_t acc8) __attribute__((always_inline)) -> uint32_t {
      return or_q(((acc8 & 0xfu) | ((acc8 & 0xf0u) << 12)) << (4 * q));
    };
    // words (coordinate j, plane p) of the value layout: bit i = the vector
    // of column i % 16 of half i / 16. Bits 16 q .. 16 q + 15 of the two
    // halves' ballots are the low and high halves of the word of coordinate
    // 32 w + 16 m + 4 q + r, so the low (high) 32 bits of a ballot pair give
    // the words of lane groups 2 h and 2 h + 1 (h = 0 (1)): pair k =
    // ((2 m + h) 4 + r) P + p puts the first half-ballot in lane k % 32 and
    // the second in lane k % 32 + 32 of ow[k / 32], as they are; the stores
    // join them.
    constexpr int NR = (16 * P + 31) / 32;
    uint32_t ow[NR];
#pragma unroll
    for (int i = 0; i < NR; ++i) ow[i] = 0u;
    auto value_words = [&](int m, int r, int p, uint64_t m0, uint64_t m1) __attribute__((always_inline)) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = ((2 * m + h) * 4 + r) * P + p;
        write_lane(ow[k >> 5], (uint32_t)(m0 >> (32 * h)), k & 31);
        write_lane(ow[k >> 5], (uint32_t)(m1 >> (32 * h)), (k & 31) + 32);
      }
    };
    // ballots of the compares themselves (a ballot of a combined flag, or a
    // per-lane combination, makes the compiler round-trip it through a
    // vector register); the sign plane applies zero and padding vectors to
    // its masks with these
    uint64_t vm[2], lm[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      vm[nt] = __builtin_amdgcn_ballot_w64(valid[nt]);
      lm[nt] = __builtin_amdgcn_ballot_w64(live[nt]);
    }
    if constexpr (KEYS) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        uint32_t acc8[B];
#pragma unroll
        for (int p = 0; p < B; ++p) acc8[p] = 0u;
#pragma unroll
        for (int m = 1; m >= 0; --m)
#pragma unroll
          for (int r = 3; r >= 0; --r) {
            bool bt[B];
            code_bits(nt, m, r, bt);
#pragma unroll
            for (int p = 0; p < B; ++p) acc8[p] = shift_in(acc8[p], __builtin_amdgcn_ballot_w64(bt[B - 1 - p]));
          }
#pragma unroll
        for (int p = 0; p < B; ++p) kw[nt][p] = key_word(acc8[p]);
      }
    } else {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          uint64_t pm[2][B];
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            bool bt[B];
            code_bits(nt, m, r, bt);
#pragma unroll
            for (int p = 0; p < B; ++p) pm[nt][p] = __builtin_amdgcn_ballot_w64(bt[B - 1 - p]);
          }
#pragma unroll
          for (int p = 0; p < B; ++p) value_words(m, r, p, pm[0][p], pm[1][p]);
        }
    }
    // 3. QJL signs: S r~ on the matrix cores, both 16-vector halves per S
    // operand read
    if constexpr (PROD) {
      // residual coordinates 32 w + 16 m + 4 q .. + 3 of vector nl: half of
      // chunk (4 w + 2 m + q / 2) of the vector's row
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          uint32_t h0, l0, h1, l1;
          split_bf16(res[nt][m][0], res[nt][m][1], h0, l0);
          split_bf16(res[nt][m][2], res[nt][m][3], h1, l1);
          const int c = swz<D>(nl, 4 * w + 2 * m + (q >> 1)), half = q & 1;
          reinterpret_cast<uint2*>(&rq[nt][0][nl][c])[half] = make_uint2(h0, h1);
          reinterpret_cast<uint2*>(&rq[nt][1][nl][c])[half] = make_uint2(l0, l1);
        }
      __syncthreads();
      // step kk contracts coordinates 8 (NG q' + kk) .. + 7 from lane group q'
      // (chunk NG q' + kk), the same assignment on both operands
      v4f pc[2][2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int m = 0; m < 2; ++m) pc[nt][m] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NG; ++kk) {
        const int ph = swz<D>(nl, NG * q + kk);
        bf16x8 rh[2], rl[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          rh[nt] = __builtin_bit_cast(bf16x8, rq[nt][0][nl][ph]);
          rl[nt] = __builtin_bit_cast(bf16x8, rq[nt][1][nl][ph]);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int row = 32 * w + 16 * m + nl;  // row % 16 == nl
          const bf16x8 sh = __builtin_bit_cast(bf16x8, Sq[0][row][ph]);
          const bf16x8 sl = __builtin_bit_cast(bf16x8, Sq[1][row][ph]);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            pc[nt][m] = mfma_bf16(sh, rh[nt], pc[nt][m]);
            pc[nt][m] = mfma_bf16(sh, rl[nt], pc[nt][m]);
            pc[nt][m] = mfma_bf16(sl, rh[nt], pc[nt][m]);
          }
        }
      }
      uint64_t zm[2][2][4];  // sign-plane masks
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            zm[nt][m][r] = (__builtin_amdgcn_ballot_w64(pc[nt][m][r] >= 0.f) | ~lm[nt]) & vm[nt];
        if constexpr (KEYS) {
          uint32_t acc8 = 0u;
#pragma unroll
          for (int m = 1; m >= 0; --m)
#pragma unroll
            for (int r = 3; r >= 0; --r) acc8 = shift_in(acc8, zm[nt][m][r]);
          kw[nt][B] = key_word(acc8);
        }
      }
      if constexpr (!KEYS) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int r = 0; r < 4; ++r) value_words(m, r, B, zm[0][m][r], zm[1][m][r]);
      }
      __syncthreads();  // every wave has read rq: its space takes the norms' partials
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float rs = sum_q(r2[nt]);
        if (q == 0) rho_part[w][16 * nt + nl] = live[nt] ? rs : 0.f;
      }
      __syncthreads();
      // residual norms (one lane per vector)
      if (w == 0 && q < 2) {
        const int vt = 16 * q + nl;  // column nl of half q
        if (col_vec(tile, q, nl) < a.n) {
          float s;
          if constexpr (NG == 4)
            s = (rho_part[0][vt] + rho_part[1][vt]) + (rho_part[2][vt] + rho_part[3][vt]);
          else {
            s = rho_part[0][vt];
#pragma unroll
            for (int i = 1; i < NG; ++i) s += rho_part[i][vt];
          }
          const float rho = __builtin_amdgcn_sqrtf(s);
          a.rnorm[col_vec(tile, q, nl)] = tqd::f32_to_half_bits(rho);
        }
      }
    }
    // 4. stores
    if constexpr (KEYS) {
      // lane (q, nl) stores plane q (and q + 4) of vector nl; the wave's
      // words of a key tile are 16 P contiguous words, word nl P + p
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        if (v0 + 16 * nt < nround) {
          const int64_t kt = (v0 >> 4) + nt;
          uint32_t* dst = a.packed + (kt * NG + w) * tqk::kKeysTile * P;
#pragma unroll
          for (int pass = 0; pass < (P + 3) / 4; ++pass) {
            const int p = 4 * pass + q;
            uint32_t wv = kw[nt][4 * pass];
#pragma unroll
            for (int pp = 4 * pass + 1; pp < P && pp < 4 * pass + 4; ++pp) wv = (p == pp) ? kw[nt][pp] : wv;
            if (p < P) dst[nl * P + p] = wv;
          }
        }
      }
    } else {
      // after the swap every lane of a pair holds its two half-ballots x
      // (first) and y; the low lane stores x.lo | y.lo << 16, the high one
      // x.hi | y.hi << 16
      uint32_t* dst = a.packed + (tile * D + 32 * w) * P;
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const auto xy = __builtin_amdgcn_permlane32_swap(ow[i], ow[i], false, false);
        const uint32_t word = __builtin_amdgcn_perm(xy[1], xy[0], wsel);
        if (32 * i + (lane & 31) < 16 * P) dst[woff[i]] = word;
      }
    }
    if constexpr (PROD) __syncthreads();  // rq (and rho_part in it) is rewritten by the next tile
  };
  XIn<D, BF16IN> xa[2], xb[2];
  load_tile(xa, blockIdx.x);
  if constexpr (BF16IN) {
    // two tiles' inputs in flight (the two buffers alternate, nothing is copied)
    load_tile(xb, (int64_t)blockIdx.x + gridDim.x);
    // (both tiles of an iteration unconditional, the odd last one after the
    // loop: a conditional second tile makes the loop head wait for every
    // load in flight, the other buffer's prefetch included)
    int64_t tile = blockIdx.x;
    for (; tile + gridDim.x < a.ntiles; tile += 2 * (int64_t)gridDim.x) {
      body(tile, xa, tile + 2 * (int64_t)gridDim.x);
      body(tile + gridDim.x, xb, tile + 3 * (int64_t)gridDim.x);
    }
    if (tile < a.ntiles) body(tile, xa, tile + 2 * (int64_t)gridDim.x);
  } else {
    for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) body(tile, xa, tile + gridDim.x);
  }
}


// ------------------------------------------------------------------ wide vectors
// Vectors of more than 128 channels (key layout): the same steps as above,
// as two GEMM-shaped passes over batches of vectors, because R and S no
// longer fit a workgroup's registers and LDS (riverfrot section 4.1 for the
// rotation and the interval index, section 4.3 for the sketch).
//
// A workgroup of 4 waves owns a tile of kWC = 128 output coordinates x kWV
// = 128 vectors; wave w the coordinates 32 w .. 32 w + 31 of the tile (two
// 16-row MFMA blocks) for all 128 vectors (8 blocks of 16). The contraction
// over the d inputs runs in steps of 32 on v_mfma_f32_16x16x32_bf16: the
// wave's matrix rows come straight from global memory (fp32, split into
// bf16 high and low parts in registers), the tile's inputs through LDS
// (split once, double-buffered, rows padded to 80 bytes so that the 16
// rows a read touches fall in different banks); three products hi hi +
// hi lo + lo hi (two for bf16 inputs, which are exact), fp32 accumulation,
// so the error is about 2^-17 of the terms' magnitudes as in the narrow
// kernel.
// Pass 1 (matrix R): |x|^2 from the staged inputs; u = (R x)_c / |x|; the
// interval index by binary search, packed from wave ballots into the key
// words of the tile's 32-coordinate groups; with the sketch, the residual
// u - c[idx] (fp32) to the batch workspace and its squared sum per vector
// and 32-coordinate group.
// Pass 2 (matrix S, on the residuals): the signs of (S r~)_c into the sign
// plane; the workgroups of coordinate tile 0 write |r~| from the partial
// sums.
// Tiles are numbered so that the coordinate tiles of one vector tile run on
// one XCD, one after another (its inputs stay in that XCD's L2).
constexpr int kWC = 128;
constexpr int kWV = 128;
constexpr int kWThreads = 256;
constexpr int kWRowB = 80;
constexpr int64_t kWBatch = 65536;  // vectors per batch (the residual workspace holds one)

struct WArgs {
  const void* x;   // input rows: pass 1 the call's vectors, pass 2 the residual workspace
  int64_t stride;  // elements per input row
  int64_t xrow0;   // input row of the batch's first vector
  const float* M;  // R (pass 1) or S (pass 2), d x d row-major
  float* res;      // [kWBatch][d] residuals of the batch (pass 1 writes, pass 2 reads)
  float* rho2;     // [kWBatch][d / 32] squared residual sums per 32-coordinate group
  int64_t v0;      // first vector of the batch
  int64_t nb;      // vectors in the batch
  int64_t n;       // vectors in the call
  int d;
  int B;
  float cent[TQ_MAX_LEVELS];
  float thr[TQ_MAX_LEVELS - 1];
  uint32_t* packed;
  uint16_t* norm;
  uint16_t* rnorm;
};

__device__ __forceinline__ uint32_t key_word_of(uint32_t acc8, int q) {
  return or_q(((acc8 & 0xfu) | ((acc8 & 0xf0u) << 12)) << (4 * q));
}

// The GEMM core shared by both passes: acc[m][nt] = rows c0 + 16 m + (4 q
// .. 4 q + 3) of M times vectors 16 nt + (lane % 16) of the tile. Returns
// the sum of squares of the inputs this thread staged (thread t: vector t /
// 2, inputs 16 (t % 2) .. + 15 of every step).
template <bool F32IN>
__device__ __forceinline__ float wide_gemm(const WArgs& a, int64_t lv0, int c0, bool wave_on, v4f (&acc)[2][8],
                                           uint8_t (*xs)[2][kWV][kWRowB]) {
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, nl = lane & 15;
  const int d = a.d, nks = d / 32;
  const int sv = tid >> 1, kh = tid & 1;
  const int64_t srow = a.xrow0 + (lv0 + sv < a.nb ? lv0 + sv : a.nb - 1);  // (padding vectors re-read the last row)
  float ss = 0.f;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[m][nt] = v4f{0.f, 0.f, 0.f, 0.f};
  // staged inputs of one step, in registers while the previous step computes
  float4 xf[4];
  uint4 xb[2];
  auto load_x = [&](int ks) __attribute__((always_inline)) {
    if constexpr (F32IN) {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(a.x) + srow * a.stride + 32 * ks + 16 * kh);
#pragma unroll
      for (int i = 0; i < 4; ++i) xf[i] = p[i];
    } else {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.x) + srow * a.stride + 32 * ks + 16 * kh);
#pragma unroll
      for (int i = 0; i < 2; ++i) xb[i] = p[i];
    }
  };
  auto stage = [&](int buf) __attribute__((always_inline)) {
    if constexpr (F32IN) {
      uint32_t h[8], l[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        split_bf16(xf[i].x, xf[i].y, h[2 * i], l[2 * i]);
        split_bf16(xf[i].z, xf[i].w, h[2 * i + 1], l[2 * i + 1]);
        ss = fmaf(xf[i].x, xf[i].x, ss);
        ss = fmaf(xf[i].y, xf[i].y, ss);
        ss = fmaf(xf[i].z, xf[i].z, ss);
        ss = fmaf(xf[i].w, xf[i].w, ss);
      }
      uint4* hp = reinterpret_cast<uint4*>(&xs[buf][0][sv][32 * kh]);
      uint4* lp = reinterpret_cast<uint4*>(&xs[buf][1][sv][32 * kh]);
      hp[0] = make_uint4(h[0], h[1], h[2], h[3]);
      hp[1] = make_uint4(h[4], h[5], h[6], h[7]);
      lp[0] = make_uint4(l[0], l[1], l[2], l[3]);
      lp[1] = make_uint4(l[4], l[5], l[6], l[7]);
    } else {
      const uint32_t wv[8] = {xb[0].x, xb[0].y, xb[0].z, xb[0].w, xb[1].x, xb[1].y, xb[1].z, xb[1].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float lo = __uint_as_float(wv[i] << 16), hi = __uint_as_float(wv[i] & 0xffff0000u);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
      }
      uint4* hp = reinterpret_cast<uint4*>(&xs[buf][0][sv][32 * kh]);
      hp[0] = xb[0];
      hp[1] = xb[1];
    }
  };
  // the wave's matrix rows c0 + 16 m + (lane % 16), inputs 32 ks + 8 q .. + 7
  float4 mr[2][2], mn[2][2];
  auto load_m = [&](int ks, float4 (&dst)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const float4* p = reinterpret_cast<const float4*>(a.M + (int64_t)(c0 + 16 * m + nl) * d + 32 * ks + 8 * q);
      dst[m][0] = p[0];
      dst[m][1] = p[1];
    }
  };
  // one step: this step's products from LDS buffer ks % 2 and the rows in
  // `cur` while the next step's inputs and rows load (into `nxt`); the loop
  // runs two steps per iteration so that the two row buffers swap roles
  // without copies
  auto step = [&](int ks, float4 (&cur)[2][2], float4 (&nxt)[2][2]) __attribute__((always_inline)) {
    const int buf = ks & 1;
    const bool more = ks + 1 < nks;
    if (more) {
      load_x(ks + 1);
      if (wave_on) load_m(ks + 1, nxt);
    }
    if (wave_on) {
      bf16x8 ah[2], al[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        uint32_t h[4], l[4];
        split_bf16(cur[m][0].x, cur[m][0].y, h[0], l[0]);
        split_bf16(cur[m][0].z, cur[m][0].w, h[1], l[1]);
        split_bf16(cur[m][1].x, cur[m][1].y, h[2], l[2]);
        split_bf16(cur[m][1].z, cur[m][1].w, h[3], l[3]);
        ah[m] = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
        al[m] = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const bf16x8 bh = *reinterpret_cast<const bf16x8*>(&xs[buf][0][16 * nt + nl][16 * q]);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          acc[m][nt] = mfma_bf16(ah[m], bh, acc[m][nt]);
          acc[m][nt] = mfma_bf16(al[m], bh, acc[m][nt]);
        }
        if constexpr (F32IN) {
          const bf16x8 bl = *reinterpret_cast<const bf16x8*>(&xs[buf][1][16 * nt + nl][16 * q]);
#pragma unroll
          for (int m = 0; m < 2; ++m) acc[m][nt] = mfma_bf16(ah[m], bl, acc[m][nt]);
        }
      }
    }
    if (more) stage(buf ^ 1);
    __syncthreads();
  };
  load_x(0);
  if (wave_on) load_m(0, mr);
  stage(0);
  __syncthreads();
  int ks = 0;
  for (; ks + 1 < nks; ks += 2) {
    step(ks, mr, mn);
    step(ks + 1, mn, mr);
  }
  if (ks < nks) step(ks, mr, mn);
  return ss;
}

// Tile of this workgroup (coordinate tiles of one vector tile on one XCD);
// false for the grid's padding.
__device__ __forceinline__ bool wide_tile(const WArgs& a, int& vt, int& ct) {
  const int nct = (a.d + kWC - 1) / kWC, nvt = (int)((a.nb + kWV - 1) / kWV);
  const int id = blockIdx.x, k8 = id >> 3;
  vt = (k8 / nct) * 8 + (id & 7);
  ct = k8 % nct;
  return vt < nvt;
}

template <bool F32IN, int B, bool PROD>
__global__ __launch_bounds__(kWThreads, 2) void wide_rotate_kernel(WArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][2][kWV][kWRowB];
  __shared__ float sinv[kWV];
  int vt, ct;
  if (!wide_tile(a, vt, ct)) return;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, nl = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int d = a.d, G = d / 32;
  const int c0 = ct * kWC + 32 * w;
  const bool wave_on = c0 < d;
  const int64_t lv0 = (int64_t)vt * kWV;
  constexpr int L = 1 << B;
  constexpr int P = B + (PROD ? 1 : 0);
  float th[L - 1], cv[L];
#pragma unroll
  for (int t = 0; t < L - 1; ++t) {
    th[t] = a.thr[t];
    asm volatile("" : "+v"(th[t]));  // held in a VGPR: the selects take one SGPR operand at most
  }
#pragma unroll
  for (int t = 0; t < L; ++t) {
    cv[t] = a.cent[t];
    asm volatile("" : "+v"(cv[t]));
  }
  v4f acc[2][8];
  float ss = wide_gemm<F32IN>(a, lv0, c0, wave_on, acc, xs);
  // |x| of the tile's vectors (two staging threads per vector)
  ss += __shfl_xor(ss, 1);
  if ((tid & 1) == 0) {
    const int sv = tid >> 1;
    const bool valid = lv0 + sv < a.nb;
    const float nrm = __builtin_amdgcn_sqrtf(ss);
    sinv[sv] = valid && nrm > 0.f ? __builtin_amdgcn_rcpf(nrm) : 0.f;
    if (ct == 0 && valid) a.norm[a.v0 + lv0 + sv] = tqd::f32_to_half_bits(nrm);
  }
  __syncthreads();
  if (!wave_on) return;
  const int64_t nround = (a.n + tqk::kKeysTile - 1) / tqk::kKeysTile * tqk::kKeysTile;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const int lvl = 16 * nt + nl;
    const int64_t lv = lv0 + lvl;
    const bool valid = lv < a.nb;
    const float inv = sinv[lvl];
    const bool live = inv > 0.f;
    const uint64_t vm = __builtin_amdgcn_ballot_w64(valid), lm = __builtin_amdgcn_ballot_w64(live);
    uint32_t acc8[B];
#pragma unroll
    for (int p = 0; p < B; ++p) acc8[p] = 0u;
    float rres[2][4];
    float r2 = 0.f;
    // (coordinates in descending order: the shift-ins build bit 4 m + r)
#pragma unroll
    for (int m = 1; m >= 0; --m)
#pragma unroll
      for (int r = 3; r >= 0; --r) {
        const float u = acc[m][nt][r] * inv;
        bool bt[B];
        interval_bits<B, B - 1>(u, th, bt);
#pragma unroll
        for (int p = 0; p < B; ++p) {
          const uint64_t c = __builtin_amdgcn_ballot_w64(bt[B - 1 - p]);
          acc8[p] = shift_in(acc8[p], (c & lm) | (p == B - 1 ? (vm & ~lm) : 0ull));
        }
        if constexpr (PROD) {
          const float rv = (u - pick<L, 0, 1>(cv, bt)) * (float)live;
          rres[m][r] = rv;
          r2 = fmaf(rv, rv, r2);
        }
      }
    uint32_t kw[B];
#pragma unroll
    for (int p = 0; p < B; ++p) kw[p] = key_word_of(acc8[p], q);
    // key tile (16 vectors) of this block; lane (q, nl) stores planes q, q + 4
    const int64_t vt16 = a.v0 + lv0 + 16 * nt;
    if (vt16 < nround) {
      uint32_t* dst = a.packed + ((vt16 / 16) * G + (c0 >> 5)) * 16 * P;
#pragma unroll
      for (int pass = 0; pass < (B + 3) / 4; ++pass) {
        const int p = 4 * pass + q;
        uint32_t wv = kw[4 * pass];
#pragma unroll
        for (int pp = 4 * pass + 1; pp < B && pp < 4 * pass + 4; ++pp) wv = (p == pp) ? kw[pp] : wv;
        if (p < B) dst[nl * P + p] = wv;
      }
    }
    if constexpr (PROD) {
      const float s = sum_q(r2);
      if (valid) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
          *reinterpret_cast<float4*>(a.res + lv * d + c0 + 16 * m + 4 * q) =
              make_float4(rres[m][0], rres[m][1], rres[m][2], rres[m][3]);
        if (q == 0) a.rho2[lv * G + (c0 >> 5)] = s;
      }
    }
  }
}

__global__ __launch_bounds__(kWThreads, 2) void wide_sketch_kernel(WArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][2][kWV][kWRowB];
  int vt, ct;
  if (!wide_tile(a, vt, ct)) return;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, nl = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int d = a.d, G = d / 32, P = a.B + 1;
  const int c0 = ct * kWC + 32 * w;
  const bool wave_on = c0 < d;
  const int64_t lv0 = (int64_t)vt * kWV;
  // |r~| from pass 1's partial sums (coordinate tile 0)
  if (ct == 0 && tid < kWV && lv0 + tid < a.nb) {
    const float* p = a.rho2 + (lv0 + tid) * G;
    float s = 0.f;
    for (int g = 0; g < G; ++g) s += p[g];
    a.rnorm[a.v0 + lv0 + tid] = tqd::f32_to_half_bits(__builtin_amdgcn_sqrtf(s));
  }
  v4f acc[2][8];
  (void)wide_gemm<true>(a, lv0, c0, wave_on, acc, xs);
  if (!wave_on) return;
  const int64_t nround = (a.n + tqk::kKeysTile - 1) / tqk::kKeysTile * tqk::kKeysTile;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const uint64_t vm = __builtin_amdgcn_ballot_w64(lv0 + 16 * nt + nl < a.nb);
    uint32_t acc8 = 0u;
#pragma unroll
    for (int m = 1; m >= 0; --m)
#pragma unroll
      for (int r = 3; r >= 0; --r) acc8 = shift_in(acc8, __builtin_amdgcn_ballot_w64(acc[m][nt][r] >= 0.f) & vm);
    const uint32_t kw = key_word_of(acc8, q);
    const int64_t vt16 = a.v0 + lv0 + 16 * nt;
    if (vt16 < nround && q == 0) a.packed[(((vt16 / 16) * G + (c0 >> 5)) * 16 + nl) * P + a.B] = kw;
  }
}

}  // namespace

namespace tqk {

bool quantize_mfma_supported(const tq_quantizer& q, tq_dtype dt, const void* x, int64_t stride) {
  const int64_t esz = dt == TQ_BF16 ? 2 : 4;
  return (q.d == 32 || q.d == 64 || q.d == 96 || q.d == 128) && ((stride * esz) % 16) == 0 &&
         ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
}

hipError_t launch_quantize_mfma(const tq_quantizer& q, tq_layout layout, tq_dtype dt, const void* x, int64_t n,
                                int64_t stride, void* packed, uint16_t* norm, uint16_t* rnorm, hipStream_t s) {
  QmArgs a{};
  a.x = x;
  a.n = n;
  a.stride = stride;
  a.bf16 = dt == TQ_BF16;
  a.R = q.R;
  a.S = q.S;
  a.B = q.mse_bits;
  a.prod = q.variant == TQ_PROD;
  a.layout = layout;
  // (value tiles: both tiles of the last 64-vector block, whose vectors interleave)
  a.ntiles = layout == TQ_LAYOUT_KEYS ? (n + kTile - 1) / kTile : (n + kValuesBlock - 1) / kValuesBlock * 2;
  for (int i = 0; i < TQ_MAX_LEVELS; ++i) a.cent[i] = q.centroids[i];
  for (int i = 0; i < TQ_MAX_LEVELS - 1; ++i) a.thr[i] = q.thresholds[i];
  a.packed = static_cast<uint32_t*>(packed);
  a.norm = norm;
  a.rnorm = rnorm;
  using Fn = void (*)(QmArgs);
  // [d / 32 - 1][bf16 input][mse bits - 1][prod][keys layout]
#define TQ_QM(D, BF, B) {{quantize_mfma_kernel<D, BF, B, false, false>, quantize_mfma_kernel<D, BF, B, false, true>}, \
                         {quantize_mfma_kernel<D, BF, B, true, false>, quantize_mfma_kernel<D, BF, B, true, true>}}
#define TQ_QD(D) {{TQ_QM(D, false, 1), TQ_QM(D, false, 2), TQ_QM(D, false, 3), TQ_QM(D, false, 4)}, \
                  {TQ_QM(D, true, 1), TQ_QM(D, true, 2), TQ_QM(D, true, 3), TQ_QM(D, true, 4)}}
  static const Fn fns[4][2][4][2][2] = {TQ_QD(32), TQ_QD(64), TQ_QD(96), TQ_QD(128)};
#undef TQ_QD
#undef TQ_QM
  const Fn fn = fns[q.d / 32 - 1][a.bf16 ? 1 : 0][a.B - 1][a.prod ? 1 : 0][layout == TQ_LAYOUT_KEYS ? 1 : 0];
  const int threads = 2 * q.d;
  // persistent grid: as many workgroups as the device holds at once (the
  // rotation-only kernels need far fewer registers and no S in LDS)
  // (both queried once per device and kernel, not per call)
  const int64_t slots = (int64_t)device_cus() * kernel_wgs_per_cu(reinterpret_cast<const void*>(fn), threads);
  const int64_t grid = a.ntiles < slots ? a.ntiles : slots;
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(threads), 0, s, a);
  return hipGetLastError();
}


bool quantize_wide_supported(const tq_quantizer& q, tq_layout layout, tq_dtype dt, const void* x, int64_t stride) {
  const int64_t esz = dt == TQ_BF16 ? 2 : 4;
  return layout == TQ_LAYOUT_KEYS && q.d > 128 && (q.d % 32) == 0 && ((stride * esz) % 16) == 0 &&
         ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
}

// Device workspace of the wide quantiser (the residuals of one batch),
// allocated on first use per device and kept until the process ends; grown
// when a call needs more.
static float* wide_workspace(size_t floats, hipError_t& err) {
  static std::mutex mu;
  static std::vector<std::pair<float*, size_t>> per_dev;
  int dev = 0;
  err = hipGetDevice(&dev);
  if (err != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)per_dev.size() <= dev) per_dev.resize(dev + 1, {nullptr, 0});
  auto& slot = per_dev[dev];
  if (slot.second < floats) {
    if (slot.first) {
      err = hipFree(slot.first);  // (waits for work in flight on the device)
      if (err != hipSuccess) return nullptr;
      slot = {nullptr, 0};
    }
    void* p = nullptr;
    err = hipMalloc(&p, floats * sizeof(float));
    if (err != hipSuccess) return nullptr;
    slot = {static_cast<float*>(p), floats};
  }
  return slot.first;
}

hipError_t launch_quantize_wide(const tq_quantizer& q, tq_dtype dt, const void* x, int64_t n, int64_t stride,
                                void* packed, uint16_t* norm, uint16_t* rnorm, hipStream_t s) {
  WArgs a{};
  a.x = x;
  a.stride = stride;
  a.M = q.R;
  a.n = n;
  a.d = q.d;
  a.B = q.mse_bits;
  for (int i = 0; i < TQ_MAX_LEVELS; ++i) a.cent[i] = q.centroids[i];
  for (int i = 0; i < TQ_MAX_LEVELS - 1; ++i) a.thr[i] = q.thresholds[i];
  a.packed = static_cast<uint32_t*>(packed);
  a.norm = norm;
  a.rnorm = rnorm;
  const bool prod = q.variant == TQ_PROD;
  if (prod) {
    hipError_t e;
    const int64_t batch = n < kWBatch ? n : kWBatch;
    float* ws = wide_workspace((size_t)batch * q.d + (size_t)batch * (q.d / 32), e);
    if (!ws) return e;
    a.res = ws;
    a.rho2 = ws + (size_t)batch * q.d;
  }
  using Fn = void (*)(WArgs);
#define TQ_WR(F, B) {wide_rotate_kernel<F, B, false>, wide_rotate_kernel<F, B, true>}
  static const Fn rot[2][4][2] = {{TQ_WR(false, 1), TQ_WR(false, 2), TQ_WR(false, 3), TQ_WR(false, 4)},
                                  {TQ_WR(true, 1), TQ_WR(true, 2), TQ_WR(true, 3), TQ_WR(true, 4)}};
#undef TQ_WR
  const Fn fr = rot[dt == TQ_F32 ? 1 : 0][q.mse_bits - 1][prod ? 1 : 0];
  const int nct = (q.d + kWC - 1) / kWC;
  for (int64_t v0 = 0; v0 < n; v0 += kWBatch) {
    a.v0 = v0;
    a.nb = n - v0 < kWBatch ? n - v0 : kWBatch;
    const int64_t nvt = (a.nb + kWV - 1) / kWV;
    const unsigned grid = (unsigned)((nvt + 7) / 8 * 8 * nct);
    WArgs a1 = a;
    a1.x = x;
    a1.stride = stride;
    a1.xrow0 = v0;
    a1.M = q.R;
    hipLaunchKernelGGL(fr, dim3(grid), dim3(kWThreads), 0, s, a1);
    if (prod) {
      WArgs a2 = a;
      a2.x = a.res;
      a2.stride = q.d;
      a2.xrow0 = 0;
      a2.M = q.S;
      hipLaunchKernelGGL(wide_sketch_kernel, dim3(grid), dim3(kWThreads), 0, s, a2);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tqk
