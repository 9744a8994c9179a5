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
// scan2 (bf16 matrix cores; used for 3 code bits with QJL): the
//        codebook is mirror-symmetric, so c[idx] = sum_{|S| odd} alpha_S
//        prod_{p in S} (2 b_p - 1), and each product of signs is 2 (xor of
//        planes) - 1. The query side carries alpha_S y~ per term and
//        gamma y^ for the QJL term, split into bf16 high and low parts
//        (qsplit_kernel); the database side is the xor-ed plane bits as bf16 {0, 2} (2.0 is
//        a single bit, so a packed 16-bit shift and a mask place it), or
//        {0, 2 rho} split the same way for the QJL term, so every
//        product is exact up to the splits (about 2^-17 relative per term,
//        fp32 accumulation). The constant parts sum_S alpha_S sum y~ and
//        rho gamma sum y^ are removed per (query, vector) at the end.
//        v_mfma_f32_16x16x32_bf16 contracts 32 coordinates at once: lane
//        group kq carries coordinates 32 g + 8 kq .. + 7 on both operands.
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

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ v4f mfma_bf16(bf16x8 a, bf16x8 b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// bf16 high and low parts (round to nearest even) of two floats, two to a
// register; s0, s1 return hi + lo as floats (the values the products use).
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo, float& s0, float& s1) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{x0, x1}, bf16x2));
  const float h0 = __uint_as_float(hi << 16), h1 = __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{x0 - h0, x1 - h1}, bf16x2));
  s0 = h0 + __uint_as_float(lo << 16);
  s1 = h1 + __uint_as_float(lo & 0xffff0000u);
}

constexpr int kMaxTerms = 9;  // up to 8 odd subsets + the QJL term

struct QsArgs {
  const float* qt;  // [Q][d]
  const float* qh;  // [Q][d]
  uint16_t* ops;    // [Q][terms][2][d] bf16 bits (high, low)
  float* cq;        // [Q][2]: sum_S alpha_S sum_c y~_c, gamma sum_c y^_c (as split)
  int Q, d;
  float gamma;
  float alpha[kMaxTerms];
};

// Per query: the bf16 operand planes of every term and the constant parts.
template <int B, bool PROD>
__global__ __launch_bounds__(kThreads) void qsplit_kernel(QsArgs a) {
  constexpr int TW = 1 << (B - 1), T = TW + (PROD ? 1 : 0);
  __shared__ float red[2][kThreads / 64];
  const int qi = blockIdx.x, tid = threadIdx.x;
  const float* yt = a.qt + (int64_t)qi * a.d;
  const float* yh = a.qh + (int64_t)qi * a.d;
  uint32_t* ops = reinterpret_cast<uint32_t*>(a.ops + (int64_t)qi * T * 2 * a.d);
  float c1 = 0.f, c2 = 0.f;
  for (int c = 2 * tid; c < a.d; c += 2 * kThreads) {
    const float t0 = yt[c], t1 = yt[c + 1];
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      uint32_t hi, lo;
      float s0, s1;
      // (the scan's B operand for these terms is 2 b, so A is alpha_S y~)
      split2(a.alpha[t] * t0, a.alpha[t] * t1, hi, lo, s0, s1);
      ops[((t * 2 + 0) * a.d + c) >> 1] = hi;
      ops[((t * 2 + 1) * a.d + c) >> 1] = lo;
      c1 += s0 + s1;
    }
    if (PROD) {
      uint32_t hi, lo;
      float s0, s1;
      split2(a.gamma * yh[c], a.gamma * yh[c + 1], hi, lo, s0, s1);
      ops[(((T - 1) * 2 + 0) * a.d + c) >> 1] = hi;
      ops[(((T - 1) * 2 + 1) * a.d + c) >> 1] = lo;
      c2 += s0 + s1;
    }
  }
  c1 = tqd::wave_sum(c1);
  c2 = tqd::wave_sum(c2);
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = c1;
    red[1][tid >> 6] = c2;
  }
  __syncthreads();
  if (tid == 0) {
    float s1 = 0.f, s2 = 0.f;
    for (int w = 0; w < kThreads / 64; ++w) {
      s1 += red[0][w];
      s2 += red[1][w];
    }
    a.cq[2 * qi] = s1;
    a.cq[2 * qi + 1] = s2;
  }
}

struct Scan2Args {
  const uint32_t* packed;
  int64_t packed_bytes;
  const uint16_t* norm;
  const uint16_t* rnorm;
  const uint16_t* ops;  // [Q][terms][2][d]
  const float* cq;      // [Q][2]
  float* scores;        // [Q][N]
  int64_t N;
  int Q, d;
};

// Odd subsets of B planes in ascending bitmask order (the order of the
// coefficients the host passes).
__host__ __device__ constexpr int odd_subset(int B, int t) {
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

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Byte k of w in both 16-bit halves (one byte permute).
__device__ __forceinline__ uint32_t byte_twice(uint32_t w, int k) {
  return __builtin_amdgcn_perm(w, w, (uint32_t)k | (0x0cu << 8) | ((uint32_t)k << 16) | (0x0cu << 24));
}

// Eight bits (a byte held in both halves of tt; bit e = coordinate e) as
// eight bf16 values 2 * bit, two to a register (register j: coordinate 2 j
// in the low half, 2 j + 1 in the high half). bf16 2.0 is the single bit
// 0x4000, so each half is the byte shifted to put its bit on bit 14 (one
// packed 16-bit shift), then masked.
__device__ __forceinline__ bf16x8 bits_to_bf16_two(uint32_t tt) {
  uint32_t r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u16x2 sh = {(unsigned short)(14 - 2 * j), (unsigned short)(13 - 2 * j)};
    r[j] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, tt) << sh) & 0x40004000u;
  }
  return __builtin_bit_cast(bf16x8, make_uint4(r[0], r[1], r[2], r[3]));
}

// The same bits as bf16 values magh * bit and magl * bit (bf16 bit patterns
// below 2^16): bits moved to bit 0 of each half, then one 24-bit multiply.
__device__ __forceinline__ void bits_to_bf16_mag(uint32_t tt, uint32_t magh, uint32_t magl, bf16x8& bh, bf16x8& bl) {
  uint32_t rh[4], rl[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u16x2 sh = {(unsigned short)(2 * j), (unsigned short)(2 * j + 1)};
    const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, tt) >> sh) & 0x00010001u;
    rh[j] = b * magh;
    rl[j] = b * magl;
  }
  bh = __builtin_bit_cast(bf16x8, make_uint4(rh[0], rh[1], rh[2], rh[3]));
  bl = __builtin_bit_cast(bf16x8, make_uint4(rl[0], rl[1], rl[2], rl[3]));
}

// Workgroup: 64 queries x 256 database vectors, 4 waves; wave w takes query
// tiles 2 (w % 2) and 2 (w % 2) + 1 and database tiles 8 (w / 2) .. + 7.
template <int B, bool PROD>
__global__ __launch_bounds__(kThreads, 2) void scan2_kernel(Scan2Args a) {
  constexpr int TW = 1 << (B - 1), T = TW + (PROD ? 1 : 0), P = B + (PROD ? 1 : 0);
  static_assert(P == 4, "one byte per plane in a register");
  // query operands of a 32-coordinate group, two groups in flight:
  // [buffer][term][plane][query][chunk of 8 coordinates]; chunk c of query
  // row r is stored at c ^ ((r / 2) % 4). Filled by direct global-to-LDS
  // loads (lane L of a load lands 16 L bytes past the instruction's base),
  // so the next group's operands arrive while this group is multiplied.
  __shared__ uint4 aq[2][T][2][kQB][4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kq = lane >> 4, nl = lane & 15;
  const int64_t vb = (int64_t)blockIdx.x * kNB;
  const int q0 = blockIdx.y * kQB;
  const int G = a.d / 32;
  const int64_t last_tile = (a.N - 1) / tqk::kKeysTile;
  const int qt0 = 2 * (w & 1), dt0 = 8 * (w >> 1);
  int64_t tile[8];
  uint32_t r2h[8], r2l[8];  // bf16 bits of 2 rho, high and low parts
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    tile[j] = min((vb >> 4) + dt0 + j, last_tile);
    const int64_t v = vb + 16 * (dt0 + j) + nl;
    const int64_t vr = v < a.N ? v : a.N - 1;
    if (PROD) {
      const float rho2 = 2.f * tqd::half_bits_to_f32(a.rnorm[vr]);
      const uint32_t hb = __builtin_bit_cast(uint16_t, (__bf16)rho2);
      r2h[j] = hb;
      r2l[j] = __builtin_bit_cast(uint16_t, (__bf16)(rho2 - __uint_as_float(hb << 16)));
    } else {
      r2h[j] = r2l[j] = 0u;
    }
  }
  v4f acc[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // this lane's plane words of its 8 database tiles, one coordinate group
  // ahead (group g + 1 is loaded while group g is processed)
  uint32_t wA[8][P], wB[8][P];
  // (through a buffer resource: uniform byte offset per tile and group, one
  // lane offset; the database is below 4 GB, which the host checks)
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint32_t*>(a.packed), (short)0, (int)(uint32_t)min(a.packed_bytes, (int64_t)0xffffffff), 0x00020000);
  const uint32_t word_off = (uint32_t)(nl * P * 4);
  auto load_words = [&](int g, uint32_t (&wn)[8][P]) __attribute__((always_inline)) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t soff = (uint32_t)((tile[j] * G + g) * (tqk::kKeysTile * P * 4));
      const u4 u = __builtin_amdgcn_raw_buffer_load_b128(wres, word_off, soff, 0);
      wn[j][0] = u[0];
      wn[j][1] = u[1];
      wn[j][2] = u[2];
      wn[j][3] = u[3];
    }
  };
  // staging of group g into buffer bf: plane tp (= term * 2 + plane) of rows
  // 16 w .. 16 w + 15 is one wave-wide load per plane; lane L carries row
  // 16 w + L / 4, physical chunk L % 4 (logical chunk (L % 4) ^ ((row / 2) % 4)).
  // The per-lane byte offset is the same for every plane and group; the
  // plane and group enter through the uniform base.
  uint32_t stage_off;
  {
    const int row = 16 * w + (lane >> 2);
    const int qr = min(q0 + row, a.Q - 1);
    const int c = (lane & 3) ^ ((row >> 1) & 3);
    stage_off = (uint32_t)(((int64_t)qr * T * 2 * a.d + 8 * c) * sizeof(uint16_t));
  }
  const __amdgpu_buffer_rsrc_t ores = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(a.ops), (short)0, (int)((int64_t)a.Q * T * 2 * a.d * 2), 0x00020000);
  auto stage = [&](int g, int bf) {
#pragma unroll
    for (int tp = 0; tp < 2 * T; ++tp)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ores, (__attribute__((address_space(3))) void*)&aq[bf][tp >> 1][tp & 1][16 * w][0],
                                               16, stage_off, (uint32_t)((tp * a.d + 32 * g) * 2), 0, 0);
  };
  load_words(0, wA);
  stage(0, 0);
  // one group; its words are in wn, the next group's go to wnext (the loop
  // below alternates two arrays, so no words are copied)
  auto group = [&](int g, const uint32_t (&wn)[8][P], uint32_t (&wnext)[8][P]) __attribute__((always_inline)) {
    const int bf = g & 1;
    // this group's staged operands and words have arrived (own loads), and
    // every wave's (barrier)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // this lane's bits (coordinates 32 g + 8 kq .. + 7) of the P = 4 planes
    // of each database tile, one byte per plane
    uint32_t wc[8];
    {
      const uint32_t sel = (uint32_t)kq | ((4u + kq) << 8) | 0x0c0c0000u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t lo = __builtin_amdgcn_perm(wn[j][1], wn[j][0], sel);
        const uint32_t hi = __builtin_amdgcn_perm(wn[j][3], wn[j][2], sel);
        wc[j] = lo | (hi << 16);
      }
    }
    // query operands of the wave's two query tiles (row 16 qt + nl, chunk kq)
    bf16x8 A[2][T][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 16 * (qt0 + i) + nl;
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int pl = 0; pl < 2; ++pl)
          A[i][t][pl] = __builtin_bit_cast(bf16x8, aq[bf][t][pl][row][kq ^ ((row >> 1) & 3)]);
    }
    // the next group's operands and words (buffer bf ^ 1 was last read in
    // group g - 1, which every wave finished before the barrier above)
    if (g + 1 < G) {
      stage(g + 1, bf ^ 1);
      load_words(g + 1, wnext);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bf16x8 Bw[TW];
#pragma unroll
      for (int t = 0; t < TW; ++t) {
        const int S = odd_subset(B, t);
        uint32_t x = 0u;
#pragma unroll
        for (int pp = 0; pp < B; ++pp)
          if ((S >> pp) & 1) x ^= wc[j] >> (8 * pp);
        Bw[t] = bits_to_bf16_two(byte_twice(x, 0));  // bf16 2.0 per set bit
      }
      bf16x8 Bh = Bw[0], Bl = Bw[0];
      if (PROD) bits_to_bf16_mag(byte_twice(wc[j], P - 1), r2h[j], r2l[j], Bh, Bl);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int t = 0; t < TW; ++t) {
          acc[i][j] = mfma_bf16(A[i][t][0], Bw[t], acc[i][j]);
          acc[i][j] = mfma_bf16(A[i][t][1], Bw[t], acc[i][j]);
        }
        if (PROD) {
          acc[i][j] = mfma_bf16(A[i][T - 1][0], Bh, acc[i][j]);
          acc[i][j] = mfma_bf16(A[i][T - 1][0], Bl, acc[i][j]);
          acc[i][j] = mfma_bf16(A[i][T - 1][1], Bh, acc[i][j]);
        }
      }
    }
  };
  for (int g = 0; g < G; g += 2) {
    group(g, wA, wB);
    if (g + 1 < G) group(g + 1, wB, wA);
  }
  // scores of queries q0 + 16 qt + 4 kq + r and vectors vb + 16 (dt0 + j) + nl:
  // n (acc - C1 - rho C2)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int qi = q0 + 16 * (qt0 + i) + 4 * kq + r;
      if (qi < a.Q) {
        const float c1 = a.cq[2 * qi], c2 = a.cq[2 * qi + 1];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int64_t v = vb + 16 * (dt0 + j) + nl;
          if (v < a.N) {
            const float n = tqd::half_bits_to_f32(a.norm[v]);
            const float rho = PROD ? tqd::half_bits_to_f32(a.rnorm[v]) : 0.f;
            a.scores[(int64_t)qi * a.N + v] = n * (acc[i][j][r] - c1 - rho * c2);
          }
        }
      }
    }
}

}  // namespace

namespace tqk {

bool search_mfma_supported(const tq_group& db) { return db.q.d % 32 == 0 && db.q.d >= 32; }

// The bf16 scan serves codes of 3 bits with the QJL sign (4-bit search
// codes); other widths take the fp32 scan.
static bool scan2_supported(const tq_group& db, int64_t N, int Q) {
  // (buffer offsets into the database and the query operands are 32-bit)
  const int64_t bytes = (N + kKeysTile - 1) / kKeysTile * kKeysTile * (db.q.d / 32) * 4 * 4;
  const int64_t qbytes = (int64_t)Q * 5 * 2 * db.q.d * 2;
  return db.q.variant == TQ_PROD && db.q.mse_bits == 3 && bytes < ((int64_t)1 << 32) && qbytes < ((int64_t)1 << 31);
}

size_t search_mfma_extra_bytes(const tq_group& db, int Q) {
  if (!search_mfma_supported(db) || !scan2_supported(db, 0, Q)) return 0;
  const int T = (1 << (db.q.mse_bits - 1)) + 1;
  return (size_t)Q * T * 2 * db.q.d * sizeof(uint16_t) + (size_t)Q * 2 * sizeof(float);
}

hipError_t launch_search_mfma_scores(const tq_group& db, int64_t N, const float* queries, int Q, float* qt,
                                     float* qh, float* scores, void* extra, hipStream_t s) {
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
  if (extra && scan2_supported(db, N, Q)) {
    const int B = db.q.mse_bits, T = (1 << (B - 1)) + 1;
    QsArgs qa{};
    qa.qt = qt;
    qa.qh = qh;
    qa.ops = static_cast<uint16_t*>(extra);
    qa.cq = reinterpret_cast<float*>(qa.ops + (size_t)Q * T * 2 * d);
    qa.Q = Q;
    qa.d = d;
    qa.gamma = (float)(sqrt(M_PI / 2.0) / d);
    // Walsh coefficients of the mirror-symmetric codebook, odd subsets in
    // ascending bitmask order: alpha_S = mean over idx of c[idx] prod_{p in S} (2 b_p - 1)
    int nt = 0;
    for (int S = 1; S < (1 << B); ++S) {
      if (!(__builtin_popcount(S) & 1)) continue;
      double acc = 0.0;
      for (int idx = 0; idx < (1 << B); ++idx) {
        double chi = 1.0;
        for (int p = 0; p < B; ++p)
          if ((S >> p) & 1) chi *= ((idx >> p) & 1) ? 1.0 : -1.0;
        acc += chi * (double)db.q.centroids[idx];
      }
      qa.alpha[nt++] = (float)(acc / (1 << B));
    }
    Scan2Args sa{};
    sa.packed = static_cast<const uint32_t*>(db.packed);
    sa.packed_bytes = (int64_t)((N + kKeysTile - 1) / kKeysTile) * kKeysTile * (d / 32) * 4 * 4;
    sa.norm = db.norm;
    sa.rnorm = db.rnorm;
    sa.ops = qa.ops;
    sa.cq = qa.cq;
    sa.scores = scores;
    sa.N = N;
    sa.Q = Q;
    sa.d = d;
    const dim3 grid2((unsigned)((N + kNB - 1) / kNB), (Q + kQB - 1) / kQB);
    hipLaunchKernelGGL((qsplit_kernel<3, true>), dim3(Q), dim3(kThreads), 0, s, qa);
    hipLaunchKernelGGL((scan2_kernel<3, true>), grid2, dim3(kThreads), 0, s, sa);
    return hipGetLastError();
  }
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
