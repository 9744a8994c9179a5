// One tile of the general TurboQuant quantiser: device code shared by the
// quantiser launches of quantize.hip and by the decode step's append, which
// runs inside the decode's query-transform launch (decode_mfma.hip).
//
// riverfrot "TurboQuant" post, section 4.1: x~ = R (x / |x|) with a random
// orthogonal R; section 4.2: each coordinate is mapped to the index of the
// Lloyd-Max interval it falls in (boundaries compared, codebook looked up);
// section 4.3: the residual r~ = x~ - c[idx] is projected with a Gaussian
// matrix S and only the signs are kept (1 bit each), together with |r~|.
//
// One workgroup quantises a tile of TV vectors. The tile is staged in LDS
// coordinate-major; each d x d product is computed as a tile GEMM in fp32
// FMA (fp32 accumulation, fixed summation order j = 0..d-1) with the matrix
// streamed through LDS in chunks of 128 rows x 32 columns (128 columns for
// tiles of 2-4 vectors), the next chunk's loads in flight while one is
// multiplied. Codes, signs and norms are then packed into the requested
// layout (key words gathered by wave ballots). The same kernel serves
// appends: each vector is then written to a caller-given cache row (one
// token per sequence and head during decoding, or the rows of a paged
// block), keys as whole words, values as one bit per tile word; one launch
// can carry a key cache and a value cache (grid row 0 and 1).
#pragma once

#include "device_common.h"
#include "internal.h"

namespace tqq {

constexpr int kQThreads = 256;  // threads of a quantiser workgroup
constexpr int kIC = 128;        // output coordinates per chunk (one per thread column)
constexpr int kMtStride = kIC + 1;
// Input coordinates per chunk of the matrix staged in LDS: small tiles (few
// vectors, latency-bound) stage 128 columns per round, large tiles 32.
template <int TV>
constexpr int jc_of() { return TV <= 4 ? 128 : 32; }

struct QArgs {
  const void* x;
  int64_t n;
  int64_t stride;
  int bf16;
  const float* R;
  const float* S;
  int d;
  int B;
  int prod;
  int layout;
  float cent[TQ_MAX_LEVELS];
  float thr[TQ_MAX_LEVELS - 1];
  uint32_t* packed;
  uint16_t* norm;
  uint16_t* rnorm;
  const int64_t* rows;  // append: cache row of each vector (null: vector i is row i)
  int64_t cache_rows;
  // decode-step append (when rows is null): vector i = b Hkv + g is the new
  // token of sequence b, KV head g, written to row i seq_stride + len_b - 1
  // with len_b = step_lens[b] (rows of sequences with len_b outside
  // 1 .. seq_stride are skipped)
  const int32_t* step_lens;
  int Hkv;
  int64_t seq_stride;
};

// Cache row of vector gv of an append (-1: skipped).
__device__ __forceinline__ int64_t dest_row(const QArgs& a, int64_t gv) {
  if (a.rows) return a.rows[gv];
  const int len = a.step_lens[gv / a.Hkv];
  return (len >= 1 && len <= a.seq_stride) ? gv * a.seq_stride + (len - 1) : -1;
}


// Vector (row of x) that slot v of tile blk quantises. A bulk value-layout
// tile (32 slots) takes the vectors its memory tile holds, slot v = bit v of
// the tile's words (the vectors of a 64-vector block interleave over its two
// tiles); every other tile takes vectors blk TV .. blk TV + TV - 1.
template <int TV>
__device__ __forceinline__ int64_t tile_vec(const QArgs& a, int64_t blk, int v) {
  if (TV == tqk::kValuesTile && a.layout == TQ_LAYOUT_VALUES && !a.rows && !a.step_lens)
    return (blk >> 1) * tqk::kValuesBlock + tqk::value_tok((int)(blk & 1), v);
  return blk * TV + v;
}

// Out[j][v] = sum_k M[j][k] In[k][v] for the TV vectors of the tile (arrays
// coordinate-major, row stride TV). Thread (ii, vh) owns output coordinate
// i0 + ii of vectors vh*TV/2 .. vh*TV/2 + TV/2 - 1.
template <int TV, int JC>
__device__ void matvec_tile(const float* __restrict__ M, int d, const float* In, float* Out, float* Mt) {
  constexpr int kJC = JC;
  constexpr int kLoads = kIC * kJC / 4 / kQThreads;  // 16-byte loads per thread per chunk
  const int tid = threadIdx.x;
  const int ii = tid % kIC;
  const int vh = tid / kIC;
  constexpr int VH = TV / 2;
  // chunks (output rows i0 .. i0 + 127) x (input columns j0 .. j0 + kJC - 1),
  // walked row block by row block; the next chunk's loads are issued before
  // the current chunk is multiplied, so they arrive meanwhile. (d is a
  // multiple of 32: a 128-column chunk may run past d, a 32-column one never
  // does; addresses are clamped into the matrix and values outside it zeroed.)
  const int nJ = (d + kJC - 1) / kJC;
  const int nQ = ((d + kIC - 1) / kIC) * nJ;
  float4 mv[kLoads];
  auto load = [&](int q) __attribute__((always_inline)) {
    const int i0 = (q / nJ) * kIC, j0 = (q % nJ) * kJC, jn = min(kJC, d - j0);
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int e4 = tid + u * kQThreads;
      const int r = e4 / (kJC / 4), c = 4 * (e4 % (kJC / 4));
      const int i = min(i0 + r, d - 1), cc = min(c, jn - 4);
      mv[u] = *reinterpret_cast<const float4*>(M + (int64_t)i * d + j0 + cc);
    }
  };
  load(0);
  float acc[VH];
#pragma unroll
  for (int k = 0; k < VH; ++k) acc[k] = 0.f;
  for (int q = 0; q < nQ; ++q) {
    const int i0 = (q / nJ) * kIC, j0 = (q % nJ) * kJC, jn = min(kJC, d - j0);
    __syncthreads();  // the previous chunk's products are done with Mt
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int e4 = tid + u * kQThreads;
      const int r = e4 / (kJC / 4), c = 4 * (e4 % (kJC / 4));
      const bool ok = i0 + r < d && c < jn;
      Mt[(c + 0) * kMtStride + r] = ok ? mv[u].x : 0.f;
      Mt[(c + 1) * kMtStride + r] = ok ? mv[u].y : 0.f;
      Mt[(c + 2) * kMtStride + r] = ok ? mv[u].z : 0.f;
      Mt[(c + 3) * kMtStride + r] = ok ? mv[u].w : 0.f;
    }
    __syncthreads();
    load(min(q + 1, nQ - 1));  // (the last chunk re-reads itself)
    if (i0 + ii < d) {
      for (int jj = 0; jj < jn; ++jj) {
        const float m = Mt[jj * kMtStride + ii];
        const float* in = In + (j0 + jj) * TV + vh * VH;
#pragma unroll
        for (int k = 0; k < VH; ++k) acc[k] = fmaf(m, in[k], acc[k]);
      }
    }
    if (q % nJ == nJ - 1) {  // row block done
      if (i0 + ii < d) {
#pragma unroll
        for (int k = 0; k < VH; ++k) Out[(i0 + ii) * TV + vh * VH + k] = acc[k];
      }
#pragma unroll
      for (int k = 0; k < VH; ++k) acc[k] = 0.f;
    }
  }
  __syncthreads();
}

// Products of a matrix with tiles of at most 2 vectors of d <= 128
// coordinates (appends), with no staging: thread t owns output coordinate
// t / 2 and half t % 2 of its row, whose d / 2 entries it loads straight into
// registers (all at once, one memory round trip), and the two halves' sums
// meet by a lane exchange.
constexpr int kDirectMaxD = 128;
__device__ __forceinline__ void load_half_row(const float* __restrict__ M, int d, float4 (&m)[kDirectMaxD / 8]) {
  const int i = min((int)threadIdx.x >> 1, d - 1), h = threadIdx.x & 1;
  const float4* p = reinterpret_cast<const float4*>(M + (int64_t)i * d + h * (d / 2));
#pragma unroll
  for (int k = 0; k < kDirectMaxD / 8; ++k) m[k] = k < d / 8 ? p[k] : make_float4(0.f, 0.f, 0.f, 0.f);
}
template <int TV>
__device__ void matvec_direct(const float4 (&m)[kDirectMaxD / 8], int d, const float* In, float* Out) {
  static_assert(2 * kDirectMaxD == kQThreads, "two threads per output coordinate");
  const int i = threadIdx.x >> 1, h = threadIdx.x & 1;
  const float* in = In + h * (d / 2) * TV;
  float acc[TV];
#pragma unroll
  for (int v = 0; v < TV; ++v) acc[v] = 0.f;
#pragma unroll
  for (int k = 0; k < kDirectMaxD / 8; ++k) {
    if (k < d / 8) {
      const float mv[4] = {m[k].x, m[k].y, m[k].z, m[k].w};
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int v = 0; v < TV; ++v) acc[v] = fmaf(mv[c], in[(4 * k + c) * TV + v], acc[v]);
    }
  }
#pragma unroll
  for (int v = 0; v < TV; ++v) acc[v] += __shfl_xor(acc[v], 1, tqd::kWave);
  if (i < d && h == 0) {
#pragma unroll
    for (int v = 0; v < TV; ++v) Out[i * TV + v] = acc[v];
  }
  __syncthreads();
}

// Key-layout word of vector v, coordinate word g, code bit sh (4: the sign)
// for the half-wave this lane is in: lane i of the half takes coordinate
// 32 g + i, a ballot gathers the 32 bits, and the half's word is returned to
// all its lanes. Every lane of the wave must call it (a wave-wide ballot).
__device__ __forceinline__ uint32_t key_word(const uint8_t* C, int TV, int v, int g, int sh, int lane) {
  const int i = lane & 31;
  const bool bit = (C[(32 * g + i) * TV + v] >> sh) & 1;
  const uint64_t m = __ballot(bit);
  return (uint32_t)(m >> (32 * (lane >> 5)));
}

// Quantise tile blk (the vectors tile_vec<TV> names) of a.x with a
// workgroup of kQThreads threads; smem holds lds_bytes(a.d, TV, JC) bytes.
// DIRECT (tiles of at most 2 vectors): matrices of d <= 128 go straight to
// registers (lower latency, about 128 more registers per thread).
template <int TV, int JC, bool DIRECT = false>
__device__ void quantize_tile(const QArgs& a, int64_t blk, float* smem) {
  static_assert(!DIRECT || TV <= 2, "direct products take tiles of at most 2 vectors");
  __shared__ float nrm[TV], rho[TV];
  __shared__ float cent[TQ_MAX_LEVELS], thr[TQ_MAX_LEVELS];
  const int d = a.d;
  float* Mt = smem;
  float* In = Mt + JC * kMtStride;
  float* Out = In + d * TV;
  uint8_t* C = reinterpret_cast<uint8_t*>(Out + d * TV);
  const int tid = threadIdx.x, lane = tid % tqd::kWave, wv = tid / tqd::kWave;
  const int64_t v0 = blk * TV;
  const int L = 1 << a.B;
  // tiles of appends (2 vectors, d <= 128): R and S rows straight to
  // registers, their loads issued before anything else
  const bool direct = DIRECT && d <= kDirectMaxD;
  float4 rm[kDirectMaxD / 8], sm[kDirectMaxD / 8];
  if constexpr (DIRECT) {
    if (direct) {
      load_half_row(a.R, d, rm);
      if (a.prod) load_half_row(a.S, d, sm);
    }
  }

  if (tid < TQ_MAX_LEVELS) {
    cent[tid] = a.cent[tid];
    thr[tid] = tid < TQ_MAX_LEVELS - 1 ? a.thr[tid] : 0.f;
  }
  // 1. load the tile, coordinate-major (vectors past n are zero)
  for (int e = tid; e < TV * d; e += kQThreads) {
    const int v = e / d, j = e % d;
    const int64_t gv = tile_vec<TV>(a, blk, v);
    In[j * TV + v] = gv < a.n ? tqd::load_elem(a.x, gv * a.stride + j, a.bf16) : 0.f;
  }
  __syncthreads();
  // 2. norms
  for (int v = wv; v < TV; v += kQThreads / tqd::kWave) {
    float s = 0.f;
    for (int j = lane; j < d; j += tqd::kWave) s = fmaf(In[j * TV + v], In[j * TV + v], s);
    s = tqd::wave_sum(s);
    if (lane == 0) nrm[v] = sqrtf(s);
  }
  // 3. rotation (unnormalised: R x, divided by |x| below)
  if constexpr (DIRECT) {
    if (direct)
      matvec_direct<TV>(rm, d, In, Out);
    else
      matvec_tile<TV, JC>(a.R, d, In, Out, Mt);
  } else {
    matvec_tile<TV, JC>(a.R, d, In, Out, Mt);
  }
  // 4. codes; the rotated residual replaces the input tile
  for (int e = tid; e < TV * d; e += kQThreads) {
    const int v = e % TV;
    const float n = nrm[v];
    const float u = n > 0.f ? Out[e] / n : 0.f;
    int idx = 0;
    for (int k = 0; k < L - 1; ++k) idx += (u >= thr[k]) ? 1 : 0;
    if (!(n > 0.f)) idx = L / 2;
    C[e] = (uint8_t)idx;
    In[e] = n > 0.f ? u - cent[idx] : 0.f;
  }
  __syncthreads();
  if (a.prod) {
    for (int v = wv; v < TV; v += kQThreads / tqd::kWave) {
      float s = 0.f;
      for (int j = lane; j < d; j += tqd::kWave) s = fmaf(In[j * TV + v], In[j * TV + v], s);
      s = tqd::wave_sum(s);
      if (lane == 0) rho[v] = sqrtf(s);
    }
    // 5. QJL projection of the residual; keep the signs (sign(0) -> +)
    if constexpr (DIRECT) {
      if (direct)
        matvec_direct<TV>(sm, d, In, Out);
      else
        matvec_tile<TV, JC>(a.S, d, In, Out, Mt);
    } else {
      matvec_tile<TV, JC>(a.S, d, In, Out, Mt);
    }
    for (int e = tid; e < TV * d; e += kQThreads) {
      const int v = e % TV;
      const bool z = (Out[e] >= 0.f) || !(nrm[v] > 0.f);
      C[e] |= (uint8_t)(z ? 16 : 0);
    }
    __syncthreads();
  }
  // 6. pack
  const int P = a.B + a.prod;
  if (a.rows || a.step_lens) {
    // append: every vector goes to its own cache row. A key row owns its
    // words; a value row owns one bit of each of its tile's words, set or
    // cleared atomically (rows of one call are distinct, so the updates of a
    // word commute). Rows outside the cache are skipped.
    if (a.layout == TQ_LAYOUT_KEYS) {
      const int G = d / 32;
      for (int w0 = 2 * wv; w0 < TV * G * P; w0 += 2 * (kQThreads / tqd::kWave)) {
        const int e = w0 + (lane >> 5);
        const int p = e % P, g = (e / P) % G, v = e / (P * G);
        const int64_t gv = v0 + v;
        const uint32_t w = key_word(C, TV, v, g, p < a.B ? p : 4, lane);
        if ((lane & 31) || gv >= a.n) continue;
        const int64_t row = dest_row(a, gv);
        if (row < 0 || row >= a.cache_rows) continue;
        const int64_t tile = row / tqk::kKeysTile;
        const int t = (int)(row % tqk::kKeysTile);
        a.packed[((tile * G + g) * tqk::kKeysTile + t) * P + p] = w;
      }
    } else {
      for (int e = tid; e < TV * d * P; e += kQThreads) {
        const int p = e % P, j = (e / P) % d, v = e / (P * d);
        const int64_t gv = v0 + v;
        if (gv >= a.n) continue;
        const int64_t row = dest_row(a, gv);
        if (row < 0 || row >= a.cache_rows) continue;
        const int sh = p < a.B ? p : 4;
        const int t = (int)(row % tqk::kValuesBlock);
        const uint32_t bit = 1u << (uint32_t)tqk::value_bit(t);
        const int64_t tile = row / tqk::kValuesBlock * 2 + tqk::value_tile(t);
        uint32_t* wp = a.packed + (tile * d + j) * P + p;
        if ((C[j * TV + v] >> sh) & 1)
          atomicOr(wp, bit);
        else
          atomicAnd(wp, ~bit);
      }
    }
    for (int v = tid; v < TV; v += kQThreads) {
      const int64_t gv = v0 + v;
      if (gv >= a.n) continue;
      const int64_t row = dest_row(a, gv);
      if (row < 0 || row >= a.cache_rows) continue;
      a.norm[row] = tqd::f32_to_half_bits(nrm[v]);
      if (a.prod) a.rnorm[row] = tqd::f32_to_half_bits(rho[v]);
    }
    return;
  }
  if (a.layout == TQ_LAYOUT_KEYS) {
    const int G = d / 32;
    const int64_t nround = (a.n + tqk::kKeysTile - 1) / tqk::kKeysTile * tqk::kKeysTile;
    for (int w0 = 2 * wv; w0 < TV * G * P; w0 += 2 * (kQThreads / tqd::kWave)) {
      const int e = w0 + (lane >> 5);
      const int p = e % P, g = (e / P) % G, v = e / (P * G);
      const int64_t gv = v0 + v;
      // (padding vectors of the last tile pack to zero words; the ballot
      // itself runs on every lane)
      uint32_t w = key_word(C, TV, v, g, p < a.B ? p : 4, lane);
      if (gv >= a.n) w = 0u;
      if ((lane & 31) || gv >= nround) continue;
      const int64_t tile = gv / tqk::kKeysTile;
      const int t = (int)(gv % tqk::kKeysTile);
      a.packed[((tile * G + g) * tqk::kKeysTile + t) * P + p] = w;
    }
  } else {
    // TV == 32 == the values tile; slot v is bit v of the tile's words
    for (int e = tid; e < d * P; e += kQThreads) {
      const int p = e % P, j = e / P;
      const int sh = p < a.B ? p : 4;
      uint32_t w = 0;
      for (int v = 0; v < TV; ++v)
        if (tile_vec<TV>(a, blk, v) < a.n) w |= (uint32_t)((C[j * TV + v] >> sh) & 1) << v;
      a.packed[(blk * d + j) * P + p] = w;
    }
  }
  // 7. norms as IEEE half
  for (int v = tid; v < TV; v += kQThreads) {
    const int64_t gv = tile_vec<TV>(a, blk, v);
    if (gv < a.n) {
      a.norm[gv] = tqd::f32_to_half_bits(nrm[v]);
      if (a.prod) a.rnorm[gv] = tqd::f32_to_half_bits(rho[v]);
    }
  }
}

inline QArgs make_args(const tq_quantizer& q, tq_layout layout, tq_dtype dt, const void* x, int64_t n,
                       int64_t stride, void* packed, uint16_t* norm, uint16_t* rnorm, const int64_t* rows,
                       int64_t cache_rows) {
  QArgs a{};
  a.rows = rows;
  a.cache_rows = cache_rows;
  a.x = x;
  a.n = n;
  a.stride = stride;
  a.bf16 = dt == TQ_BF16;
  a.R = q.R;
  a.S = q.S;
  a.d = q.d;
  a.B = q.mse_bits;
  a.prod = q.variant == TQ_PROD;
  a.layout = layout;
  for (int i = 0; i < TQ_MAX_LEVELS; ++i) a.cent[i] = q.centroids[i];
  for (int i = 0; i < TQ_MAX_LEVELS - 1; ++i) a.thr[i] = q.thresholds[i];
  a.packed = static_cast<uint32_t*>(packed);
  a.norm = norm;
  a.rnorm = rnorm;
  return a;
}

// The appends of a decode step: one argument set per key group, then one per
// value group, each taking its channels of the B x Hkv new rows; returns the
// number of sets written to out.
inline int step_args(const tq_kv_desc& k, const tq_kv_desc& v, const tqk::StepRows& st, int B, int Hkv,
                     QArgs* out) {
  int n = 0, D = 0, Dv = 0;
  for (int i = 0; i < k.n_groups; ++i) D += k.g[i].q.d;
  for (int i = 0; i < v.n_groups; ++i) Dv += v.g[i].q.d;
  const int64_t nv = (int64_t)B * Hkv;
  const int esz = st.dt == TQ_BF16 ? 2 : 4;
  for (int t = 0; t < 2; ++t) {
    const tq_kv_desc& c = t == 0 ? k : v;
    const char* x = static_cast<const char*>(t == 0 ? st.k_new : st.v_new);
    for (int i = 0; i < c.n_groups; ++i) {
      const tq_group& g = c.g[i];
      // (the step writes into the cache the descriptors point at)
      QArgs a = make_args(g.q, t == 0 ? TQ_LAYOUT_KEYS : TQ_LAYOUT_VALUES, st.dt, x + (size_t)g.ch_offset * esz, nv,
                          t == 0 ? D : Dv, const_cast<void*>(g.packed), const_cast<uint16_t*>(g.norm),
                          g.q.variant == TQ_PROD ? const_cast<uint16_t*>(g.rnorm) : nullptr, nullptr,
                          nv * g.seq_stride);
      a.step_lens = st.seq_lens;
      a.Hkv = Hkv;
      a.seq_stride = g.seq_stride;
      out[n++] = a;
    }
  }
  return n;
}

// Dynamic LDS bytes of quantize_tile<TV, JC> for d-wide vectors.
inline size_t lds_bytes(int d, int TV, int JC) {
  return (size_t)(JC * kMtStride + 2 * d * TV) * 4 + (size_t)d * TV;
}

}  // namespace tqq
