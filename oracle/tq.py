"""TurboQuant quantiser, estimator, decode attention and search (oracle, fp64).

Sources:
* riverfrot "TurboQuant" post, section 4.1: x~ = R (x / |x|) with a random
  orthogonal R; the norm |x| is kept.
* same post, section 4.2: per-coordinate Lloyd-Max scalar quantisation;
  quantise = count the boundaries the value passes, dequantise = look up the
  representative (worked 3-bit example: 0.065 lands in the sixth interval).
  No per-block scale or zero-point is stored.
* same post, section 4.3: stage 1 residual r = x - Q^-1(Q(x)); stage 2 QJL:
  random projection of r, keep only the signs (1 bit each); the estimate
  <y, Q^-1(Q(x)) + QJL^-1(QJL(r))> of <y, x> is unbiased, y unquantised.
  An MSE-only quantiser shrinks inner products (factor 2/pi at 1 bit).
* same post, sections 2.2-2.4: decode attention softmax(q K^T / sqrt(d)) V
  over all cached tokens; GQA (fewer KV heads than query heads); the KV
  size formula 2 x layers x kv_heads x head_dim x seq_len x bytes.
* uiyeonassociation post, results section: the same codes serve top-k
  inner-product vector search.

Readings where the pages are silent (each listed in the design notes):
* QJL acts on the residual in the rotated domain, r~ = x~ - c[idx], with a
  d x d matrix S of i.i.d. N(0,1) entries; the query side is S (R y). The
  scale that makes the sign sketch unbiased is gamma = sqrt(pi/2) / d
  (E[s sign(<s, r>)] = sqrt(2/pi) r/|r| for s ~ N(0, I)).
* "b-bit TurboQuant_prod" = (b-1) Lloyd-Max bits + 1 QJL bit.
* codes: idx_j = number of thresholds t_i with x~_j >= t_i (ties go up).
* sign(0) -> +1: z_j = [ (S r~)_j >= 0 ].
* |x| and |r~| are stored as IEEE half (round to nearest even); every
  reconstruction uses the stored halves.
* a zero vector stores n = 0, rho = 0, every code = L/2 and every sign = 1.

Pinned by tests/test_oracle_tq.py: unbiasedness over 10^4 seeds, the 2/pi
shrinkage law, the reconstruction-norm closed form, hand-derived codes for
basis vectors, nearest-centroid brute force, the page's worked 3-bit
example, textbook softmax attention on reconstructed vectors, and the
KV-size examples of section 2.4.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from . import codebook as _cb

KEYS_TILE = 16    # vectors per tile of the key (coordinate-contiguous) layout
VALUES_TILE = 32  # vectors per tile (word) of the value (token-contiguous) layout
VALUES_BLOCK = 64  # vectors per block of two value tiles (their tokens interleave)


@dataclass
class Quantizer:
    """One TurboQuant quantiser: dimension, MSE bits, variant, R, S, codebook."""

    d: int
    mse_bits: int
    prod: bool
    R: np.ndarray            # d x d, row-major, fp64 (widened from what the caller holds)
    S: np.ndarray | None     # d x d for PROD
    centroids: np.ndarray    # 2^B ascending, fp64
    thresholds: np.ndarray   # 2^B - 1 ascending, fp64

    @property
    def levels(self) -> int:
        return 1 << self.mse_bits

    @property
    def planes(self) -> int:
        return self.mse_bits + (1 if self.prod else 0)

    @property
    def gamma(self) -> float:
        return math.sqrt(math.pi / 2.0) / self.d


def symmetric_codebook(d: int, mse_bits: int):
    """Lloyd-Max codebook with the (exact) mirror symmetry c_i = -c_{L-1-i} imposed.

    The density is even and its Lloyd-Max fixed point unique, so the fixed
    point is symmetric; imposing it removes the last-ulp asymmetry of the
    iteration and makes the middle threshold exactly 0.
    """
    c, _, _, _ = _cb.lloyd_max(d, mse_bits)
    c = 0.5 * (c - c[::-1])
    t = 0.5 * (c[:-1] + c[1:])
    return c, t


def make_quantizer(d, mse_bits, prod, R, S=None, centroids=None, thresholds=None) -> Quantizer:
    if centroids is None:
        centroids, thresholds = symmetric_codebook(d, mse_bits)
    R = np.asarray(R, dtype=np.float64)
    S = None if S is None else np.asarray(S, dtype=np.float64)
    if prod and S is None:
        raise ValueError("PROD needs S")
    return Quantizer(d, mse_bits, bool(prod), R, S if prod else None,
                     np.asarray(centroids, np.float64), np.asarray(thresholds, np.float64))


@dataclass
class Codes:
    """Result of quantising N vectors (any leading batch shape ``shape``)."""

    idx: np.ndarray          # [..., d] uint8 codes
    z: np.ndarray | None     # [..., d] bool signs (PROD)
    n: np.ndarray            # [...] fp64 norms (exact)
    rho: np.ndarray          # [...] fp64 residual norms (exact; 0 for MSE)
    n16: np.ndarray          # [...] float16 stored norms
    rho16: np.ndarray        # [...] float16 stored residual norms
    urot: np.ndarray         # [..., d] fp64 rotated unit vectors (decision values)
    proj: np.ndarray | None  # [..., d] fp64 S r~ (sign decision values)


def quantize(x, q: Quantizer) -> Codes:
    """Quantise each row of x (shape [..., d]) in fp64, step by step."""
    x = np.asarray(x, dtype=np.float64)
    shape = x.shape[:-1]
    X = x.reshape(-1, q.d)
    # 1. norm and direction
    n = np.sqrt(np.sum(X * X, axis=1))
    zero = n == 0.0
    u = np.zeros_like(X)
    u[~zero] = X[~zero] / n[~zero, None]
    # 2. random rotation  x~ = R u
    urot = u @ q.R.T
    # 3. scalar quantisation against the thresholds (count passed boundaries)
    idx = np.sum(urot[:, :, None] >= q.thresholds[None, None, :], axis=2).astype(np.uint8)
    idx[zero] = q.levels // 2
    rho = np.zeros(len(X))
    z = proj = None
    if q.prod:
        # 4. residual in the rotated domain and its norm
        r = urot - q.centroids[idx]
        r[zero] = 0.0
        rho = np.sqrt(np.sum(r * r, axis=1))
        # 5. QJL: project with S, keep the signs
        proj = r @ q.S.T
        z = proj >= 0.0
        z[zero] = True
    codes = Codes(
        idx=idx.reshape(shape + (q.d,)),
        z=None if z is None else z.reshape(shape + (q.d,)),
        n=n.reshape(shape), rho=rho.reshape(shape),
        n16=n.astype(np.float16).reshape(shape),
        rho16=rho.astype(np.float16).reshape(shape),
        urot=urot.reshape(shape + (q.d,)),
        proj=None if proj is None else proj.reshape(shape + (q.d,)),
    )
    return codes


def dequantize(c: Codes, q: Quantizer) -> np.ndarray:
    """Reconstruction x^ = n (R^T c[idx] + gamma rho R^T S^T (2z - 1)), from stored halves."""
    n = c.n16.astype(np.float64)[..., None]
    rot = q.centroids[c.idx.astype(np.int64)]
    if q.prod:
        sig = np.where(c.z, 1.0, -1.0)
        rot = rot + q.gamma * c.rho16.astype(np.float64)[..., None] * (sig @ q.S)
    return n * (rot @ q.R)


def estimate_ip(y, c: Codes, q: Quantizer) -> np.ndarray:
    """Estimated <y_m, x_i> for queries y [M, d] against quantised rows -> [M, N].

    est = n (<R y, c[idx]> + gamma rho <S R y, 2z - 1>), y unquantised.
    """
    y = np.asarray(y, dtype=np.float64).reshape(-1, q.d)
    yr = y @ q.R.T
    idx = c.idx.reshape(-1, q.d).astype(np.int64)
    n = c.n16.reshape(-1).astype(np.float64)
    s = yr @ q.centroids[idx].T
    if q.prod:
        ys = yr @ q.S.T
        sig = np.where(c.z.reshape(-1, q.d), 1.0, -1.0)
        rho = c.rho16.reshape(-1).astype(np.float64)
        s = s + q.gamma * rho[None, :] * (ys @ sig.T)
    return s * n[None, :]


# ----------------------------------------------------------------------------
# Packed layouts (library's own choice; the pages fix none)
#
# KEYS (coordinate-contiguous), tiles of 16 vectors, uint32 words indexed
#   [tile][g][t][p], g = coordinate word (d/32 of them), t = vector in tile,
#   p = plane (0..B-1: code bit p, LSB first; B: QJL sign, PROD only);
#   bit i of the word = coordinate 32 g + i.
# VALUES (token-contiguous), tiles of 32 vectors, words indexed [tile][j][p],
#   j = coordinate. Tiles come in blocks of two covering 64 vectors: vector
#   64 B + t (t = 0..63) sits in tile 2 B + (t // 8) % 2, at bit
#   16 (t % 2) + 4 (t // 16) + (t % 8) // 2 of its words (value_tile_bit
#   below), so a tile holds the vectors t = 16 q + 8 s + e (q = 0..3,
#   e = 0..7) of its block.
# Vectors past N in the last block are all-zero bits.
# ----------------------------------------------------------------------------

def value_tile_bit(t):
    """(tile within the block, bit) of vector t (0..63) of a 64-vector block of the value layout."""
    return (t // 8) % 2, 16 * (t % 2) + 4 * (t // 16) + (t % 8) // 2


# [block position t] -> position in the block's two tiles' bits (tile * 32 + bit)
_VALUE_POS = np.array([32 * value_tile_bit(t)[0] + value_tile_bit(t)[1] for t in range(64)])
_VALUE_ORDER = np.argsort(_VALUE_POS)  # tile * 32 + bit -> block position t


def _planes(idx, z, mse_bits):
    N, d = idx.shape
    P = mse_bits + (0 if z is None else 1)
    pl = np.zeros((N, P, d), dtype=bool)
    for p in range(mse_bits):
        pl[:, p] = (idx >> p) & 1
    if z is not None:
        pl[:, mse_bits] = z
    return pl


def _bits_to_words(bits):  # [..., 32] bool -> [...] uint32
    w = np.zeros(bits.shape[:-1], dtype=np.uint64)
    for i in range(32):
        w |= bits[..., i].astype(np.uint64) << np.uint64(i)
    return w.astype(np.uint32)


def _words_to_bits(w):  # [...] uint32 -> [..., 32] bool, bit i of the word at position i
    b = np.ascontiguousarray(w, dtype="<u4").view(np.uint8).reshape(w.shape + (4,))
    return np.unpackbits(b, axis=-1, bitorder="little").reshape(w.shape + (32,)).astype(bool)


def packed_words(d, mse_bits, prod, n, layout):
    P = mse_bits + (1 if prod else 0)
    unit = KEYS_TILE if layout == "keys" else VALUES_BLOCK
    return -(-n // unit) * unit * d * P // 32


def pack(idx, z, mse_bits, layout):
    """Pack codes [N, d] (+ signs) into the named layout; returns uint32 words."""
    idx = np.asarray(idx).reshape(-1, idx.shape[-1])
    N, d = idx.shape
    if z is not None:
        z = np.asarray(z).reshape(N, d)
    pl = _planes(idx, z, mse_bits)
    P = pl.shape[1]
    unit = KEYS_TILE if layout == "keys" else VALUES_BLOCK
    NT = -(-N // unit)
    full = np.zeros((NT * unit, P, d), dtype=bool)
    full[:N] = pl
    if layout == "keys":
        G = d // 32
        w = _bits_to_words(full.reshape(NT * unit, P, G, 32))           # [V, P, G]
        w = w.reshape(NT, unit, P, G).transpose(0, 3, 1, 2)             # [tile, g, t, p]
    elif layout == "values":
        b = full.reshape(NT, unit, P, d)[:, _VALUE_ORDER]               # [block, tile * 32 + bit, p, j]
        b = b.reshape(NT, 2, 32, P, d).transpose(0, 1, 4, 3, 2)         # [block, tile, j, p, bit]
        w = _bits_to_words(b)                                           # [block, tile, j, p]
    else:
        raise ValueError(layout)
    return np.ascontiguousarray(w).reshape(-1)


def unpack(words, N, d, mse_bits, prod, layout):
    """Inverse of ``pack``: returns (idx [N, d] uint8, z [N, d] bool or None)."""
    P = mse_bits + (1 if prod else 0)
    unit = KEYS_TILE if layout == "keys" else VALUES_BLOCK
    NT = -(-N // unit)
    w = np.asarray(words, dtype=np.uint32)
    if layout == "keys":
        G = d // 32
        w = w.reshape(NT, G, unit, P).transpose(0, 2, 3, 1)            # [tile, t, p, g]
        pl = _words_to_bits(w).reshape(NT * unit, P, d)
    else:
        w = w.reshape(NT, 2, d, P)                                      # [block, tile, j, p]
        bits = _words_to_bits(w)                                        # [block, tile, j, p, bit]
        bits = bits.transpose(0, 1, 4, 3, 2).reshape(NT, 64, P, d)      # [block, tile * 32 + bit, p, j]
        pl = bits[:, _VALUE_POS].reshape(NT * unit, P, d)
    pl = pl[:N]
    idx = np.zeros((N, d), dtype=np.uint8)
    for p in range(mse_bits):
        idx |= (pl[:, p].astype(np.uint8) << p)
    z = pl[:, mse_bits].copy() if prod else None
    return idx, z


# ----------------------------------------------------------------------------
# Decode attention over the compressed cache
# ----------------------------------------------------------------------------

@dataclass
class Group:
    """A contiguous channel range [lo, lo + q.d) quantised by its own quantiser."""

    lo: int
    q: Quantizer
    codes: Codes   # arrays shaped [B, Hkv, T, ...]


def decode_scores(qry, kgroups, Hkv):
    """Raw estimated <q_h, k_t> for every (b, h, t): [B, Hq, T] fp64."""
    qry = np.asarray(qry, dtype=np.float64)
    B, Hq, _ = qry.shape
    G = Hq // Hkv
    T = kgroups[0].codes.idx.shape[2]
    s = np.zeros((B, Hq, T))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for grp in kgroups:
                y = qry[b, h, grp.lo:grp.lo + grp.q.d][None, :]
                c = grp.codes
                # the estimator reads only the stored fields: codes, signs, halves
                sub = Codes(c.idx[b, g], None if c.z is None else c.z[b, g], None, None,
                            c.n16[b, g], c.rho16[b, g], None, None)
                s[b, h] += estimate_ip(y, sub, grp.q)[0]
    return s


def decode_attention(qry, kgroups, vgroups, Hkv, seq_lens=None, scale=None):
    """softmax(scale * est<q, k>) over t < seq_len, applied to the reconstructed values.

    qry [B, Hq, D]; query head h reads KV head h // (Hq / Hkv). Plain (not
    online) softmax in fp64. Returns (out [B, Hq, D_v], scores [B, Hq, T]),
    scores being the raw estimates (before the scale).
    """
    qry = np.asarray(qry, dtype=np.float64)
    B, Hq, D = qry.shape
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    scores = decode_scores(qry, kgroups, Hkv)
    T = scores.shape[2]
    if seq_lens is None:
        seq_lens = np.full(B, T)
    Dv = sum(g.q.d for g in vgroups)
    out = np.zeros((B, Hq, Dv))
    vhat = {}
    for gi, grp in enumerate(vgroups):
        c = grp.codes
        vhat[gi] = dequantize(c, grp.q)     # [B, Hkv, T, d_g]
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        for h in range(Hq):
            g = h // G
            logit = scale * scores[b, h, :L]
            w = np.exp(logit - logit.max())
            p = w / w.sum()
            for gi, grp in enumerate(vgroups):
                out[b, h, grp.lo:grp.lo + grp.q.d] = p @ vhat[gi][b, g, :L]
    return out, scores


# ----------------------------------------------------------------------------
# Inner-product search
# ----------------------------------------------------------------------------

def search_topk(queries, codes: Codes, q: Quantizer, k: int, chunk: int = 65536):
    """Top-k database rows by estimated inner product; ties -> lower index.

    Scores are computed in chunks of database rows (plain fp64 GEMMs), then
    each query's candidates are ordered by (-score, index).
    """
    queries = np.asarray(queries, dtype=np.float64)
    N = codes.idx.shape[0]
    Q = queries.shape[0]
    best_s = np.full((Q, 0), -np.inf)
    best_i = np.zeros((Q, 0), dtype=np.int64)
    for lo in range(0, N, chunk):
        hi = min(N, lo + chunk)
        sub = Codes(codes.idx[lo:hi], None if codes.z is None else codes.z[lo:hi], None, None,
                    codes.n16[lo:hi], codes.rho16[lo:hi], None, None)
        s = estimate_ip(queries, sub, q)
        cand_s = np.concatenate([best_s, s], axis=1)
        cand_i = np.concatenate([best_i, np.broadcast_to(np.arange(lo, hi), (Q, hi - lo))], axis=1)
        order = np.lexsort((cand_i, -cand_s), axis=1)[:, :k]
        best_s = np.take_along_axis(cand_s, order, axis=1)
        best_i = np.take_along_axis(cand_i, order, axis=1)
    return best_i, best_s


def exact_topk(queries, db, k):
    """Exact fp64 inner-product top-k (ties -> lower index): the recall reference."""
    s = np.asarray(queries, np.float64) @ np.asarray(db, np.float64).T
    order = np.lexsort((np.broadcast_to(np.arange(s.shape[1]), s.shape), -s), axis=1)[:, :k]
    return order, np.take_along_axis(s, order, axis=1)


def recall_at_k(found, truth):
    k = truth.shape[1]
    return float(np.mean([len(set(f[:k]) & set(t)) / k for f, t in zip(found, truth)]))


# ----------------------------------------------------------------------------
# KV-cache size (riverfrot post, section 2.4)
# ----------------------------------------------------------------------------

def kv_cache_bytes(layers, kv_heads, head_dim, seq_len, bytes_per_elem):
    """2 x layers x kv_heads x head_dim x seq_len x bytes (K and V)."""
    return 2 * layers * kv_heads * head_dim * seq_len * bytes_per_elem


def compressed_kv_bytes(layers, kv_heads, seq_len, k_groups, v_groups):
    """Compressed K + V bytes: per token and KV head, each group stores
    (planes x d / 8) packed bytes plus its half-precision norms
    (n and rho for PROD, n for MSE). Groups are (d, mse_bits, prod) triples."""
    per_tok = 0
    for (d, B, prod) in list(k_groups) + list(v_groups):
        per_tok += (B + (1 if prod else 0)) * d // 8 + (4 if prod else 2)
    return layers * kv_heads * seq_len * per_tok


# ----------------------------------------------------------------------------
# Key/value bit allocation from the norm ratio (riverfrot post, section 4.5)
# ----------------------------------------------------------------------------

KV_UNIFORM, KV_ASYMMETRIC, KV_MIXED = 0, 1, 2


def kv_norm_sensitivity(key_norm, value_norm):
    """How much more the keys' quantisation error weighs than the values':
    the error of a quantised vector scales with its squared norm, so the
    ratio is (key_norm / value_norm)^2 (section 4.5's "~37,000x" for key
    norms up to 778 against value norms of 4)."""
    return (float(key_norm) / float(value_norm)) ** 2


def kv_bit_allocation(key_norm, value_norm):
    """Section 4.5's rule for the K/V norm ratio r = key_norm / value_norm:
    r < 10 -> uniform 3-bit keys and values; 10 <= r <= 60 -> asymmetric,
    4-bit keys and 2-bit values; r > 100 -> mixed precision (per channel
    group). The section leaves 60 < r <= 100 open: read as asymmetric (the
    next stated threshold is 100). Returns (class, key_bits, value_bits); a
    mixed allocation keeps 4/2 as the base widths of its channel groups.
    Parity: the section's own table (pinned in the tests at each band)."""
    k, v = float(key_norm), float(value_norm)
    if not (np.isfinite(k) and np.isfinite(v) and k > 0 and v > 0):
        raise ValueError("norms must be finite and positive")
    r = k / v
    if r < 10.0:
        return KV_UNIFORM, 3, 3
    if r <= 100.0:
        return KV_ASYMMETRIC, 4, 2
    return KV_MIXED, 4, 2
