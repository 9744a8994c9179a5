"""Seeded synthetic inputs shared by the fp64 oracle and the HIP path.

This module holds no arithmetic of the TurboQuant method. It only draws the
random numbers the method consumes (the Haar rotation R and the Gaussian QJL
matrix S are random draws, so both sides receive them as inputs) and the
synthetic workloads whose shapes and laws follow the pages' examples:

* Llama-3.1-8B attention shapes (32 query heads, 8 KV heads, head_dim 128) and
  context lengths of 32K-128K (riverfrot "TurboQuant" post, section 2.4);
* unit-normalised Gaussian vectors for the inner-product checks;
* a Gaussian-mixture database standing in for the unnamed vector-search
  datasets of the paper summary (uiyeonassociation post, results section).

Every generator is deterministic in (seed, stream); numpy PCG64 is used for
host data. Large workloads that only the GPU can hold are generated on the
device by ``synth.device`` with torch's Philox generator from the same seeds.
"""
from __future__ import annotations

import numpy as np

# Named sub-streams of one seed, so that the data, R and S of a run are
# independent draws that do not shift when another stream's size changes.
STREAM_DATA = 0
STREAM_QUERY = 1
STREAM_R = 2
STREAM_S = 3
STREAM_OUTLIER = 4
STREAM_R_V = 5
STREAM_S_V = 6
STREAM_NORM = 7


def rng(seed: int, stream: int) -> np.random.Generator:
    """Independent PCG64 generator for (seed, stream)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(stream)])))


def haar_orthogonal(d: int, seed: int, stream: int = STREAM_R, dtype=np.float32) -> np.ndarray:
    """Haar-distributed d x d orthogonal matrix, row-major.

    Drawn as the Q factor of a Gaussian matrix with the column signs fixed by
    the diagonal of R (Mezzadri's construction), so that the law is exactly
    Haar. Returned in ``dtype`` (fp32 is what the library consumes; fp64 is
    used only by tests that need an exactly orthogonal matrix).
    """
    g = rng(seed, stream).standard_normal((d, d))
    q, r = np.linalg.qr(g)
    q = q * np.sign(np.diag(r))[None, :]
    return np.ascontiguousarray(q.astype(dtype))


def gaussian_matrix(m: int, d: int, seed: int, stream: int = STREAM_S, dtype=np.float32) -> np.ndarray:
    """m x d matrix of i.i.d. N(0, 1) entries, row-major."""
    return np.ascontiguousarray(rng(seed, stream).standard_normal((m, d)).astype(dtype))


def unit_gaussian(n: int, d: int, seed: int, stream: int = STREAM_DATA, dtype=np.float32) -> np.ndarray:
    """n rows drawn i.i.d. N(0, I_d) and scaled to unit norm (in fp64, then cast)."""
    x = rng(seed, stream).standard_normal((n, d))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    return np.ascontiguousarray(x.astype(dtype))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest-even); return the raw uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def outlier_channels(n_sets: int, d: int, n_out: int, seed: int, stream: int = STREAM_OUTLIER) -> np.ndarray:
    """For each of n_sets KV heads, n_out distinct channel indices (sorted)."""
    g = rng(seed, stream)
    return np.stack([np.sort(g.choice(d, size=n_out, replace=False)) for _ in range(n_sets)])


def kv_with_outliers(B: int, H: int, T: int, d: int, n_out: int, scale: float, seed: int,
                     data_stream: int, outlier_stream: int) -> np.ndarray:
    """bf16-valued [B, H, T, d] tensor (returned as fp32 holding bf16 values).

    Entries are N(0, 1); per KV head, ``n_out`` seeded channels are multiplied
    by ``scale`` (the outlier channels of real keys and values).
    """
    x = rng(seed, data_stream).standard_normal((B, H, T, d), dtype=np.float32)
    ch = outlier_channels(H, d, n_out, seed, outlier_stream)
    for h in range(H):
        x[:, h, :, ch[h]] *= scale
    return bf16_bits_to_f32(to_bf16_bits(x))


def lognormal_norm_vectors(n: int, d: int, seed: int, sigma: float = 0.5) -> np.ndarray:
    """x = l * g / |g| with g ~ N(0, I) and l ~ LogNormal(0, sigma), bf16-valued fp32."""
    g = rng(seed, STREAM_DATA).standard_normal((n, d))
    g /= np.linalg.norm(g, axis=1, keepdims=True)
    ell = rng(seed, STREAM_NORM).lognormal(0.0, sigma, size=(n, 1))
    return bf16_bits_to_f32(to_bf16_bits((g * ell).astype(np.float32)))


def gaussian_mixture(n: int, d: int, n_comp: int, seed: int, stream: int = STREAM_DATA,
                     means: np.ndarray | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Unit-normalised draws from a uniform mixture of N(mu_k, I), mu_k ~ N(0, I).

    Returns (x [n, d] fp32, means [n_comp, d] fp64). Pass ``means`` to draw a
    second sample (the queries) from the same mixture.
    """
    if means is None:
        means = rng(seed, STREAM_OUTLIER).standard_normal((n_comp, d))
    g = rng(seed, stream)
    comp = g.integers(0, n_comp, size=n)
    x = means[comp] + g.standard_normal((n, d))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    return np.ascontiguousarray(x.astype(np.float32)), means


def plant_needles(K: np.ndarray, qdir: np.ndarray, cosine: float, seed: int, stream: int = STREAM_QUERY):
    """Needle-in-a-haystack keys: one planted key per (sequence, KV head).

    K [B, H, T, d] (modified in place and returned with the positions [B, H]);
    qdir [B, H, d] the query each needle is aimed at. The needle has cosine
    ``cosine`` with qdir (the rest a random direction orthogonal to it) and
    the median key norm of its (sequence, head); bf16-valued like K.
    """
    B, H, T, d = K.shape
    g = rng(seed, stream)
    pos = g.integers(0, T, size=(B, H))
    qh = qdir / np.linalg.norm(qdir, axis=-1, keepdims=True)
    rnd = g.standard_normal((B, H, d))
    rnd -= np.sum(rnd * qh, axis=-1, keepdims=True) * qh
    rnd /= np.linalg.norm(rnd, axis=-1, keepdims=True)
    knorm = np.median(np.linalg.norm(K.astype(np.float64), axis=-1), axis=-1)
    needle = (cosine * qh + np.sqrt(1.0 - cosine * cosine) * rnd) * knorm[..., None]
    needle = bf16_bits_to_f32(to_bf16_bits(needle.astype(np.float32)))
    for b in range(B):
        for h in range(H):
            K[b, h, pos[b, h]] = needle[b, h]
    return K, pos
