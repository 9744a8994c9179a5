"""Helpers for the GPU parity tests: device round trips and acceptance rules.

Acceptance (TurboQuant quantiser on fp32 hardware against the fp64 oracle):
* codes bit-exact, except coordinate j of vector i when the oracle's rotated
  value lies within 1e-5 of a decision threshold;
* signs bit-exact, except the whole sign plane of a vector with an excluded
  code, and sign j when |(S r~)_j| < 1e-5 in the oracle;
* stored half norms bit-exact, except when the oracle's fp64 norm lies within
  a relative 1e-5 of the midpoint between two adjacent halves (the
  round-to-nearest decision point);
* scores and outputs within 2e-3 relative, normwise per (batch, head) row;
* top-k identical except for positions whose oracle scores tie within 1e-6.
"""
from __future__ import annotations

import numpy as np

from oracle import tq as otq

CODE_WINDOW = 1e-5
NORM_REL_WINDOW = 1e-5
REL_TOL = 2e-3


def torch_dev(a, dtype=None):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def code_exclusions(codes: otq.Codes, q: otq.Quantizer):
    """Boolean masks (code_excluded [N, d], sign_excluded [N, d])."""
    u = codes.urot.reshape(-1, q.d)
    gap = np.min(np.abs(u[:, :, None] - q.thresholds[None, None, :]), axis=2)
    cex = gap < CODE_WINDOW
    sex = np.zeros_like(cex)
    if q.prod:
        sex = np.abs(codes.proj.reshape(-1, q.d)) < CODE_WINDOW
        sex |= np.any(cex, axis=1, keepdims=True)
    # a zero vector's codes and signs are fixed by convention, not decided:
    # they must match exactly
    zero = codes.n.reshape(-1) == 0.0
    cex[zero] = False
    sex[zero] = False
    return cex, sex


def half_near_tie(x64: np.ndarray) -> np.ndarray:
    """True where rounding x to half sits within NORM_REL_WINDOW of a midpoint."""
    x64 = np.asarray(x64, np.float64).reshape(-1)
    h = x64.astype(np.float16)
    up = np.nextafter(h, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(h, np.float16(-np.inf)).astype(np.float64)
    hf = h.astype(np.float64)
    mid = np.where(x64 >= hf, 0.5 * (hf + up), 0.5 * (hf + dn))
    return np.abs(x64 - mid) <= NORM_REL_WINDOW * np.maximum(np.abs(x64), 1e-30)


def assert_codes_match(gpu_idx, gpu_z, gpu_n16, gpu_r16, codes: otq.Codes, q: otq.Quantizer,
                       max_excluded_frac=0.01):
    N = gpu_idx.shape[0]
    cex, sex = code_exclusions(codes, q)
    oi = codes.idx.reshape(N, q.d)
    bad = (gpu_idx != oi) & ~cex
    assert not bad.any(), f"{bad.sum()} code mismatches outside the threshold window, first at {np.argwhere(bad)[:3]}"
    assert cex.mean() <= max_excluded_frac
    if q.prod:
        oz = codes.z.reshape(N, q.d)
        badz = (gpu_z != oz) & ~sex
        assert not badz.any(), f"{badz.sum()} sign mismatches, first at {np.argwhere(badz)[:3]}"
    on = codes.n.reshape(-1)
    nex = half_near_tie(on)
    badn = (gpu_n16.view(np.uint16) != codes.n16.reshape(-1).view(np.uint16)) & ~nex
    assert not badn.any(), f"{badn.sum()} norm mismatches, e.g. {np.argwhere(badn)[:3].ravel()}"
    if q.prod:
        rex = half_near_tie(codes.rho.reshape(-1)) | np.any(cex, axis=1)
        badr = (gpu_r16.view(np.uint16) != codes.rho16.reshape(-1).view(np.uint16)) & ~rex
        assert not badr.any(), f"{badr.sum()} residual-norm mismatches, e.g. {np.argwhere(badr)[:3].ravel()}"


def normwise_rel_err(got, want, axis=-1):
    """max over rows of |got - want|_2 / |want|_2 (rows along ``axis``)."""
    num = np.linalg.norm(np.asarray(got, np.float64) - want, axis=axis)
    den = np.linalg.norm(want, axis=axis)
    return float(np.max(num / np.maximum(den, 1e-300)))


def rowmax_rel_err(got, want, axis=-1):
    """max over rows of max_t |got - want| / max_t |want| (the score rule)."""
    num = np.max(np.abs(np.asarray(got, np.float64) - want), axis=axis)
    den = np.max(np.abs(want), axis=axis)
    return float(np.max(num / np.maximum(den, 1e-300)))


def assert_topk_match(gpu_idx, gpu_score, full_scores, k, tie=1e-6):
    """GPU top-k against the oracle's full fp64 score matrix (ties within `tie`)."""
    Q = full_scores.shape[0]
    for i in range(Q):
        s = full_scores[i]
        order = np.lexsort((np.arange(len(s)), -s))[:k]
        g = gpu_idx[i]
        assert len(set(g.tolist())) == k, "duplicate indices"
        kth = s[order[-1]]
        for r in range(k):
            if g[r] != order[r]:
                assert abs(s[g[r]] - s[order[r]]) < tie, (i, r, g[r], order[r], s[g[r]], s[order[r]])
            assert s[g[r]] >= kth - tie
        np.testing.assert_allclose(gpu_score[i], s[g], rtol=1e-4, atol=1e-6)
