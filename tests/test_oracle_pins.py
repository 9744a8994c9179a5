"""More pins of the oracle, each against something other than its own code path (CPU).

Sources: riverfrot "TurboQuant" post, section 4.2 (Lloyd-Max codebook of the
rotated-coordinate law), section 4.3 (two-stage quantiser, unbiased
estimator), section 5.5 (distortion table: cosine similarity and per-element
MSE at 4, 3 and 2 bits), sections 2.2-2.3 (decode attention); the
uiyeonassociation post, results section (top-k inner-product search scored
by recall).
"""
import math

import numpy as np
import pytest
from scipy import integrate
from scipy.special import gammaln, softmax

import synth
from oracle import codebook as cb
from oracle import tq


# --------------------------------------------------------------------------
# codebook values at d = 128, 3 bits (section 4.2)
# --------------------------------------------------------------------------

def test_codebook_d128_b3_values_and_fixed_point_by_quadrature():
    c, t = tq.symmetric_codebook(128, 3)
    # four-digit positive halves of the Lloyd-Max codebook for d = 128, B = 3
    assert np.allclose(c[4:], [0.0216, 0.0666, 0.1181, 0.1884], atol=5e-5)
    assert np.allclose(t[3:], [0.0, 0.0441, 0.0924, 0.1533], atol=5e-5)
    # and the Lloyd-Max conditions re-derived by adaptive quadrature of the
    # marginal density (not the oracle's incomplete-beta / closed-form moments):
    # each centroid is the conditional mean of its cell, thresholds are midpoints
    d = 128
    logc = gammaln(d / 2) - 0.5 * math.log(math.pi) - gammaln((d - 1) / 2)
    f = lambda x: math.exp(logc + (d - 3) / 2 * math.log1p(-x * x))
    edges = [-1.0] + list(t) + [1.0]
    for i in range(8):
        m0 = integrate.quad(f, edges[i], edges[i + 1], epsabs=0, epsrel=1e-13, limit=200)[0]
        m1 = integrate.quad(lambda x: x * f(x), edges[i], edges[i + 1], epsabs=0, epsrel=1e-13, limit=200)[0]
        assert abs(m1 / m0 - c[i]) < 1e-10, (i, m1 / m0, c[i])
    np.testing.assert_allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-15)


# --------------------------------------------------------------------------
# orientation of R and S (section 4.1: x~ = R x/|x|; section 4.3: signs of S r~)
# --------------------------------------------------------------------------

def _signed_permutation(d, mult, add, sign_rule):
    """M with M[perm(j), j] = sign(j): M e_j = sign(j) e_perm(j). Not symmetric."""
    M = np.zeros((d, d))
    perm = [(mult * j + add) % d for j in range(d)]
    for j in range(d):
        M[perm[j], j] = sign_rule(j)
    return M, perm


@pytest.mark.parametrize("B", [1, 2, 3])
def test_codes_and_signs_under_signed_permutations(B):
    d, L, j = 32, 1 << B, 7
    R, pr = _signed_permutation(d, 5, 3, lambda i: -1.0 if i % 3 == 0 else 1.0)
    S, ps = _signed_permutation(d, 3, 1, lambda i: -1.0 if i % 4 == 1 else 1.0)
    assert not np.allclose(R, R.T) and not np.allclose(S, S.T)
    q = tq.make_quantizer(d, B, True, R, S)
    x = np.zeros(d)
    x[j] = 5.0
    c = tq.quantize(x[None], q)
    # x~ = R e_j = sign(j) e_perm(j): that coordinate passes every boundary
    # (or none, for a negative sign); every other coordinate is exactly 0,
    # on the middle boundary, and goes up to L/2
    hot = pr[j]
    sj = -1.0 if j % 3 == 0 else 1.0
    want_idx = np.full(d, L // 2)
    want_idx[hot] = L - 1 if sj > 0 else 0
    assert np.array_equal(c.idx[0], want_idx)
    cen = q.centroids
    r = -cen[want_idx].astype(np.float64)
    r[hot] += sj
    assert c.rho[0] == pytest.approx(math.sqrt(np.sum(r * r)), rel=1e-14)
    # (S r~)_{perm_s(i)} = sign_s(i) r~_i, so the sign at perm_s(i) is
    # [sign_s(i) r~_i >= 0]
    want_z = np.zeros(d, bool)
    for i in range(d):
        si = -1.0 if i % 4 == 1 else 1.0
        want_z[ps[i]] = si * r[i] >= 0
    assert np.array_equal(c.z[0], want_z)
    # the estimator's query side: <y, x^> for y = e_k picks row k of R^T c[idx] etc.
    y = np.zeros((1, d))
    y[0, 11] = 1.0
    xh = 5.0 * (R.T @ (cen[want_idx] + q.gamma * np.float16(c.rho[0]).astype(np.float64) *
                       (S.T @ np.where(want_z, 1.0, -1.0))))
    assert tq.estimate_ip(y, c, q)[0, 0] == pytest.approx(xh[11], rel=1e-12, abs=1e-15)


# --------------------------------------------------------------------------
# constructed vectors that quantise losslessly (rho = 0 up to rounding)
# --------------------------------------------------------------------------

def _lossless_quantizer(d, prod, seed):
    # B = 2 with centroids (-3a, -a, a, 3a), a = 1/sqrt(96 d / 32): a code
    # vector with d/4 entries of magnitude 3a and 3d/4 of magnitude a has
    # unit norm, so x = n R^T c[idx] rotates back onto c[idx] exactly
    a = 1.0 / math.sqrt(3.0 * d)
    cen = np.array([-3 * a, -a, a, 3 * a])
    thr = 0.5 * (cen[:-1] + cen[1:])
    R = synth.haar_orthogonal(d, seed, dtype=np.float64)
    S = synth.gaussian_matrix(d, d, seed, dtype=np.float64) if prod else None
    return tq.make_quantizer(d, 2, prod, R, S, cen, thr)


def _lossless_vectors(q, N, seed):
    g = synth.rng(seed, 31)
    d = q.d
    idx = np.empty((N, d), np.int64)
    for i in range(N):
        big = g.permutation(d)[: d // 4]
        sgn = g.integers(0, 2, d)
        row = np.where(sgn == 1, 2, 1)                  # magnitude a
        row[big] = np.where(sgn[big] == 1, 3, 0)         # magnitude 3a
        idx[i] = row
    norms = g.choice([0.5, 1.75, 3.0, 7.0, 12.25], size=N)   # exact halves
    return norms[:, None] * (q.centroids[idx] @ q.R), idx


def test_constructed_keys_have_zero_residual_and_exact_inner_products():
    d = 64
    q = _lossless_quantizer(d, True, 3)
    x, idx = _lossless_vectors(q, 40, 1)
    c = tq.quantize(x, q)
    assert np.array_equal(c.idx, idx)
    assert np.all(c.rho < 1e-14) and np.all(c.rho16 == 0)
    y = synth.rng(2, 0).standard_normal((9, d))
    np.testing.assert_allclose(tq.estimate_ip(y, c, q), y @ x.T, rtol=0, atol=1e-12 * np.abs(y @ x.T).max())


def test_decode_on_lossless_cache_equals_textbook_attention():
    B, Hq, Hkv, T, d = 2, 8, 2, 33, 64
    qk = _lossless_quantizer(d, True, 5)
    qv = _lossless_quantizer(d, False, 6)
    K, _ = _lossless_vectors(qk, B * Hkv * T, 7)
    V, _ = _lossless_vectors(qv, B * Hkv * T, 8)
    K = K.reshape(B, Hkv, T, d)
    V = V.reshape(B, Hkv, T, d)
    qry = synth.rng(9, 0).standard_normal((B, Hq, d))
    lens = [T, 17]
    out, sc = tq.decode_attention(qry, [tq.Group(0, qk, tq.quantize(K, qk))], [tq.Group(0, qv, tq.quantize(V, qv))],
                                  Hkv, seq_lens=lens)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            s = K[b, g, :lens[b]] @ qry[b, h]
            np.testing.assert_allclose(sc[b, h, :lens[b]], s, rtol=0, atol=1e-12 * np.abs(s).max())
            p = softmax(s / math.sqrt(d))
            o = p @ V[b, g, :lens[b]]
            assert np.linalg.norm(out[b, h] - o) <= 1e-12 * np.linalg.norm(o)


# --------------------------------------------------------------------------
# distortion table of section 5.5 (cosine similarity and per-element MSE)
# --------------------------------------------------------------------------

@pytest.mark.slow
def test_distortion_matches_the_section_5_5_table():
    # b-bit TurboQuant_prod = (b - 1) codebook bits + 1 sign bit. After a Haar
    # rotation the distortion of a vector does not depend on its direction,
    # so random unit vectors stand in for the post's Llama-3.1-8B keys.
    d, N, seeds = 128, 1500, 4
    table_cos = {4: 0.9749, 3: 0.9225, 2: 0.8031}
    table_mse = {4: 0.274, 3: 0.917, 2: 2.890}
    cos, mse = {}, {}
    for b in (4, 3, 2):
        cs, ms = [], []
        cen, thr = tq.symmetric_codebook(d, b - 1)
        for s in range(seeds):
            q = tq.make_quantizer(d, b - 1, True, synth.haar_orthogonal(d, 100 + s, dtype=np.float64),
                                  synth.gaussian_matrix(d, d, 100 + s, dtype=np.float64), cen, thr)
            x = synth.unit_gaussian(N, d, 200 + s).astype(np.float64)
            xh = tq.dequantize(tq.quantize(x, q), q)
            cs.append(np.sum(x * xh, axis=1) / np.linalg.norm(xh, axis=1))
            ms.append(np.sum((x - xh) ** 2, axis=1) / d)
        cos[b], mse[b] = float(np.mean(cs)), float(np.mean(ms))
        assert abs(cos[b] - table_cos[b]) < 0.004, (b, cos[b])
    # per-element MSE scales with |x|^2: the ratios between widths do not
    # depend on the keys' norms (within 4 % of the table's)
    assert abs(mse[3] / mse[4] - table_mse[3] / table_mse[4]) < 0.04 * table_mse[3] / table_mse[4]
    assert abs(mse[2] / mse[3] - table_mse[2] / table_mse[3]) < 0.04 * table_mse[2] / table_mse[3]
    # the closed form (pi/2 - 1/d) D_B |x|^2 / d, with |x|^2 fitted to the
    # table's 4-bit row, predicts the 3- and 2-bit rows within 5 %
    D = {b: cb.lloyd_max(d, b - 1)[2] for b in (4, 3, 2)}
    for b in (4, 3, 2):
        assert abs(mse[b] - (math.pi / 2 - 1 / d) * D[b] / d) < 0.03 * mse[b]
    n2 = table_mse[4] * d / ((math.pi / 2 - 1 / d) * D[4])
    for b in (3, 2):
        pred = (math.pi / 2 - 1 / d) * D[b] * n2 / d
        assert abs(pred - table_mse[b]) < 0.05 * table_mse[b], (b, pred)


# --------------------------------------------------------------------------
# exact top-k and recall (the search workload's reference)
# --------------------------------------------------------------------------

def test_exact_topk_by_brute_force():
    g = synth.rng(4, 0)
    db = g.standard_normal((57, 16))
    db[30] = db[3]           # an exact tie: index 3 must come first
    qs = g.standard_normal((4, 16))
    qs[0] = db[3]            # query equal to the tied row
    idx, sc = tq.exact_topk(qs, db, 6)
    for i in range(4):
        s = [float(np.dot(qs[i], db[j])) for j in range(57)]
        rem, want = list(range(57)), []
        for _ in range(6):
            best = rem[0]
            for j in rem[1:]:
                if s[j] > s[best]:
                    best = j
            want.append(best)
            rem.remove(best)
        assert list(idx[i]) == want
        np.testing.assert_allclose(sc[i], [s[j] for j in want], rtol=1e-15)
    assert list(idx[0][:2]) == [3, 30]


def test_recall_at_k_by_hand():
    truth = np.array([[1, 2, 3, 4], [5, 6, 7, 8], [9, 10, 11, 12]])
    found = np.array([[4, 3, 2, 1], [5, 0, 0, 0], [13, 14, 15, 16]])
    # per query 4/4, 1/4, 0/4 -> mean 5/12
    assert tq.recall_at_k(found, truth) == pytest.approx(5 / 12)
    # longer found lists count only their first k entries
    assert tq.recall_at_k(np.array([[7, 1, 2, 3, 4]]), truth[:1]) == pytest.approx(3 / 4)
