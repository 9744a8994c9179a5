"""Pins of the oracle's quantiser, estimator, layouts, decode and search (CPU).

Sources: riverfrot "TurboQuant" post sections 2.2-2.4 and 4.1-4.3;
uiyeonassociation post (two-stage method, 2/pi shrinkage, unbiased
estimator, vector search). Every pin is something the pages or the
mathematics fix independently of the oracle's own code path.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import synth
from oracle import tq
from oracle import codebook as cb

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def quantizer(d, B, prod, seed=0, R=None, S=None):
    if R is None:
        R = synth.haar_orthogonal(d, seed)
    if prod and S is None:
        S = synth.gaussian_matrix(d, d, seed)
    return tq.make_quantizer(d, B, prod, R, S)


# --------------------------------------------------------------------------
# half-precision storage and the page's worked example
# --------------------------------------------------------------------------

def test_half_rounding_is_nearest_even():
    # numpy's float64 -> float16 must round to nearest, ties to even (the
    # stored-norm convention); check against brackets built from float16 ulps.
    g = synth.rng(3, 0)
    vals = np.concatenate([g.lognormal(0, 2, 20000), [1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0]])
    h = vals.astype(np.float16)
    lo = np.where(h.astype(np.float64) <= vals, h, np.nextafter(h, np.float16(0)))
    hi = np.nextafter(lo, np.float16(np.inf))
    dlo = vals - lo.astype(np.float64)
    dhi = hi.astype(np.float64) - vals
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi,
                    np.where((lo.view(np.uint16) & 1) == 0, lo, hi)))
    assert np.array_equal(h.view(np.uint16), want.view(np.uint16))
    # the four exact ties: 1+2^-11 -> 1, 1+3*2^-11 -> 1+2^-9, 2049 -> 2048, 2051 -> 2052
    assert list(h[-4:].astype(np.float64)) == [1.0, 1.0 + 2.0 ** -9, 2048.0, 2052.0]


def test_page_worked_example_3bit():
    ex = json.load(open(os.path.join(GOLD, "page_3bit_worked_example.json")))
    c = np.array(ex["centroids"])
    t = 0.5 * (c[:-1] + c[1:])
    R = np.eye(1)
    q = tq.make_quantizer(1, 3, False, R, centroids=c, thresholds=t)
    # a one-dimensional "vector" would be normalised to +-1, so apply the
    # scalar step directly: count boundaries passed (ties go up)
    idx = int(np.sum(ex["input"] >= q.thresholds))
    assert idx + 1 == ex["expected_interval_1based"]
    assert q.centroids[idx] == pytest.approx(ex["expected_value"])


# --------------------------------------------------------------------------
# quantiser special cases
# --------------------------------------------------------------------------

@pytest.mark.parametrize("B", [1, 2, 3])
def test_basis_vector_codes_by_hand(B):
    # R = S = I (valid orthogonal / projection matrices): x = 5 e_j rotates to
    # e_j. Coordinate j passes every boundary (code L-1); all others are
    # exactly 0, on the middle boundary 0, so they go up to code L/2.
    d, j = 32, 7
    L = 1 << B
    q = tq.make_quantizer(d, B, True, np.eye(d), np.eye(d))
    x = np.zeros(d)
    x[j] = 5.0
    c = tq.quantize(x[None], q)
    want = np.full(d, L // 2)
    want[j] = L - 1
    assert np.array_equal(c.idx[0], want)
    assert c.n[0] == 5.0
    cen = q.centroids
    rho = math.sqrt((1 - cen[L - 1]) ** 2 + (d - 1) * cen[L // 2] ** 2)
    assert c.rho[0] == pytest.approx(rho, rel=1e-14)
    # with S = I the signs are the signs of the residual: + at j (1 > c_max),
    # - elsewhere (0 - c_{L/2} < 0 since c_{L/2} > 0)
    wz = np.zeros(d, bool)
    wz[j] = True
    assert np.array_equal(c.z[0], wz)


def test_zero_vector_convention():
    q = quantizer(64, 2, True)
    c = tq.quantize(np.zeros((1, 64)), q)
    assert c.n[0] == 0 and c.rho[0] == 0
    assert np.all(c.idx == 2) and np.all(c.z)
    assert np.all(tq.estimate_ip(np.ones((1, 64)), c, q) == 0)


def test_codes_are_nearest_centroid():
    d = 128
    q = quantizer(d, 3, True)
    x = synth.unit_gaussian(500, d, 1)
    c = tq.quantize(x, q)
    u = c.urot
    near = np.argmin(np.abs(u[:, :, None] - q.centroids[None, None, :]), axis=2)
    # away from the midpoints the threshold count and argmin agree
    gap = np.min(np.abs(u[:, :, None] - q.thresholds[None, None, :]), axis=2)
    ok = gap > 1e-12
    assert np.array_equal(c.idx[ok], near[ok])
    # rotation preserves the norm of the unit direction
    np.testing.assert_allclose(np.linalg.norm(u, axis=1), 1.0, atol=1e-6)


def test_reconstruction_equals_rotated_domain_estimator():
    # <y, x^> with x^ rebuilt in the original domain (R^T, S^T) must equal
    # the estimator evaluated in the rotated domain (R y, S R y): catches a
    # transposed R or S anywhere.
    d = 96
    for prod in (True, False):
        q = quantizer(d, 2, prod, seed=5)
        x = synth.unit_gaussian(40, d, 2) * 3.0
        y = synth.unit_gaussian(7, d, 3)
        c = tq.quantize(x, q)
        xh = tq.dequantize(c, q)
        np.testing.assert_allclose(y @ xh.T, tq.estimate_ip(y, c, q), rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------------
# statistical pins (spec: mean over 10^4 seeds within 3 sigma)
# --------------------------------------------------------------------------

def _pair(d, ip, seed):
    g = synth.rng(seed, 9)
    x = g.standard_normal(d)
    x /= np.linalg.norm(x)
    w = g.standard_normal(d)
    w -= (w @ x) * x
    w /= np.linalg.norm(w)
    y = ip * x + math.sqrt(1 - ip * ip) * w
    return x, y


@pytest.mark.slow
def test_prod_estimator_unbiased_over_1e4_seeds():
    d, B, ip = 128, 3, 0.6
    x, y = _pair(d, ip, 0)
    cen, thr = tq.symmetric_codebook(d, B)
    est = np.empty(10000)
    for s in range(10000):
        q = tq.make_quantizer(d, B, True, synth.haar_orthogonal(d, s, dtype=np.float64),
                              synth.gaussian_matrix(d, d, s, dtype=np.float64), cen, thr)
        est[s] = tq.estimate_ip(y[None], tq.quantize(x[None], q), q)[0, 0]
    se = est.std(ddof=1) / math.sqrt(len(est))
    assert abs(est.mean() - ip) < 3 * se, (est.mean(), se)


@pytest.mark.slow
def test_mse_one_bit_shrinks_by_one_minus_D():
    # E_R <y, x^_mse> = (1 - D_B) <x, y> for unit x; at B = 1, 1 - D_1 = d c^2,
    # the finite-d form of the 2/pi factor (uiyeonassociation post; riverfrot 4.3).
    d, ip = 128, 0.6
    x, y = _pair(d, ip, 1)
    cen, thr = tq.symmetric_codebook(d, 1)
    est = np.empty(4000)
    for s in range(4000):
        q = tq.make_quantizer(d, 1, False, synth.haar_orthogonal(d, s, dtype=np.float64), None, cen, thr)
        est[s] = tq.estimate_ip(y[None], tq.quantize(x[None], q), q)[0, 0]
    factor = d * cb.one_bit_centroid(d) ** 2
    se = est.std(ddof=1) / math.sqrt(len(est))
    assert abs(est.mean() - factor * ip) < 3 * se
    assert abs(est.mean() - ip) > 20 * se       # visibly biased without QJL
    assert abs(factor - 2 / math.pi) < 3e-3


@pytest.mark.slow
def test_prod_reconstruction_norm_closed_form():
    # E|x^|^2 = 1 + D_B (pi/2 - 1/d) for unit x (QJL adds gamma^2 rho^2 |S^T z|^2
    # with E|S^T z|^2 = d^2 + d(d-1)(2/pi) - this pins gamma = sqrt(pi/2)/d).
    d, B = 128, 2
    _, _, D, _ = cb.lloyd_max(d, B)
    x, _ = _pair(d, 0.0, 2)
    cen, thr = tq.symmetric_codebook(d, B)
    sq = np.empty(3000)
    for s in range(3000):
        q = tq.make_quantizer(d, B, True, synth.haar_orthogonal(d, s, dtype=np.float64),
                              synth.gaussian_matrix(d, d, s, dtype=np.float64), cen, thr)
        c = tq.quantize(x[None], q)
        sq[s] = np.sum(tq.dequantize(c, q) ** 2)
    want = 1 + D * (math.pi / 2 - 1 / d)
    se = sq.std(ddof=1) / math.sqrt(len(sq))
    assert abs(sq.mean() - want) < 3.5 * se + 2e-3   # + fp16 storage of rho


# --------------------------------------------------------------------------
# packed layouts
# --------------------------------------------------------------------------

def test_keys_layout_hand_fixture():
    # d = 32, B = 1, PROD, one vector: word [tile 0][g 0][t 0][p] holds
    # coordinate i at bit i. Codes 1 at coordinates 0 and 31, signs at 1.
    idx = np.zeros((1, 32), np.uint8)
    idx[0, [0, 31]] = 1
    z = np.zeros((1, 32), bool)
    z[0, 1] = True
    w = tq.pack(idx, z, 1, "keys")
    assert w.shape == (16 * 2,)                       # 16-vector tile x 2 planes
    assert w[0] == 0x80000001 and w[1] == 0x00000002
    assert np.all(w[2:] == 0)                         # vectors 1..15 are padding


def test_values_layout_hand_fixture():
    # d = 32, B = 2, MSE: words [tile][j][p]; tiles come in blocks of two
    # covering 64 vectors, vector 64 B + t in tile 2 B + (t // 8) % 2 at bit
    # 16 (t % 2) + 4 (t // 16) + (t % 8) // 2:
    #   vector 0  -> tile 0, bit 0;      vector 9  -> tile 1, bit 16;
    #   vector 31 -> tile 1, bit 23;     vector 63 -> tile 1, bit 31;
    #   vector 50 -> tile 0, bit 13;     vector 64 -> tile 2, bit 0 (the next block).
    idx = np.zeros((65, 32), np.uint8)
    idx[0, 5] = 3          # both planes set at coordinate 5 of vector 0
    idx[64, 0] = 2         # plane 1 set at coordinate 0 of vector 64
    idx[9, 2] = 1          # plane 0 at coordinate 2 of vector 9
    idx[31, 2] = 1         # plane 0 at coordinate 2 of vector 31
    idx[63, 2] = 1         # plane 0 at coordinate 2 of vector 63
    idx[50, 7] = 1         # plane 0 at coordinate 7 of vector 50
    w = tq.pack(idx, None, 2, "values")
    assert w.shape == (4 * 32 * 2,)                   # two blocks of two tiles, 32 coordinates, 2 planes
    w = w.reshape(4, 32, 2)
    assert w[0, 5, 0] == 1 and w[0, 5, 1] == 1
    assert w[2, 0, 0] == 0 and w[2, 0, 1] == 1
    assert w[1, 2, 0] == (1 << 16) | (1 << 23) | (1 << 31) and w[1, 2, 1] == 0
    assert w[0, 7, 0] == 1 << 13
    assert int(w.astype(np.uint64).sum()) == 1 + 1 + 1 + (1 << 16) + (1 << 23) + (1 << 31) + (1 << 13)


@pytest.mark.parametrize("layout", ["keys", "values"])
@pytest.mark.parametrize("d,B,prod,N", [(32, 1, True, 1), (96, 2, False, 45), (128, 3, True, 67), (64, 4, True, 31)])
def test_pack_roundtrip(layout, d, B, prod, N):
    g = synth.rng(7, 0)
    idx = g.integers(0, 1 << B, size=(N, d)).astype(np.uint8)
    z = g.integers(0, 2, size=(N, d)).astype(bool) if prod else None
    w = tq.pack(idx, z, B, layout)
    assert w.size == tq.packed_words(d, B, prod, N, layout)
    i2, z2 = tq.unpack(w, N, d, B, prod, layout)
    assert np.array_equal(i2, idx)
    if prod:
        assert np.array_equal(z2, z)


# --------------------------------------------------------------------------
# decode attention and search
# --------------------------------------------------------------------------

def _kv(B, Hkv, T, d, kB, vB, seed=0):
    qk = quantizer(d, kB, True, seed=seed)
    qv = tq.make_quantizer(d, vB, False, synth.haar_orthogonal(d, seed, synth.STREAM_R_V))
    K = synth.rng(seed, 20).standard_normal((B, Hkv, T, d))
    V = synth.rng(seed, 21).standard_normal((B, Hkv, T, d))
    return qk, qv, K, V, tq.quantize(K, qk), tq.quantize(V, qv)


def test_decode_matches_textbook_attention_on_reconstructions():
    B, Hq, Hkv, T, d = 2, 8, 2, 37, 64
    qk, qv, K, V, ck, cv = _kv(B, Hkv, T, d, 3, 2)
    qry = synth.rng(0, 22).standard_normal((B, Hq, d))
    out, sc = tq.decode_attention(qry, [tq.Group(0, qk, ck)], [tq.Group(0, qv, cv)], Hkv, seq_lens=[T, 20])
    Kh, Vh = tq.dequantize(ck, qk), tq.dequantize(cv, qv)
    for b, L in ((0, T), (1, 20)):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            s = Kh[b, g, :L] @ qry[b, h]
            np.testing.assert_allclose(sc[b, h, :L], s, rtol=1e-10, atol=1e-10)
            p = softmax(s / math.sqrt(d))
            np.testing.assert_allclose(out[b, h], p @ Vh[b, g, :L], rtol=1e-10, atol=1e-12)


def test_decode_single_token_and_identical_keys():
    d = 32
    qk, qv, K, V, ck, cv = _kv(1, 1, 5, d, 2, 2, seed=3)
    qry = synth.rng(1, 0).standard_normal((1, 4, d))
    out1, _ = tq.decode_attention(qry, [tq.Group(0, qk, ck)], [tq.Group(0, qv, cv)], 1, seq_lens=[1])
    vh = tq.dequantize(cv, qv)
    for h in range(4):
        np.testing.assert_allclose(out1[0, h], vh[0, 0, 0], rtol=1e-12)
    Ksame = np.repeat(K[:, :, :1], 5, axis=2)
    cks = tq.quantize(Ksame, qk)
    out, _ = tq.decode_attention(qry, [tq.Group(0, qk, cks)], [tq.Group(0, qv, cv)], 1)
    for h in range(4):
        np.testing.assert_allclose(out[0, h], vh[0, 0].mean(axis=0), rtol=1e-10, atol=1e-12)


def test_decode_channel_groups_sum():
    # Two channel groups: the score is the sum of the per-group estimates and
    # each value group fills its own channel range.
    B, Hq, Hkv, T = 1, 4, 1, 9
    qa = quantizer(32, 2, True, seed=1)
    qb = quantizer(96, 1, True, seed=2)
    va = tq.make_quantizer(32, 2, False, synth.haar_orthogonal(32, 3))
    vb = tq.make_quantizer(96, 1, False, synth.haar_orthogonal(96, 4))
    K = synth.rng(5, 0).standard_normal((B, Hkv, T, 128))
    V = synth.rng(5, 1).standard_normal((B, Hkv, T, 128))
    qry = synth.rng(5, 2).standard_normal((B, Hq, 128))
    kg = [tq.Group(0, qa, tq.quantize(K[..., :32], qa)), tq.Group(32, qb, tq.quantize(K[..., 32:], qb))]
    vg = [tq.Group(0, va, tq.quantize(V[..., :32], va)), tq.Group(32, vb, tq.quantize(V[..., 32:], vb))]
    out, sc = tq.decode_attention(qry, kg, vg, Hkv)
    kh = np.concatenate([tq.dequantize(g.codes, g.q) for g in kg], axis=-1)
    vh = np.concatenate([tq.dequantize(g.codes, g.q) for g in vg], axis=-1)
    for h in range(Hq):
        s = kh[0, 0] @ qry[0, h]
        np.testing.assert_allclose(sc[0, h], s, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(out[0, h], softmax(s / math.sqrt(128)) @ vh[0, 0], rtol=1e-10, atol=1e-12)


def test_search_topk_matches_selection_by_hand():
    d, N, Q, k = 64, 300, 5, 7
    q = quantizer(d, 3, True, seed=4)
    db = synth.unit_gaussian(N, d, 6)
    c = tq.quantize(db, q)
    ys = synth.unit_gaussian(Q, d, 7)
    idx, sc = tq.search_topk(ys, c, q, k, chunk=64)
    full = tq.estimate_ip(ys, c, q)
    for i in range(Q):
        # repeated arg-max selection, lowest index first on ties
        rem = list(range(N))
        want = []
        for _ in range(k):
            best = rem[0]
            for j in rem[1:]:
                if full[i, j] > full[i, best]:
                    best = j
            want.append(best)
            rem.remove(best)
        assert list(idx[i]) == want
        np.testing.assert_allclose(sc[i], full[i, want], rtol=1e-12)


def test_search_tie_breaks_to_lower_index():
    d = 32
    q = quantizer(d, 2, True, seed=1)
    db = np.repeat(synth.unit_gaussian(3, d, 1), 4, axis=0)   # every row four times
    c = tq.quantize(db, q)
    idx, sc = tq.search_topk(synth.unit_gaussian(1, d, 2), c, q, 12, chunk=5)
    for a, b in zip(idx[0][:-1], idx[0][1:]):
        if sc[0][list(idx[0]).index(a)] == sc[0][list(idx[0]).index(b)]:
            assert a < b


# --------------------------------------------------------------------------
# KV size formula (riverfrot introduction and section 2.4)
# --------------------------------------------------------------------------

def test_kv_size_examples():
    ex = json.load(open(os.path.join(GOLD, "kv_size_examples.json")))["examples"]
    a, b, c = ex
    v = tq.kv_cache_bytes(a["layers"], a["kv_heads"], a["head_dim"], a["seq_len"], a["bytes"])
    assert v == a["expected_bytes"] and v == a["expected_mib"] * 2 ** 20
    v = tq.kv_cache_bytes(b["layers"], b["kv_heads"], b["head_dim"], b["seq_len"], b["bytes"])
    assert v == b["expected_bytes"] and v == b["expected_gib"] * 2 ** 30
    v = c["requests"] * tq.kv_cache_bytes(c["layers"], c["kv_heads"], c["head_dim"], c["seq_len"], c["bytes"])
    assert abs(v / 1e9 - c["approx_total_gb"]) / c["approx_total_gb"] < 0.1


def test_compressed_size_of_the_long_context_workload():
    # 2.5 bits per channel: 32 outlier channels at 3 bits (2 + 1 QJL for keys),
    # 96 at 2 bits (1 + 1); values MSE-only 3 / 2 bits; half norms per group.
    per = tq.compressed_kv_bytes(1, 1, 1, [(32, 2, True), (96, 1, True)], [(32, 3, False), (96, 2, False)])
    assert per == 84
    # ratio to bf16 K and V (2 x 128 x 2 bytes)
    assert 512 / per > 6.0


# --------------------------------------------------------------------------
# key/value bit allocation (riverfrot section 4.5)
# --------------------------------------------------------------------------

def test_kv_bit_allocation_follows_the_norm_ratio_table():
    # the section's bands: below 10x uniform 3-bit, 10-60x asymmetric
    # 4-bit keys / 2-bit values, above 100x mixed precision
    assert tq.kv_bit_allocation(5.0, 1.0) == (tq.KV_UNIFORM, 3, 3)
    assert tq.kv_bit_allocation(9.99, 1.0)[0] == tq.KV_UNIFORM
    assert tq.kv_bit_allocation(10.0, 1.0) == (tq.KV_ASYMMETRIC, 4, 2)
    assert tq.kv_bit_allocation(37.0, 1.0) == (tq.KV_ASYMMETRIC, 4, 2)
    assert tq.kv_bit_allocation(60.0, 1.0)[0] == tq.KV_ASYMMETRIC
    assert tq.kv_bit_allocation(80.0, 1.0)[0] == tq.KV_ASYMMETRIC  # the open band, read as asymmetric
    assert tq.kv_bit_allocation(100.5, 1.0)[0] == tq.KV_MIXED
    # the section's Qwen measurement: key norms 172-778 against value norms
    # 2-4 put the typical ratio (~160x at the middles) in the mixed band
    assert tq.kv_bit_allocation((172 + 778) / 2, (2 + 4) / 2)[0] == tq.KV_MIXED
    # and its "~37,000x" sensitivity is the squared ratio 778 / 4
    assert abs(tq.kv_norm_sensitivity(778, 4) - 37000) / 37000 < 0.03
    # the ratio is what matters, not the scale
    assert tq.kv_bit_allocation(500.0, 50.0) == tq.kv_bit_allocation(10.0, 1.0)
    for bad in [(0.0, 1.0), (1.0, 0.0), (-1.0, 1.0), (float("inf"), 1.0), (float("nan"), 1.0)]:
        with pytest.raises(ValueError):
            tq.kv_bit_allocation(*bad)
