"""Pins of the oracle's codebook against closed forms and brute force (CPU).

Each check is independent of the Lloyd iteration it tests: closed forms
derived from the density, a dynamic-programming global optimum, quadrature
moments, and sampling of Haar-rotated unit vectors (riverfrot "TurboQuant"
post, sections 4.1, 4.2 and 4.4).
"""
import math

import numpy as np
import pytest
from scipy import stats

import synth
from oracle import codebook as cb


@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_d3_is_uniform_quantiser(B):
    # d = 3: (1-x^2)^0 -> uniform density on [-1, 1]; the optimal L-level
    # quantiser has equal cells, centroids -1 + (2i+1)/L, MSE (2/L)^2/12 per
    # coordinate, i.e. D = 3 * 1/(3 L^2) = 4^-B for the whole vector.
    L = 1 << B
    c, t, D, _ = cb.lloyd_max(3, B)
    np.testing.assert_allclose(c, -1 + (2 * np.arange(L) + 1) / L, atol=1e-9)
    assert abs(D - 4.0 ** -B) < 1e-9


@pytest.mark.parametrize("d", [4, 16, 128, 1536])
def test_one_bit_levels_are_mean_abs(d):
    # 1 bit: cells split at 0, centroid = +-E|X|, E|X| = Gamma(d/2)/(sqrt(pi) Gamma((d+1)/2)).
    c, t, D, _ = cb.lloyd_max(d, 1)
    e = cb.one_bit_centroid(d)
    np.testing.assert_allclose(c, [-e, e], rtol=1e-12)
    assert abs(t[0]) < 1e-15
    # D = 1 - d E|X|^2 (the centroid captures d c^2 of the unit energy)
    assert abs(D - (1 - d * e * e)) < 1e-9


def test_one_bit_energy_tends_to_two_over_pi():
    # d c^2 is the 1-bit inner-product shrinkage factor; it tends to 2/pi
    # (uiyeonassociation post: 1-bit MSE quantisation shrinks inner products
    # by 2/pi; riverfrot section 4.3).
    for d, tol in [(10 ** 4, 1e-4), (10 ** 6, 1e-6)]:
        e = cb.one_bit_centroid(d)
        assert abs(d * e * e - 2 / math.pi) < tol


@pytest.mark.parametrize("d,B", [(8, 2), (16, 3), (64, 2)])
def test_matches_global_optimum_by_dynamic_programming(d, B):
    L = 1 << B
    c, _, _, _ = cb.lloyd_max(d, B)
    bf = cb.brute_force_quantizer(d, L, grid=2000)
    # grid cell width 1e-3: centroids agree to a fraction of it
    np.testing.assert_allclose(c, bf, atol=1.5e-3)


@pytest.mark.parametrize("d", [32, 96, 128, 1536])
@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_symmetry_and_distortion_bounds(d, B):
    c, t, D, _ = cb.lloyd_max(d, B)
    np.testing.assert_allclose(c, -c[::-1], atol=1e-14)
    assert np.all(np.diff(c) > 0)
    # riverfrot section 4.4: lower bound 4^-b, TurboQuant within about 2.7x of it
    assert 4.0 ** -B <= D <= 2.7 * 4.0 ** -B


@pytest.mark.parametrize("d", [3, 16, 128, 1536])
def test_density_moments(d):
    # integral 1, variance 1/d (std 1/sqrt(128) = 0.0884 at d = 128, the value
    # riverfrot section 5.3 quotes as theory), kurtosis 3d/(d+2) (-> 3, the
    # Gaussian value the post compares against).
    xs, ws = np.polynomial.legendre.leggauss(400)
    f = cb.pdf(xs, d)
    m0 = np.sum(ws * f)
    m2 = np.sum(ws * xs ** 2 * f)
    m4 = np.sum(ws * xs ** 4 * f)
    assert abs(m0 - 1) < 1e-10
    assert abs(m2 - 1 / d) < 1e-10 / d
    assert abs(m4 / m2 ** 2 - 3 * d / (d + 2)) < 1e-8
    if d == 128:
        assert abs(math.sqrt(m2) - 0.0884) < 1e-4


def test_haar_rotated_coordinate_follows_marginal():
    # A Haar rotation of a fixed unit vector is uniform on the sphere, so any
    # coordinate of R e_1 (column 1 of R) follows f_d (section 4.1).
    d, n = 16, 3000
    vals = np.array([synth.haar_orthogonal(d, seed, dtype=np.float64)[3, 0] for seed in range(n)])
    ks = stats.kstest(vals, lambda x: cb.cdf(x, d))
    assert ks.pvalue > 1e-3
    kurt = np.mean(vals ** 4) / np.mean(vals ** 2) ** 2
    assert abs(kurt - 3 * d / (d + 2)) < 0.25


def test_haar_is_orthogonal():
    R32 = synth.haar_orthogonal(128, 0)
    assert R32.dtype == np.float32
    err = np.abs(R32.astype(np.float64).T @ R32.astype(np.float64) - np.eye(128)).max()
    assert err <= 1e-6
    R64 = synth.haar_orthogonal(128, 0, dtype=np.float64)
    assert np.abs(R64.T @ R64 - np.eye(128)).max() <= 1e-12
