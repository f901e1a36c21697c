"""Pins of the 3-bit value oracle (oracle/values3.py) against facts that do not
come from it: the Lloyd-Max optimality conditions checked by numerical
quadrature (scipy), the two-level closed form, the Hadamard matrix of
scipy.linalg, a hand-worked bit layout, and the codec's distortion on
Gaussian vectors against the quantiser's distortion (PolyKV, section 2B)."""
import math

import numpy as np
import pytest
import scipy.integrate
import scipy.linalg

import synth
from oracle import values3 as V3


def _phi(x):
    return math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)


def _distortion(cent, bnd):
    """E[(X - Q(X))^2] for X ~ N(0, 1) by quadrature over each cell."""
    edges = [-math.inf] + list(bnd) + [math.inf]
    tot = 0.0
    for i, c in enumerate(cent):
        tot += scipy.integrate.quad(lambda x, c=c: (x - c) ** 2 * _phi(x), edges[i], edges[i + 1],
                                    epsabs=1e-14, epsrel=1e-12)[0]
    return tot


def test_two_levels_closed_form():
    """Two levels: the centroids are +-E|X| = +-sqrt(2 / pi), the boundary 0."""
    cent, bnd = V3.lloyd_max_normal(2)
    assert np.allclose(cent, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], rtol=0, atol=1e-14)
    assert np.array_equal(bnd, [0.0])


def test_eight_levels_satisfy_the_optimality_conditions():
    """Every centroid is the N(0, 1) mean of its cell (quadrature), every inner
    boundary the midpoint of its neighbours, the quantiser symmetric, and
    moving any centroid or boundary raises the distortion."""
    cent, bnd = V3.lloyd_max_normal()
    assert cent.shape == (8,) and bnd.shape == (7,)
    assert np.all(np.diff(cent) > 0) and np.all(np.diff(bnd) > 0)
    assert np.array_equal(cent, -cent[::-1]) and bnd[3] == 0.0
    edges = [-math.inf] + list(bnd) + [math.inf]
    for i, c in enumerate(cent):
        m = scipy.integrate.quad(lambda x: x * _phi(x), edges[i], edges[i + 1], epsabs=1e-15, epsrel=1e-13)[0]
        p = scipy.integrate.quad(_phi, edges[i], edges[i + 1], epsabs=1e-15, epsrel=1e-13)[0]
        assert abs(m / p - c) <= 1e-9, (i, m / p, c)
    assert np.allclose(bnd, 0.5 * (cent[:-1] + cent[1:]), rtol=0, atol=1e-15)
    d0 = _distortion(cent, bnd)
    assert 0.03 < d0 < 0.04
    for i in range(8):
        for eps in (1e-3, -1e-3):
            c2 = cent.copy()
            c2[i] += eps
            assert _distortion(c2, bnd) > d0
    for i in range(7):
        for eps in (1e-3, -1e-3):
            b2 = bnd.copy()
            b2[i] += eps
            assert _distortion(cent, b2) > d0


@pytest.mark.parametrize("d", [8, 64, 128])
def test_fwht_is_the_hadamard_matrix(d):
    x = np.random.default_rng(d).standard_normal((5, d))
    h = scipy.linalg.hadamard(d).astype(np.float64)
    assert np.allclose(V3.fwht(x), x @ h.T, rtol=0, atol=1e-12)
    assert np.allclose(V3.fwht(V3.fwht(x)), d * x, rtol=0, atol=1e-11)


def test_fwht_exact_on_bf16_inputs():
    """The butterflies add +-1 multiples of bf16 values: exact in fp64, so any
    summation order gives the same z (the codes do not depend on the order)."""
    v = synth.bf16_to_f32(synth.bf16_bits(np.random.default_rng(1).standard_normal((50, 128)))).astype(np.float64)
    z = V3.fwht(v)
    h = scipy.linalg.hadamard(128).astype(np.float64)
    zz = np.array([[math.fsum(h[j] * row) for j in range(128)] for row in v])
    assert np.array_equal(z, zz)


def test_coordinates_have_unit_mean_square():
    v = synth.bf16_bits(np.random.default_rng(2).standard_normal((7, 64)) * 3.0)
    u = V3.normalized_coords(v)
    assert np.allclose(np.mean(u * u, axis=-1), 1.0, rtol=0, atol=1e-13)
    assert np.array_equal(V3.normalized_coords(np.zeros((2, 8), np.float32)), np.zeros((2, 8)))


def test_codes_count_boundaries_at_or_below():
    _, bnd = V3.lloyd_max_normal()
    u = np.array([-10.0, bnd[0] - 1e-9, bnd[0], 0.0, -0.0, -1e-12, bnd[6], 10.0])
    assert V3.codes_of(u, bnd).tolist() == [0, 0, 1, 4, 4, 3, 7, 7]


def test_plane_layout_by_hand():
    """Codes j % 8 over d = 8: plane 0 holds the low bits 0,1,0,1,... (byte
    0b10101010), plane 1 0,0,1,1,... (0b11001100), plane 2 0b11110000."""
    codes = np.arange(8, dtype=np.uint8)[None]
    assert V3.pack_planes(codes).tolist() == [[0xAA, 0xCC, 0xF0]]
    rnd = np.random.default_rng(3).integers(0, 8, (4, 128)).astype(np.uint8)
    assert np.array_equal(V3.unpack_planes(V3.pack_planes(rnd), 128), rnd)


def test_codec_distortion_matches_the_quantiser():
    """For Gaussian vectors the rotated coordinates are close to N(0, 1), so
    the relative squared error of decode(encode(v)) is the quantiser's
    distortion (quadrature); a wrong decode scale or a missing inverse
    transform misses it by far."""
    cent, bnd = V3.lloyd_max_normal()
    d0 = _distortion(cent, bnd)
    v = np.random.default_rng(4).standard_normal((20000, 128)).astype(np.float32)
    packed, s = V3.quantize_values(v)
    assert packed.shape == (20000, 48) and s.dtype == np.float32
    vh = V3.dequantize_values(packed, s, 128)
    rel = np.sum((vh - v) ** 2) / np.sum(v.astype(np.float64) ** 2)
    assert abs(rel - d0) < 0.002, (rel, d0)


def test_scale_is_norm_over_d():
    v = np.zeros((1, 64), np.float32)
    v[0, 5] = 3.0
    v[0, 9] = -4.0
    _, s = V3.quantize_values(v)
    assert s[0] == np.float32(5.0 / 64)
