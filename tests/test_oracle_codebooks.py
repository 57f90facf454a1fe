"""Pins of oracle.codebooks against closed forms, textbook tables and library routines."""
import math
import os
import struct

import numpy as np
import pytest
from scipy import integrate, special, stats

from oracle import codebooks as cbk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lloyd_max_gaussian.txt")


def _read_golden():
    rows = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows[(int(parts[0]), parts[1])] = [float(v) for v in parts[2:]]
    return rows


def test_one_bit_closed_form():
    # optimum 1-bit quantizer of N(0,1): +-E|Z| = +-sqrt(2/pi), MSE 1 - 2/pi
    r = cbk.lloyd_max_real(1)
    assert np.allclose(r, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], atol=1e-15)
    c = float(cbk.codebook(1)[1])
    # with the fp16 centroid c: E[(|Z| - c)^2] = 1 - 2c sqrt(2/pi) + c^2
    assert cbk.distortion(1) == pytest.approx(1 - 2 * c * math.sqrt(2 / math.pi) + c * c, abs=1e-15)
    assert cbk.boundaries(1).tolist() == [0.0]


def test_textbook_max_1960():
    g = _read_golden()
    for L in (4, 8, 16):
        b = int(math.log2(L))
        r = cbk.lloyd_max_real(b)
        pos = r[L // 2:]
        # the table gives 4 significant digits (last-digit rounding tolerated)
        assert np.allclose(pos, g[(L, "output")], rtol=3.5e-4, atol=1e-4), L
        bd = 0.5 * (r[:-1] + r[1:])
        assert np.allclose(bd[L // 2 - 1:], g[(L, "boundary")], rtol=3.5e-4, atol=1e-4), L
        assert cbk.mse_of(r, bd) == pytest.approx(g[(L, "mse")][0], rel=1e-3)


@pytest.mark.parametrize("bits", range(1, 9))
def test_centroid_condition_with_scipy(bits):
    # each fp64 centroid is the conditional mean of its cell (scipy's normal distribution)
    r = cbk.lloyd_max_real(bits)
    edges = np.concatenate([[-np.inf], 0.5 * (r[:-1] + r[1:]), [np.inf]])
    for k in range(r.size):
        a, b = edges[k], edges[k + 1]
        if a >= 0:
            mass = stats.norm.sf(a) - stats.norm.sf(b)
        else:
            mass = stats.norm.cdf(b) - stats.norm.cdf(a)
        mean = (stats.norm.pdf(a) - stats.norm.pdf(b)) / mass
        assert mean == pytest.approx(r[k], abs=5e-13), (bits, k)


@pytest.mark.parametrize("bits", range(1, 9))
def test_codebook_shape_symmetry_monotone(bits):
    cb = cbk.codebook(bits).astype(np.float64)
    bd = cbk.boundaries(bits).astype(np.float64)
    assert cb.size == 2 ** bits and bd.size == 2 ** bits - 1
    assert np.all(np.diff(cb) > 0) and np.all(np.diff(bd) > 0)
    assert np.array_equal(cb, -cb[::-1])
    assert np.array_equal(bd, -bd[::-1])
    assert bd[bd.size // 2] == 0.0
    # every centroid lies strictly inside its cell
    assert np.all(cb[:-1] < bd) and np.all(bd < cb[1:])


@pytest.mark.parametrize("bits", range(1, 9))
def test_fp16_rounding_is_unambiguous(bits):
    # distance of every fp64 centroid to the nearest fp16 rounding midpoint is far above the
    # ~1e-13 solver accuracy, so any accurate implementation rounds to the same fp16 codebook
    r = cbk.lloyd_max_real(bits)
    h = r.astype(np.float16)
    up = np.nextafter(h, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(h, np.float16(-np.inf)).astype(np.float64)
    hv = h.astype(np.float64)
    dist = np.minimum(np.abs(r - 0.5 * (hv + up)), np.abs(r - 0.5 * (hv + dn)))
    assert dist.min() > 1e-9


@pytest.mark.parametrize("bits", range(1, 9))
def test_distortion_matches_quadrature(bits):
    cb = cbk.codebook(bits).astype(np.float64)
    bd = cbk.boundaries(bits).astype(np.float64)
    edges = np.concatenate([[-np.inf], bd, [np.inf]])
    tot = 0.0
    for k in range(cb.size):
        v, _ = integrate.quad(lambda z: (z - cb[k]) ** 2 * stats.norm.pdf(z), edges[k], edges[k + 1],
                              epsabs=1e-15, epsrel=1e-12, limit=200)
        tot += v
    assert cbk.distortion(bits) == pytest.approx(tot, rel=1e-9)


def test_distortion_monte_carlo():
    rng = np.random.default_rng(7)
    z = rng.standard_normal(2_000_000)
    for bits in range(1, 9):
        cb = cbk.codebook(bits).astype(np.float64)
        idx = np.searchsorted(cbk.boundaries(bits).astype(np.float64), z, side="left")
        err = (z - cb[idx]) ** 2
        mc, se = err.mean(), err.std() / math.sqrt(z.size)
        assert abs(mc - cbk.distortion(bits)) < 4.5 * se, bits


def test_delta_strictly_decreasing():
    d = cbk.delta_table()
    assert d.dtype == np.float32 and d.size == 8
    assert np.all(d > 0) and np.all(np.diff(d.astype(np.float64)) < 0)
    assert d[0] == np.float32(1.0 - cbk.distortion(1))
    # delta(0) = 1 - c(1) ~ 2/pi
    assert float(d[0]) == pytest.approx(2 / math.pi, rel=2e-4)


def test_distortion_values_published_scale():
    # Gaussian Lloyd-Max MSE roughly quarters per added bit (about 6 dB/bit)
    c = [cbk.distortion(b) for b in range(0, 9)]
    ratios = [c[b] / c[b + 1] for b in range(1, 8)]
    assert all(3.0 < x < 4.1 for x in ratios)
    assert c[8] == pytest.approx(4.12e-5, rel=5e-3)


def test_nf16_levels_are_gaussian_quantiles():
    lv = cbk.nf16_real()
    z = stats.norm.ppf(31 / 32)
    assert z == pytest.approx(1.8627319, abs=1e-7)
    for k in range(16):
        assert stats.norm.cdf(lv[k] * z) == pytest.approx((k + 0.5) / 16, abs=1e-12)
    h = cbk.nf16_levels()
    assert h[0] == -1 and h[15] == 1
    assert np.array_equal(h, -h[::-1]) and np.all(np.diff(h.astype(np.float64)) > 0)
    bd = cbk.nf16_boundaries()
    assert bd.size == 15 and bd[7] == 0.0
    hv = h.astype(np.float64)
    assert np.all(hv[:-1] < bd) and np.all(bd < hv[1:])


def test_numpy_half_rounding_is_rne():
    # the oracle relies on numpy's fp64->fp32->fp16 casts being round-to-nearest-even;
    # compare with Python's struct 'e' packing (IEEE binary16, round-half-even)
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 4, 20000),
                           np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 2 ** -24 * 1.5, 65504.0, 2 ** -25])])
    vals32 = vals.astype(np.float32)
    for v32, h in zip(vals32, vals32.astype(np.float16)):
        ref = struct.unpack("<e", struct.pack("<e", float(v32)))[0]
        assert float(h) == ref or (math.isnan(ref) and math.isnan(float(h)))
    # erfc-based tail agrees with scipy
    for x in (0.0, 0.5, 2.0, 6.0, -3.0):
        assert cbk.upper_tail(x) == pytest.approx(special.ndtr(-x), rel=1e-14)
