"""Pins of the codec compositions (oracle/codecs.py) and of the decision boundaries
(oracle/codebooks.py boundaries, nf16_boundaries) against brute force, explicit library
matrices and the codebooks' own distortion."""
import numpy as np
import pytest
from scipy import linalg

from oracle import allocation as al
from oracle import codebooks as cbk
from oracle import codecs as cd
from oracle import quantize as qz


def _nearest(u32, levels):
    """Index of the nearest level to every u (brute force over all levels, exact in fp64; the
    first of two equidistant levels, i.e. the lower one)."""
    lv = np.asarray(levels).astype(np.float64)
    d = np.abs(np.asarray(u32, dtype=np.float64)[:, None] - lv[None, :])
    return np.argmin(d, axis=1)


def _grid_away_from(bounds32, lo, hi, n, seed):
    """n fp32 points in [lo, hi] (dense uniform grid plus random points) whose distance to every
    boundary is more than 2 ulp, so the nearest level is unambiguous."""
    rng = np.random.default_rng(seed)
    u = np.concatenate([np.linspace(lo, hi, n), rng.uniform(lo, hi, n)]).astype(np.float32)
    b = np.asarray(bounds32, dtype=np.float64)
    dist = np.min(np.abs(u.astype(np.float64)[:, None] - b[None, :]), axis=1)
    return u[dist > 2.0 * np.spacing(np.abs(u)).astype(np.float64)]


def _sliver_points(cb16, real64):
    """fp32 points between the midpoint of neighbouring fp16 centroids and the midpoint of the
    fp64 centroids they round from, away from both by more than 2 ulp: there the nearest fp16
    centroid and the nearest fp64 centroid disagree, so a boundary taken from the wrong ones
    mis-codes them."""
    c16 = np.asarray(cb16, dtype=np.float16).astype(np.float64)
    r = np.asarray(real64, dtype=np.float64)
    pts = []
    for k in range(c16.size - 1):
        m16 = 0.5 * (c16[k] + c16[k + 1])
        m64 = 0.5 * (r[k] + r[k + 1])
        a, b = min(m16, m64), max(m16, m64)
        x = np.float32(a)
        for _ in range(4):
            x = np.nextafter(x, np.float32(np.inf))
        while float(x) < b:
            xs = float(x)
            sp = float(np.spacing(np.abs(x)))
            if xs - a > 2 * sp and b - xs > 2 * sp:
                pts.append(x)
            # at most a few hundred points per gap
            step = max((b - a) / 200.0, sp)
            x = np.float32(xs + step)
    return np.array(pts, dtype=np.float32)


@pytest.mark.parametrize("bits", range(1, 9))
def test_boundaries_give_the_nearest_fp16_centroid(bits):
    """code_of(u, boundaries(b)) is the index of the nearest fp16 centroid, by brute force over
    every centroid, on a dense grid away from the boundaries."""
    cb = cbk.codebook(bits)
    bd = cbk.boundaries(bits)
    top = float(cb[-1]) * 1.3 + 0.5
    u = _grid_away_from(bd, -top, top, 200_001, bits)
    assert u.size > 300_000
    assert np.array_equal(qz.code_of(u, bd), _nearest(u, cb))


@pytest.mark.parametrize("bits", range(2, 9))
def test_boundaries_use_the_fp16_centroids_in_the_sliver(bits):
    """Between the midpoints of the fp16 and the fp64 centroids the two nearest-centroid rules
    disagree; the codebook's boundaries must follow the fp16 centroids (they are the codebook)."""
    cb = cbk.codebook(bits)
    real = cbk.lloyd_max_real(bits)
    u = _sliver_points(cb, real)
    assert u.size > 0
    got = qz.code_of(u, cbk.boundaries(bits))
    assert np.array_equal(got, _nearest(u, cb))
    # and the sliver really separates the two rules
    assert not np.array_equal(got, _nearest(u, real.astype(np.float64)))


def test_nf16_boundaries_give_the_nearest_level():
    lv = cbk.nf16_levels()
    bd = cbk.nf16_boundaries()
    u = _grid_away_from(bd, -1.05, 1.05, 200_001, 99)
    assert np.array_equal(qz.code_of(u, bd), _nearest(u, lv))
    u2 = _sliver_points(lv, cbk.nf16_real())
    assert u2.size > 0
    assert np.array_equal(qz.code_of(u2, bd), _nearest(u2, lv))


def _rows(n, seed, scale=None):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 128))
    if scale is not None:
        x = x * scale[None, :]
    return x.astype(np.float16)


def _mixed_plan(seed):
    """Block widths with runs of several widths (2..8, and two zero-width blocks) summing to
    128 * 5 bits, with gains from a spread of block energies."""
    rng = np.random.default_rng(seed)
    w = np.array([8] * 11 + [7] * 6 + [6] * 12 + [5] * 8 + [4] * 10 + [3] * 8 + [2] * 7 + [0] * 2)
    w = w[rng.permutation(64)]
    assert w.size == 64 and 2 * w.sum() == 128 * 5
    m = np.exp(rng.standard_normal(64))
    g, ig = al.gains(m)
    return w, g, ig


def _hadamard_groups(widths, signs, pairing="half"):
    """The group rotation as one explicit 128 x 128 matrix: in plan field order, each run of
    equal-width fields is cut into power-of-two chunks (binary digits of the run length, largest
    first) and every chunk gets scipy's Sylvester-Hadamard matrix times the signs of its dims
    (divided by sqrt(m) afterwards, so the integer matrix stays exact)."""
    dims, ws = al.field_order(widths, 128, pairing)
    H = np.eye(128)
    div = np.ones(128)
    f = 0
    while f < len(ws):
        e = f
        while e < len(ws) and ws[e] == ws[f]:
            e += 1
        start = f
        for size in [1 << k for k in range(7, -1, -1) if (e - f) >> k & 1]:
            d = np.asarray(dims[start:start + size])
            blk = linalg.hadamard(size).astype(np.float64) * np.asarray(signs, np.float64)[d][None, :]
            H[np.ix_(d, d)] = blk
            div[d] = np.sqrt(float(size))
            start += size
        f = e
    return H, div


def test_group_rotated_input_equals_explicit_hadamard_matrices():
    w, g, ig = _mixed_plan(1)
    signs = np.random.default_rng(2).choice([-1, 1], size=128).astype(np.int8)
    x = _rows(300, 3, scale=al.dim_values(np.asarray(g, np.float64), 128) * 3.0)
    H, div = _hadamard_groups(w, signs)
    # v = fp32(x * ig) (one fp32 multiply), the matrix product exact in fp64, one division
    v = (x.astype(np.float32) * al.dim_values(np.asarray(ig, np.float32), 128)[None, :]).astype(np.float32)
    ref = ((v.astype(np.float64) @ H.T) / div[None, :]).astype(np.float32)
    got = cd.group_rotated_input(x, w, ig, signs)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # codes: the group-rotated rows through the plain quantizer with unit gains
    c, s16 = cd.quantize_bgtq_group_rotated(x, w, ig, signs)
    c_ref, s_ref, _ = qz.quantize_rows(ref, al.dim_widths(w, 128))
    assert np.array_equal(c, c_ref) and np.array_equal(s16.view(np.uint16), s_ref.view(np.uint16))
    # zero-width blocks are neither stored nor rotated
    zero = al.dim_widths(w, 128) == 0
    assert np.all(c[:, zero] == 0)


def test_group_rotation_never_mixes_widths():
    """The explicit matrix only couples dims of one width, and the dequantizer inverts the rotation
    exactly on any stored row (codes at the centroids reconstruct to g * R^T y)."""
    w, g, ig = _mixed_plan(4)
    signs = np.random.default_rng(5).choice([-1, 1], size=128).astype(np.int8)
    H, _ = _hadamard_groups(w, signs)
    wd = al.dim_widths(w, 128)
    nz = np.argwhere(H != 0)
    assert np.all(wd[nz[:, 0]] == wd[nz[:, 1]])
    rng = np.random.default_rng(6)
    codes = np.zeros((5, 128), np.uint8)
    for i in range(128):
        if wd[i]:
            codes[:, i] = rng.integers(0, 1 << wd[i], size=5)
    s16 = np.full(5, 1.5, np.float16)
    kh = cd.dequant_bgtq_group_rotated(codes, s16, w, g, signs)
    # rotate back with the explicit matrix: R (kh / g) must be the dequantized rotated row
    gd = al.dim_values(np.asarray(g, np.float32), 128).astype(np.float64)
    Hm, div = _hadamard_groups(w, signs)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(gd > 0, kh / gd, 0.0)
    yr = (y @ Hm.T) / div[None, :]
    y_hat = np.zeros((5, 128))
    for i in range(128):
        if wd[i]:
            y_hat[:, i] = 1.5 * cbk.codebook(int(wd[i])).astype(np.float64)[codes[:, i]]
    assert np.allclose(yr, y_hat, rtol=0, atol=1e-12)


def _rel_mse(x, x_hat):
    x = np.asarray(x, dtype=np.float64)
    return float(np.mean((x - x_hat) ** 2) / np.mean(x ** 2))


def test_round_trips_within_the_codebook_error():
    """At 8 bits every codec's reconstruction error is the codebook's own distortion c(8)
    (per unit of row energy), and at a mixed plan the energy-weighted mix of c(b): a dropped
    gain, a missing inverse rotation or a transposed operand would be orders of magnitude off."""
    c8 = cbk.distortion(8)
    x = _rows(4000, 7)
    ones = np.ones(64, np.float32)
    w8 = np.full(64, 8)
    signs = np.random.default_rng(8).choice([-1, 1], size=128).astype(np.int8)
    # Block-GTQ at a uniform 8 bits with unit gains
    c, s = cd.quantize_bgtq_keys(x, w8, ones)
    assert 0.7 * c8 < _rel_mse(x, cd.dequant_bgtq_keys(c, s, w8, ones)) < 1.4 * c8
    # values
    c, s = cd.quantize_values(x, 8)
    assert 0.7 * c8 < _rel_mse(x, cd.dequant_values(c, s, 8)) < 1.4 * c8
    # rotated uniform
    c, s = cd.quantize_rotated_uniform(x, 8, signs)
    assert 0.7 * c8 < _rel_mse(x, cd.dequant_rotated_uniform(c, s, 8, signs)) < 1.4 * c8
    # group rotated, uniform plan (one run of 128 fields)
    c, s = cd.quantize_bgtq_group_rotated(x, w8, ones, signs)
    assert 0.7 * c8 < _rel_mse(x, cd.dequant_bgtq_group_rotated(c, s, w8, ones, signs)) < 1.4 * c8
    # gains: rows with a spread of block energies, the allocation's gains equalise them
    w, g, ig = _mixed_plan(9)
    gd = al.dim_values(np.asarray(g, np.float64), 128)
    xs = _rows(4000, 10, scale=gd)
    wd = al.dim_widths(w, 128)
    stored = wd > 0
    # expected error: sum over stored dims of g_i^2 c(b_i) per unit of gain-normalised energy
    want = np.sum((gd ** 2 * np.array([cbk.distortion(int(b)) for b in wd]))[stored]) / np.sum(gd[stored] ** 2)
    for kh in (cd.dequant_bgtq_keys(*cd.quantize_bgtq_keys(xs, w, ig), w, g),
               cd.dequant_bgtq_group_rotated(*cd.quantize_bgtq_group_rotated(xs, w, ig, signs), w, g, signs)):
        got = float(np.mean((xs[:, stored].astype(np.float64) - kh[:, stored]) ** 2) /
                    np.mean(xs[:, stored].astype(np.float64) ** 2))
        assert 0.6 * want < got < 1.6 * want, (got, want)
        assert np.all(kh[:, ~stored] == 0)


def test_nf16_head_slices_take_their_block_scale():
    """Four KV heads = two 256-value blocks per token: heads 0, 1 share block 0's absmax scale and
    heads 2, 3 block 1's; each head's slice reconstructs its values within half the widest gap
    between neighbouring levels times the scale."""
    rng = np.random.default_rng(11)
    N = 64
    x = rng.standard_normal((N, 512)).astype(np.float32)
    # plant the absmax of each block in a known head
    x[:, 130] = 9.0      # block 0, head 1
    x[:, 300] = -7.0     # block 1, head 2
    x = x.astype(np.float16)
    codes, s16 = cd.quantize_nf16_tokens(x)
    assert s16.shape == (N, 2)
    lv = cbk.nf16_levels().astype(np.float64)
    half_gap = 0.5 * np.max(np.diff(lv))
    for h in range(4):
        ch, sh = cd.nf16_head_slice(codes, s16, h)
        assert ch.shape == (N, 128) and sh.shape == (N,)
        want = np.float16(9.0) if h < 2 else np.float16(7.0)
        assert np.all(sh == want)
        xh = cd.dequant_nf16_head(ch, sh)
        err = np.abs(x[:, 128 * h:128 * (h + 1)].astype(np.float64) - xh)
        assert np.all(err <= half_gap * float(want) * (1 + 1e-3)), h
        # the slice's codes are the token-vector codes of those columns
        assert np.array_equal(ch, codes[:, 128 * h:128 * (h + 1)])
    # the planted maxima take the end codes
    assert np.all(codes[:, 130] == 15) and np.all(codes[:, 300] == 0)
