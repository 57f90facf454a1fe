"""Pins of oracle.quantize and oracle.layout."""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import allocation as al
from oracle import codebooks as cbk
from oracle import layout as lay
from oracle import quantize as qz


def _half_rne(x: float) -> float:
    return struct.unpack("<e", struct.pack("<e", x))[0]


def _f32(x: float) -> float:
    return struct.unpack("<f", struct.pack("<f", x))[0]


@pytest.mark.parametrize("bits", range(1, 9))
def test_idempotence_and_cells(bits):
    cb = cbk.codebook(bits).astype(np.float32)
    bd = cbk.boundaries(bits)
    codes = np.arange(cb.size)
    # a centroid re-quantizes to its own code
    assert np.array_equal(qz.code_of(cb, bd), codes)
    # saturation and boundary ties (a u exactly on a boundary takes the lower code)
    assert qz.code_of(np.array([1e30], np.float32), bd)[0] == cb.size - 1
    assert qz.code_of(np.array([-1e30], np.float32), bd)[0] == 0
    assert np.array_equal(qz.code_of(bd, bd), np.arange(bd.size))
    up = np.nextafter(bd, np.float32(np.inf))
    assert np.array_equal(qz.code_of(up, bd), np.arange(bd.size) + 1)
    # monotone in u
    u = np.sort(np.random.default_rng(bits).standard_normal(5000).astype(np.float32) * 3)
    assert np.all(np.diff(qz.code_of(u, bd).astype(int)) >= 0)


def test_scale_chain_against_exact_arithmetic():
    # steps 2-5 recomputed with exact rationals and correctly rounded casts from the standard library
    rng = np.random.default_rng(12)
    for trial in range(200):
        x = (rng.standard_normal(128) * 10.0 ** rng.uniform(-3, 3)).astype(np.float16)
        ig = (np.exp(rng.standard_normal(128))).astype(np.float32)
        codes, s16, u = qz.quantize_rows(x[None, :], np.full(128, 3), ig)
        y = [_f32(float(xi) * float(gi)) for xi, gi in zip(x, ig)]
        ss = 0.0
        for v in y:                       # fp64 running sum, i ascending (Python floats are fp64)
            ss = ss + v * v
        r = ss / 128.0
        s64 = math.sqrt(r)                # correctly rounded fp64 sqrt
        s_ref = _half_rne(_f32(s64))
        assert float(s16[0]) == s_ref
        is_ref = 0.0 if s_ref == 0 else _f32(float(Fraction(1) / Fraction(s_ref)))
        u_ref = [_f32(v * is_ref) for v in y]
        assert np.array_equal(u[0], np.array(u_ref, dtype=np.float32))
        bd = [float(b) for b in cbk.boundaries(3)]
        assert [int(c) for c in codes[0]] == [sum(1 for b in bd if b < v) for v in u_ref]


def test_zero_row_and_zero_width():
    codes, s16, u = qz.quantize_rows(np.zeros((1, 128), np.float16), np.full(128, 4))
    assert s16[0] == 0 and np.all(u == 0)
    assert np.all(codes == 7)              # 7 negative boundaries; the zero boundary is not < 0
    wd = np.full(128, 3)
    wd[:10] = 0
    codes, _, _ = qz.quantize_rows(np.ones((2, 128), np.float32), wd)
    assert np.all(codes[:, :10] == 0)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_quantizer_mse_on_gaussian_rows(bits):
    rng = np.random.default_rng(bits)
    x = rng.standard_normal((20000, 128)).astype(np.float32)
    codes, s16, u = qz.quantize_rows(x, np.full(128, bits))
    cb = cbk.codebook(bits).astype(np.float64)
    xhat = s16.astype(np.float64)[:, None] * cb[codes]
    mse = np.mean((x.astype(np.float64) - xhat) ** 2)
    # the row RMS scale is ~1 for N(0,1) rows of 128 values, so the per-value MSE is ~c(b)
    assert mse == pytest.approx(cbk.distortion(bits), rel=0.06)


def test_gains_equalise_blocks():
    # a block with 10x the energy clips without gains and is fine with them
    rng = np.random.default_rng(1)
    d = 128
    sig = np.ones(64)
    sig[3] = 10.0
    x = rng.standard_normal((4000, d)) * al.dim_values(sig, d)[None, :]
    m = al.energy(x[:, None, :])[0]
    g, ig = al.gains(m[None])
    wd = np.full(d, 3)
    c0, s0, _ = qz.quantize_rows(x, wd)
    c1, s1, _ = qz.quantize_rows(x, wd, al.dim_values(ig[0], d))
    cb = cbk.codebook(3).astype(np.float64)
    e0 = (x - s0.astype(np.float64)[:, None] * cb[c0]) ** 2
    gd = al.dim_values(g[0], d).astype(np.float64)
    e1 = (x - s1.astype(np.float64)[:, None] * gd[None, :] * cb[c1]) ** 2
    p0, p1 = al.block_pairs(d)
    assert e1[:, [p0[3], p1[3]]].mean() < 0.2 * e0[:, [p0[3], p1[3]]].mean()


def test_nf16_codec():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((300, 1024)).astype(np.float16)
    codes, s16, u = qz.quantize_nf16(x)
    assert s16.shape == (300, 4)
    xb = x.astype(np.float32).reshape(300, 4, 256)
    # the scale is the block's absmax (exact for fp16 input)
    assert np.array_equal(s16.astype(np.float32), np.abs(xb).max(axis=2))
    # the max-magnitude element of each block maps to an end level
    cb = codes.reshape(300, 4, 256)
    amax = np.abs(xb).argmax(axis=2)
    ends = np.take_along_axis(cb, amax[..., None], axis=2)[..., 0]
    assert np.all((ends == 0) | (ends == 15))
    # mirrored input gives mirrored codes (no exact zeros in this sample)
    assert not np.any(x == 0)
    cm, sm, _ = qz.quantize_nf16(-x)
    assert np.array_equal(cm, 15 - codes) and np.array_equal(sm, s16)
    # an all-zero block stores code 7 and dequantizes to 0
    z = np.zeros((1, 256), np.float16)
    cz, sz, _ = qz.quantize_nf16(z)
    assert np.all(cz == 7) and sz[0, 0] == 0


def test_pack_hand_example():
    # fields (dim, width) = (2,3) (0,3) (1,2) then six (3,4) fillers: 3+3+2+24 = 32 bits.
    # codes dim0=5 (101), dim1=2 (10), dim2=6 (110), dim3=9 (1001); LSB first:
    # bits [0,3)=6, [3,6)=5, [6,8)=2, [8,32)=9 repeated six times
    codes = np.array([[5, 2, 6, 9]], dtype=np.uint8)
    dims = np.array([2, 0, 1, 3, 3, 3, 3, 3, 3])
    widths = np.array([3, 3, 2, 4, 4, 4, 4, 4, 4])
    words = lay.pack_k_rows(codes, dims, widths, 1)
    expect = 6 | (5 << 3) | (2 << 6)
    for k in range(6):
        expect |= 9 << (8 + 4 * k)
    assert int(words[0, 0]) == expect == 0x999999AE
    assert np.array_equal(lay.unpack_k_rows(words, dims, widths, 4)[0], [5, 2, 6, 9])


def test_pack_straddle_and_roundtrip():
    rng = np.random.default_rng(8)
    for budget in (2, 3, 4, 5, 7):
        s = np.exp(2 * rng.standard_normal(64))
        b = al.greedy_allocate(s, budget, 0, 8, cbk.delta_table())
        for pairing in ("half", "interleaved"):
            dims, ws = al.field_order(b, 128, pairing)
            wd = al.dim_widths(b, 128, pairing)
            codes = np.zeros((50, 128), np.uint8)
            for i in range(128):
                if wd[i]:
                    codes[:, i] = rng.integers(0, 1 << wd[i], 50)
            words = lay.pack_k_rows(codes, dims, ws, 4 * budget)
            assert words.shape == (50, 4 * budget)
            assert np.array_equal(lay.unpack_k_rows(words, dims, ws, 128), codes)
            # the bit count check: each field contributes exactly its width
            total = sum(bin(int(w)).count("1") for w in words.ravel())
            assert total == sum(bin(int(c)).count("1") for c in codes.ravel())


def test_v_tile_layout():
    rng = np.random.default_rng(3)
    for bits in (1, 2, 3, 4, 8):
        T = 300
        codes = rng.integers(0, 1 << bits, (T, 128)).astype(np.uint8)
        words = lay.pack_v_tiles(codes, bits)
        assert words.shape == (3, 512, bits)
        assert np.array_equal(lay.unpack_v_tiles(words, bits, T), codes)
        # token 32g + e of dim d in tile t sits at bit e*bits of segment ((d//16)*4 + g)*16 + d%16
        for (t, d, tok) in ((1, 77, 45), (0, 0, 0), (2, 127, 31), (0, 16, 100)):
            g, e = divmod(tok, 32)
            seg = ((d // 16) * 4 + g) * 16 + d % 16
            stream = 0
            for k, w in enumerate(words[t, seg]):
                stream |= int(w) << (32 * k)
            assert (stream >> (e * bits)) & ((1 << bits) - 1) == codes[t * 128 + tok, d]
        # padding tokens of the last tile are zero
        assert np.all(lay.unpack_v_tiles(words, bits, 384)[T:] == 0)
