"""Pins of the KIVI-style asymmetric integer codec's oracle (oracle/kivi.py): exact grids,
the rounding error bound, degenerate groups, which axis a group runs along, brute-force
nearest levels and the stored parameter layout."""
import numpy as np
import pytest

from oracle import allocation as al
from oracle import kivi as kv


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_exact_grid_is_reproduced(bits):
    """Values lying exactly on lo + s k (all fp16-exact) come back with code k, and the
    reconstruction is exact."""
    L = 1 << bits
    lo, s = -1.5, 0.25
    rng = np.random.default_rng(bits)
    k = rng.integers(0, L, size=(3, 128))
    k[:, 0], k[:, 1] = 0, L - 1                 # the group spans the whole grid
    x = (lo + s * k).astype(np.float32)
    codes, s16, lo16 = kv.quantize_groups(x, bits)
    assert np.all(s16 == np.float16(s)) and np.all(lo16 == np.float16(lo))
    assert np.array_equal(codes, k)
    assert np.array_equal(kv.reconstruct(codes, s16[:, None], lo16[:, None]), x.astype(np.float64))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_error_bound(bits):
    """|x - x_hat| <= s / 2 plus the fp16 roundings of lo, hi, s and of the reconstruction."""
    rng = np.random.default_rng(10 + bits)
    x = rng.standard_normal((64, 128)).astype(np.float16).astype(np.float32)
    codes, s16, lo16 = kv.quantize_groups(x, bits)
    xh = kv.reconstruct(codes, s16[:, None], lo16[:, None])
    s = s16.astype(np.float64)[:, None]
    L = (1 << bits) - 1
    # s itself is rounded to fp16 (relative 2^-11), which moves the top level by up to L s 2^-11
    bound = s / 2 + L * s * 2.0 ** -11 + np.spacing(np.abs(x).max(axis=1, keepdims=True).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(x - xh) <= bound)


def test_uniform_mse_matches_step_squared_over_12():
    rng = np.random.default_rng(3)
    x = rng.uniform(-1, 1, size=(512, 128)).astype(np.float32)
    codes, s16, lo16 = kv.quantize_groups(x, 4)
    err = x - kv.reconstruct(codes, s16[:, None], lo16[:, None])
    mse, step = np.mean(err ** 2), np.mean(s16.astype(np.float64))
    assert abs(mse / (step ** 2 / 12) - 1) < 0.1


def test_constant_group():
    """A constant group has s = 0: every code 0, reconstructed exactly as lo."""
    x = np.full((2, 128), 0.3, dtype=np.float32)
    x[1] = -7.0
    codes, s16, lo16 = kv.quantize_groups(x, 3)
    assert np.all(s16 == 0) and np.all(codes == 0)
    assert np.array_equal(kv.reconstruct(codes, s16[:, None], lo16[:, None])[:, 0],
                          np.array([np.float16(0.3), -7.0], dtype=np.float64))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_extremes_take_the_end_codes(bits):
    rng = np.random.default_rng(20 + bits)
    x = rng.standard_normal((32, 128)).astype(np.float16).astype(np.float32)
    codes, _, _ = kv.quantize_groups(x, bits)
    r = np.arange(32)
    assert np.all(codes[r, x.argmin(axis=1)] == 0)
    assert np.all(codes[r, x.argmax(axis=1)] == (1 << bits) - 1)


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_nearest_level_brute_force(bits):
    """Every code is a nearest level of the exact (x - lo) / s, up to the fp32 rounding of u."""
    rng = np.random.default_rng(30 + bits)
    x = rng.standard_normal((16, 128)).astype(np.float16).astype(np.float32)
    codes, s16, lo16 = kv.quantize_groups(x, bits)
    L = 1 << bits
    t = (x.astype(np.float64) - lo16.astype(np.float64)[:, None]) / s16.astype(np.float64)[:, None]
    dist = np.abs(t[..., None] - np.arange(L)[None, None, :])          # [16, 128, L]
    best = dist.min(axis=-1)
    got = np.take_along_axis(dist, codes[..., None], axis=-1)[..., 0]
    assert np.all(got <= best + 1e-5)


def test_keys_group_per_channel_and_values_per_position():
    """Channel c of a key tile spans (c + 1) times the base range, so its step grows with c;
    position p of a value row block spans (p + 1) times it, so the step grows with p."""
    rng = np.random.default_rng(5)
    z = rng.uniform(-1, 1, size=128)
    z[0], z[1] = -1.0, 1.0
    xk = np.outer(z, np.arange(1, 129) / 128.0).astype(np.float32)     # [position, channel]
    _, sk, lok = kv.quantize_k_tile(xk, 3)
    assert np.all(np.diff(sk.astype(np.float64)) >= 0) and sk[-1] > 100 * sk[0]
    assert np.allclose(lok.astype(np.float64), -np.arange(1, 129) / 128.0, rtol=1e-3)
    _, sv, lov = kv.quantize_v(xk.T, 3)                                 # rows are positions now
    assert np.array_equal(sv, sk) and np.array_equal(lov, lok)


def test_tiles_are_independent():
    """Each 128-position key tile has its own parameters: quantizing two tiles together
    equals quantizing each alone."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((256, 128)).astype(np.float32)
    x[128:] *= 4.0
    c, s, lo = kv.quantize_k(x, 2)
    c0, s0, lo0 = kv.quantize_k_tile(x[:128], 2)
    c1, s1, lo1 = kv.quantize_k_tile(x[128:], 2)
    assert np.array_equal(c, np.concatenate([c0, c1]))
    assert np.array_equal(s, np.stack([s0, s1])) and np.array_equal(lo, np.stack([lo0, lo1]))
    assert np.all(s1.astype(np.float64) > 2 * s0.astype(np.float64))


@pytest.mark.parametrize("pairing", ["half", "interleaved"])
def test_key_parameter_layout(pairing):
    """Block j's entry holds (s, s, lo, lo) of its two dims, p0 first."""
    s = np.arange(128, dtype=np.float16)[None, :]
    lo = -np.arange(128, dtype=np.float16)[None, :]
    lay = kv.k_params_layout(s, lo, pairing)
    assert lay.shape == (1, 64, 4)
    if pairing == "half":
        assert list(lay[0, 5]) == [5, 69, -5, -69]
    else:
        assert list(lay[0, 5]) == [10, 11, -10, -11]
    p0, p1 = al.block_pairs(128, pairing)
    assert np.array_equal(lay[0, :, 0], s[0, p0]) and np.array_equal(lay[0, :, 3], lo[0, p1])


def test_value_parameter_layout_and_bytes():
    s = np.arange(256, dtype=np.float16)
    lo = -s
    lay = kv.v_params_layout(s, lo)
    assert lay.shape == (2, 2, 128)
    assert lay[1, 0, 3] == 131 and lay[1, 1, 3] == -131
    # K3V3: 96 B of codes, 4 B of key parameters (2 fp16 per channel over 128 positions),
    # 4 B of value parameters per token-head
    assert kv.bytes_per_token_head(3, 3) == 96 + 4 + 4
