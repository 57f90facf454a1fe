"""Pins of the rotation oracle (oracle/rotation.py): the Hadamard matrix of a library routine,
orthogonality, exactness on fp16 inputs, and the effect the rotation exists for."""
import numpy as np
import pytest
from scipy import linalg

from oracle import allocation as al
from oracle import attention as at
from oracle import fidelity as fd
from oracle import quantize as qz
from oracle import rotation as rt
from synth import WORKLOADS, gen_layer, gen_query


@pytest.mark.parametrize("d", [2, 8, 128])
def test_fwht_equals_sylvester_hadamard(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((5, d))
    assert np.allclose(rt.fwht(x), x @ linalg.hadamard(d).T, rtol=0, atol=1e-12)


def test_rotation_is_orthogonal_and_inverted():
    rng = np.random.default_rng(1)
    s = rng.choice([-1.0, 1.0], size=128)
    x = rng.standard_normal((7, 128))
    y = rt.rotate(x, s)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    assert np.allclose(rt.unrotate(y, s), x, atol=1e-14)
    R = rt.rotate(np.eye(128), s)          # rows: R e_i = column i of R
    assert np.allclose(R @ R.T, np.eye(128), atol=1e-14)


def test_fwht_exact_on_fp16_rows():
    # sums of fp16 values with signs are exact in fp64: the order of the butterflies does not
    # change the result, so the product path's transform matches bit for bit
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 128)).astype(np.float16).astype(np.float64) * 37.0
    s = rng.choice([-1.0, 1.0], size=128)
    direct = (x * s) @ linalg.hadamard(128).T.astype(np.float64)
    assert np.array_equal(rt.fwht(x * s), direct)


def test_rotation_spreads_outlier_blocks():
    """The reason for the rotation: with a uniform width and one scale per row, the synthetic
    x10 outlier blocks dominate the row scale; rotated rows have a flat coordinate law, so the
    logit MAE drops.  (Block-GTQ's own answer is per-block widths and gains.)"""
    w = WORKLOADS["llama8b_32k"]
    T, bits = 2048, 3
    k, _ = gen_layer(w, 0, 0, T)
    k = np.asarray(k, dtype=np.float64)
    q = np.asarray(gen_query(w, 0, T), dtype=np.float64)
    rng = np.random.default_rng(3)
    kt = np.transpose(k, (1, 0, 2))
    wu = np.full(128, bits)
    kh_u, kh_r = [], []
    for h in range(w.n_kv):
        s = rng.choice([-1.0, 1.0], size=128)
        cu, su, _ = qz.quantize_rows(k[:, h], wu)
        kh_u.append(at.dequant_k(cu, su, wu, np.ones(128, np.float32)))
        cr, sr, _ = qz.quantize_rows(rt.rotate_rows_fp32(k[:, h], s), wu)
        kh_r.append(rt.unrotate(at.dequant_k(cr, sr, wu, np.ones(128, np.float32)), s))
    mae_u, _ = fd.logit_fidelity(q, kt, np.stack(kh_u))
    mae_r, _ = fd.logit_fidelity(q, kt, np.stack(kh_r))
    assert mae_r.mean() < 0.5 * mae_u.mean(), (mae_r.mean(), mae_u.mean())


@pytest.mark.parametrize("bits", [2, 3])
def test_block_allocation_beats_rotated_uniform_on_logit_mae(bits):
    """The pages' claim against uniform TQ-MSE (abstract: lower per-layer logit MAE at 2 and 3
    bits per dim, keys only), here against the rotated flat-vector baseline."""
    w = WORKLOADS["llama8b_32k"]
    T = 2048
    k, _ = gen_layer(w, 0, 0, T)
    k = np.asarray(k, dtype=np.float64)
    q = np.asarray(gen_query(w, 0, T), dtype=np.float64)
    rng = np.random.default_rng(4)
    widths, g, ig, _ = al.allocate(k, bits)
    wu = np.full(128, bits)
    kb, kr = [], []
    for h in range(w.n_kv):
        wd = al.dim_widths(widths[h], 128)
        ck, sk, _ = qz.quantize_rows(k[:, h], wd, al.dim_values(ig[h], 128))
        kb.append(at.dequant_k(ck, sk, wd, al.dim_values(g[h], 128)))
        s = rng.choice([-1.0, 1.0], size=128)
        cr, sr, _ = qz.quantize_rows(rt.rotate_rows_fp32(k[:, h], s), wu)
        kr.append(rt.unrotate(at.dequant_k(cr, sr, wu, np.ones(128, np.float32)), s))
    kt = np.transpose(k, (1, 0, 2))
    mae_b, _ = fd.logit_fidelity(q, kt, np.stack(kb))
    mae_r, _ = fd.logit_fidelity(q, kt, np.stack(kr))
    assert mae_b.mean() < mae_r.mean(), (mae_b.mean(), mae_r.mean())


# ---- rotations inside equal-width groups ---------------------------------------------------

def test_group_chunks_hand_example():
    w = np.array([5, 5, 4, 4, 4, 4, 4, 4, 3, 3, 3, 3, 3, 3, 3, 3, 3, 3, 3, 3, 3, 3, 2, 2])
    # runs: 2 fives, 6 fours (4 + 2), 14 threes (8 + 4 + 2), 2 twos
    assert rt.group_chunks(w) == [(0, 2), (2, 4), (6, 2), (8, 8), (16, 4), (20, 2), (22, 2)]


@pytest.mark.parametrize("seed", range(5))
def test_group_chunks_partition_runs_in_binary_order(seed):
    rng = np.random.default_rng(seed)
    w = np.sort(rng.integers(1, 9, size=64))[::-1].repeat(2)     # a plan: pairs, widest first
    ch = rt.group_chunks(w)
    assert [s for s, _ in ch] == list(np.cumsum([0] + [m for _, m in ch])[:-1])
    assert sum(m for _, m in ch) == len(w)
    for s, m in ch:
        assert m & (m - 1) == 0 and len(set(w[s:s + m])) == 1
    for width in set(w.tolist()):
        sizes = [m for s, m in ch if w[s] == width]
        assert sizes == sorted(sizes, reverse=True) and sum(sizes) == int((w == width).sum())
        assert len(sizes) == bin(sum(sizes)).count("1")


def _plan(seed):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((256, 1, 128)) * np.exp(rng.standard_normal(128))
    widths, _, _, _ = al.allocate(K, 3)
    dims, ws = al.field_order(widths[0], 128, "half")
    return widths[0], dims, ws


@pytest.mark.parametrize("seed", range(3))
def test_group_rotation_matrix_structure(seed):
    """R is orthogonal, never mixes dims of different widths, and each chunk is the Sylvester
    Hadamard matrix with the signs, over sqrt(m), in field order."""
    widths, dims, ws = _plan(seed)
    s = np.random.default_rng(50 + seed).choice([-1.0, 1.0], size=128)
    R = rt.rotate_in_groups(np.eye(128), s, dims, ws).T       # column j = R e_j
    stored = np.zeros(128, bool)
    stored[dims] = True
    Rs = R[np.ix_(stored, stored)]
    assert np.allclose(Rs @ Rs.T, np.eye(stored.sum()), atol=1e-14)
    wd = al.dim_widths(widths, 128, "half")
    nz = np.abs(R) > 0
    assert not np.any(nz & (wd[:, None] != wd[None, :]))
    for st, m in rt.group_chunks(ws):
        d = dims[st:st + m]
        assert np.allclose(R[np.ix_(d, d)], linalg.hadamard(m) * s[d][None, :] / np.sqrt(m), atol=1e-15)
    # width-0 dims pass through
    for i in np.flatnonzero(~stored):
        assert R[i, i] == 1.0 and np.count_nonzero(R[:, i]) == 1


def test_group_rotation_inverts_and_keeps_group_energy():
    widths, dims, ws = _plan(7)
    rng = np.random.default_rng(8)
    s = rng.choice([-1.0, 1.0], size=128)
    x = rng.standard_normal((9, 128))
    y = rt.rotate_in_groups(x, s, dims, ws)
    assert np.allclose(rt.unrotate_in_groups(y, s, dims, ws), x, atol=1e-13)
    wd = al.dim_widths(widths, 128, "half")
    for width in set(wd.tolist()):
        g = wd == width
        assert np.allclose((y[:, g] ** 2).sum(1), (x[:, g] ** 2).sum(1), rtol=1e-13)
