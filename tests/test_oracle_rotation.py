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
