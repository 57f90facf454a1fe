"""Pins of the fidelity oracle (oracle/fidelity.py) against facts fixed by mathematics and a
library routine, plus the pages' claimed direction of the method on synthetic keys."""
import numpy as np
import pytest
from scipy import special, stats

from oracle import allocation as al
from oracle import attention as at
from oracle import fidelity as fd
from oracle import quantize as qz
from synth import WORKLOADS, gen_layer, gen_query


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_identical_keys_give_zero():
    rng = np.random.default_rng(1)
    q, k = _rand(rng, 4, 16), _rand(rng, 2, 50, 16)
    mae, kl = fd.logit_fidelity(q, k, k.copy())
    assert np.all(mae == 0.0) and np.all(np.abs(kl) < 1e-15)


def test_constant_logit_shift():
    # k_hat_t = k_t + c q: every logit moves by sigma c |q|^2, so MAE is that shift and the
    # softmax (hence KL) does not change
    rng = np.random.default_rng(2)
    q, k = _rand(rng, 1, 32), _rand(rng, 1, 40, 32)
    c = 0.37
    mae, kl = fd.logit_fidelity(q, k, k + c * q[0][None, None, :], scale=0.5)
    assert mae[0] == pytest.approx(0.5 * c * float(q[0] @ q[0]), rel=1e-12)
    assert abs(kl[0]) < 1e-13


def test_two_token_closed_form():
    # logits (0, 0) against (0, delta): KL(p || p_hat) = log((1 + e^delta) / 2) - delta / 2
    for delta in (1e-3, 0.3, 2.0, -5.0):
        q = np.array([[1.0, 0.0]])
        k = np.zeros((1, 2, 2))
        kh = np.zeros((1, 2, 2))
        kh[0, 1, 0] = delta
        mae, kl = fd.logit_fidelity(q, k, kh, scale=1.0)
        assert mae[0] == pytest.approx(abs(delta) / 2, rel=1e-14)
        assert kl[0] == pytest.approx(np.log1p(np.exp(delta)) - np.log(2.0) - delta / 2, rel=1e-9, abs=1e-15)


def test_kl_matches_scipy_entropy_and_is_nonnegative():
    rng = np.random.default_rng(3)
    d = 128
    q, k = _rand(rng, 4, d), _rand(rng, 2, 300, d)
    kh = k + 0.2 * _rand(rng, 2, 300, d)
    mae, kl = fd.logit_fidelity(q, k, kh)
    for h in range(4):
        a = (k[h // 2] @ q[h]) / np.sqrt(d)
        b = (kh[h // 2] @ q[h]) / np.sqrt(d)
        assert kl[h] == pytest.approx(stats.entropy(special.softmax(a), special.softmax(b)), rel=1e-9)
        assert mae[h] == pytest.approx(sum(abs(x - y) for x, y in zip(a, b)) / len(a), rel=1e-12)
        assert kl[h] > 0.0


def test_grouped_query_mapping():
    # only KV head 1 differs: query heads 0, 1 (KV head 0) see nothing, heads 2, 3 do
    rng = np.random.default_rng(4)
    q, k = _rand(rng, 4, 8), _rand(rng, 2, 20, 8)
    kh = k.copy()
    kh[1] += 0.1 * _rand(rng, 20, 8)
    mae, kl = fd.logit_fidelity(q, k, kh)
    assert np.all(mae[:2] == 0.0) and np.all(mae[2:] > 0.0) and np.all(kl[2:] > 0.0)


@pytest.mark.parametrize("bits", [2, 3])
def test_block_allocation_beats_uniform_on_logit_mae(bits):
    """The pages' direction: at 2 and 3 bits per dim (keys only), the RoPE-aware allocation
    gives a lower per-layer logit MAE than the same quantizer at a uniform width."""
    w = WORKLOADS["llama8b_32k"]
    T = 2048
    k, _ = gen_layer(w, 0, 0, T)
    k = np.asarray(k, dtype=np.float64)
    H = w.n_kv
    widths, g, ig, _ = al.allocate(k, bits)
    q = np.stack([np.asarray(gen_query(w, 0, T, seq=0), dtype=np.float64)])[0]
    kh_b, kh_u = [], []
    for h in range(H):
        wd = al.dim_widths(widths[h], 128)
        ck, sk, _ = qz.quantize_rows(k[:, h], wd, al.dim_values(ig[h], 128))
        kh_b.append(at.dequant_k(ck, sk, wd, al.dim_values(g[h], 128)))
        wu = np.full(128, bits)
        cu, su, _ = qz.quantize_rows(k[:, h], wu)
        kh_u.append(at.dequant_k(cu, su, wu, np.ones(128, np.float32)))
    kt = np.transpose(k, (1, 0, 2))
    mae_b, kl_b = fd.logit_fidelity(q, kt, np.stack(kh_b))
    mae_u, kl_u = fd.logit_fidelity(q, kt, np.stack(kh_u))
    assert mae_b.mean() < mae_u.mean(), (mae_b.mean(), mae_u.mean())
    assert kl_b.mean() < kl_u.mean(), (kl_b.mean(), kl_u.mean())
