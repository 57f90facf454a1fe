"""Pins of oracle.attention: library attention, special cases, RoPE identity, byte arithmetic."""
import numpy as np
import pytest
import torch

from oracle import allocation as al
from oracle import attention as at
from oracle import codebooks as cbk
from oracle import layout as lay
from oracle import quantize as qz
from synth import apply_rope


def _torch_sdpa(q, k, v, scale):
    # library routine: torch's scaled_dot_product_attention in float64 on the CPU, GQA expanded
    H_q, d = q.shape
    H_kv = k.shape[0]
    G = H_q // H_kv
    qt = torch.from_numpy(q).reshape(1, H_q, 1, d)
    kt = torch.from_numpy(np.repeat(k, G, axis=0)).reshape(1, H_q, -1, d)
    vt = torch.from_numpy(np.repeat(v, G, axis=0)).reshape(1, H_q, -1, d)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return o.reshape(H_q, d).numpy()


@pytest.mark.parametrize("H_q,H_kv,T", [(1, 1, 37), (8, 2, 300), (32, 8, 129)])
def test_decode_attention_matches_torch(H_q, H_kv, T):
    rng = np.random.default_rng(H_q + T)
    q = rng.standard_normal((H_q, 128))
    k = rng.standard_normal((H_kv, T, 128))
    v = rng.standard_normal((H_kv, T, 128))
    for scale in (None, 0.03):
        ref = _torch_sdpa(q, k, v, 1 / np.sqrt(128) if scale is None else scale)
        assert np.allclose(at.decode_attention(q, k, v, scale), ref, rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((4, 128))
    k = rng.standard_normal((1, 1, 128))
    v = rng.standard_normal((1, 1, 128))
    assert np.allclose(at.decode_attention(q, k, v), np.repeat(v[0], 4, axis=0), rtol=0, atol=1e-15)
    k = np.repeat(rng.standard_normal((1, 1, 128)), 50, axis=1)
    v = rng.standard_normal((1, 50, 128))
    assert np.allclose(at.decode_attention(q, k, v), v[0].mean(axis=0)[None], atol=1e-14)


@pytest.mark.parametrize("pairing", ["half", "interleaved"])
def test_rope_block_decomposition(pairing):
    rng = np.random.default_rng(1)
    for theta in (1.0e4, 5.0e5, 1.0e6):
        q0, k0 = rng.standard_normal(128), rng.standard_normal(128)
        m, n = 131072, 77777
        qr = apply_rope(q0[None], np.array([m]), theta, pairing)[0]
        kr = apply_rope(k0[None], np.array([n]), theta, pairing)[0]
        flat = float(qr @ kr)
        assert at.rope_block_logit(q0, k0, m, n, theta, pairing) == pytest.approx(flat, rel=1e-11, abs=1e-11)
        # rotation keeps every block's norm
        p0, p1 = al.block_pairs(128, pairing)
        assert np.allclose(kr[p0] ** 2 + kr[p1] ** 2, k0[p0] ** 2 + k0[p1] ** 2, rtol=1e-12)


def test_dequant_round_trip_error():
    rng = np.random.default_rng(5)
    sig = np.exp(rng.standard_normal(64))
    x = (rng.standard_normal((3000, 128)) * al.dim_values(sig, 128)[None]).astype(np.float16)
    m = al.energy(x[:, None, :])[0]
    b = al.greedy_allocate(m, 3, 0, 8, cbk.delta_table())
    g, ig = al.gains(m[None])
    wd = al.dim_widths(b, 128)
    codes, s16, _ = qz.quantize_rows(x, wd, al.dim_values(ig[0], 128))
    xh = at.dequant_k(codes, s16, wd, al.dim_values(g[0], 128))
    err = np.mean((xh - x.astype(np.float64)) ** 2, axis=0)
    # per-dim error follows m_j * c(b_j) (the allocator's model) within Monte-Carlo slack
    c = np.array([cbk.distortion(w) for w in range(9)])
    model = al.dim_values(m, 128) * c[wd]
    assert np.allclose(err, model, rtol=0.35)
    v = rng.standard_normal((500, 128)).astype(np.float16)
    cv, sv, _ = qz.quantize_rows(v, np.full(128, 2))
    vh = at.dequant_v(cv, sv, 2)
    assert np.mean((vh - v.astype(np.float64)) ** 2) == pytest.approx(cbk.distortion(2), rel=0.1)
    xn = rng.standard_normal((200, 1024)).astype(np.float16)
    cn, sn, _ = qz.quantize_nf16(xn)
    xnh = at.dequant_nf16(cn, sn)
    assert np.max(np.abs(xnh - xn.astype(np.float64))) <= np.max(sn.astype(np.float64)) * 0.3


def test_compression_arithmetic_from_packed_buffers():
    # bytes of actually packed K rows + V tiles + fp16 scales for 1024 tokens of one head
    rng = np.random.default_rng(2)
    T = 1024
    for kb, vb, expect in ((2, 2, 7.53), (3, 3, 5.12), (4, 4, 3.88), (3, 2, 6.10)):
        s = np.exp(2 * rng.standard_normal(64))
        b = al.greedy_allocate(s, kb, 0, 8, cbk.delta_table())
        dims, ws = al.field_order(b, 128)
        kw = lay.pack_k_rows(np.zeros((T, 128), np.uint8), dims, ws, 4 * kb)
        vw = lay.pack_v_tiles(np.zeros((T, 128), np.uint8), vb)
        packed = kw.nbytes + vw.nbytes + 2 * T * np.dtype(np.float16).itemsize
        fp16 = 2 * T * 128 * 2
        assert packed / T == at.bytes_per_token_head(kb, vb)
        assert fp16 / packed == pytest.approx(expect, abs=0.005)
        assert at.compression_ratio(kb, vb) == pytest.approx(fp16 / packed, rel=1e-15)
    # the per-256-value absmax codec: 4-bit codes for K and V + one fp16 per 256 values each
    codes, s16, _ = qz.quantize_nf16(np.ones((T, 1024), np.float16))
    per_head = (2 * (codes.size // 2 + s16.nbytes)) / (T * 8)
    assert per_head == at.nf16_bytes_per_token_head() == 130.0
    assert 2 * 2 * 128 / per_head == pytest.approx(3.94, abs=0.005)
    # the headline workload: 36 layers x 2 KV heads x 131072 tokens at K3V3
    assert 36 * 2 * 131072 * at.bytes_per_token_head(3, 3) == 943_718_400
