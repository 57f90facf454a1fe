"""GPU (HIP, gfx950) vs oracle parity through the C ABI.

Plans, codes, packed words and scales must be bit-exact; decode attention
must match the oracle's fp64 attention over its own dequantized cache within
max-abs 2e-3 and relative L2 1e-3.  The key-fidelity diagnostics (fp64 on both
sides, the same exact products, sums in another order) must match the oracle's
within 1e-9 relative + 1e-12 absolute.
"""
import numpy as np
import pytest

from oracle import allocation as al
from oracle import attention as at
from oracle import fidelity as fd
from oracle import layout as lay
from oracle import window as wn
from synth import WORKLOADS, gen_layer, gen_query, seq_block_sigmas
from tests.parity import CODEC, PAIRING, OracleLayer, assert_attention_close, errors

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def _kvq():
    from rope_aware_bit_amd import kvq
    return kvq


def run_case(wname, T, k_bits, v_bits, codec="bgtq", pairing="half", batch=None, layer=0,
             chunks=None, n_splits=0, noise="gauss", temper=False, check_codes=True, sample_rows=None,
             b_min=0, b_max=8, fidelity=True, recent=0, query_weighted=False, zero_blocks=(),
             per_seq=False):
    """Quantize T tokens of one layer on the GPU and in the oracle; compare everything.

    recent > 0: the last `recent` positions stay in the fp16 window.  A position that was inside
    the window at the end of its append went through fp16 (fp32 inputs are rounded), and the
    packed storage holds positions 0 .. T - recent - 1.

    per_seq: every sequence draws its own block profile and gets plans of its own from its own
    calibration keys (and its own query-energy weights)."""
    torch = _torch()
    kvq = _kvq()
    w = WORKLOADS[wname]
    B = w.batch if batch is None else batch
    H, Hq = w.n_kv, w.n_q
    ks, vs, qs = [], [], []
    for b in range(B):
        sig = seq_block_sigmas(w, layer, b) if per_seq else None
        k, v = gen_layer(w, layer, 0, T, seq=b, noise=noise, pairing=pairing, sigmas=sig)
        ks.append(k)
        vs.append(v)
        qs.append(gen_query(w, layer, T, seq=b, noise=noise, pairing=pairing, sigmas=sig))
    K = np.stack(ks)            # [B, T, H, d]
    if zero_blocks:
        # degenerate blocks: both coordinates zero in every key (zero energy, zero gain)
        p0, p1 = al.block_pairs(128, pairing)
        for j in zero_blocks:
            K[..., p0[j]] = 0
            K[..., p1[j]] = 0
    V = np.stack(vs)
    Q = np.stack(qs)            # [B, Hq, d]
    print(f"[{wname} T={T} K{k_bits}V{v_bits} {codec}] inputs generated", flush=True)
    tc = min(T, w.calib_tokens)
    # calibration keys: the first tc positions of every sequence, pooled (one plan per KV head)
    # or per sequence ([B, tc, H, 128], one plan per (sequence, KV head))
    calib = np.ascontiguousarray(K[:, :tc]) if per_seq else K[:, :tc].reshape(B * tc, H, 128)
    # query-energy block weights w[h, j] (mean squared norm of block j over the queries of KV
    # head h's group, and over the batch unless plans are per sequence), an input of the allocation
    bw = None
    if query_weighted:
        qv = Q.astype(np.float64).reshape(B, H, w.group, 128)
        p0, p1 = al.block_pairs(128, pairing)
        e = qv[..., p0] ** 2 + qv[..., p1] ** 2
        bw = np.ascontiguousarray(np.mean(e, axis=2) if per_seq else np.mean(e, axis=(0, 2)))   # [(B,) H, 64]
    # the rotated codec's signs are drawn here and passed to both sides
    signs = (np.random.default_rng(7).choice([-1, 1], size=(H, 128)).astype(np.int8)
             if codec in ("rot", "bgtq_rot") else None)
    alloc = codec in ("bgtq", "bgtq_rot")     # widths from the allocation (calibration keys)
    if per_seq:
        ols = [OracleLayer(calib[b] if alloc else K[b, :1], k_bits, v_bits, codec, pairing,
                           b_min, b_max, block_weight=None if bw is None else bw[b], signs=signs)
               for b in range(B)]
        # the sequences' plans must really differ, or the case would not test the indexing
        assert B == 1 or not alloc or any(not np.array_equal(ols[0].widths, o.widths) for o in ols[1:])
    else:
        ols = [OracleLayer(calib if alloc else K[:, :1].reshape(B, H, 128), k_bits, v_bits,
                           codec, pairing, b_min, b_max, block_weight=bw, signs=signs)] * B

    cfg = kvq.Config(n_layers=1, n_kv_heads=H, n_q_heads=Hq, batch=B, max_tokens=T, k_bits=k_bits,
                     v_bits=v_bits, b_min=b_min, b_max=b_max, codec=CODEC[codec],
                     pairing=PAIRING[pairing], recent_window=recent, per_sequence_plans=int(per_seq))
    cache = kvq.Cache(cfg)
    dev = torch.device("cuda:0")
    cache.alloc_bits(0, torch.from_numpy(np.ascontiguousarray(calib)).to(dev) if alloc else None,
                     block_weight=torch.from_numpy(bw).to(dev) if bw is not None else None)
    if signs is not None:
        cache.set_rotation(0, signs)
    bits, gains = cache.get_plan(0)
    want_w = np.stack([o.widths for o in ols]) if per_seq else ols[0].widths
    want_g = np.stack([o.g for o in ols]) if per_seq else ols[0].g
    assert np.array_equal(bits, want_w), "plan widths differ"
    assert np.array_equal(gains.view(np.uint32), want_g.astype(np.float32).view(np.uint32)), "gains differ"

    bounds = [0, T] if chunks is None else [0, *np.cumsum(chunks).tolist()]
    assert bounds[-1] == T
    grp = 128 if codec == "kivi" else 1                   # KIVI packs whole key tiles only
    P = wn.packed_len(T, recent, grp)                     # packed positions
    # the rows each position is stored from (fp16 copies where it went through the window)
    Ke = np.stack([wn.stored_rows(K[b], bounds, recent, grp) for b in range(B)])
    Ve = np.stack([wn.stored_rows(V[b], bounds, recent, grp) for b in range(B)])
    Kt = torch.from_numpy(K).to(dev)
    Vt = torch.from_numpy(V).to(dev)
    for a, z in zip(bounds[:-1], bounds[1:]):
        cache.quantize_append(0, Kt[:, a:z].contiguous(), Vt[:, a:z].contiguous())
    assert cache.seq_len(0) == T

    sigma = 0.0
    refs = []
    for b in range(B):
        kh_all, vh_all, qo = [], [], []
        ol = ols[b]
        for h in range(H):
            kh = np.zeros((0, 128))
            vh = np.zeros((0, 128))
            r = None
            if P > 0:
                r = ol.quantize_head(Ke[b, :P, h], Ve[b, :P, h], h,
                                     Ke[b, :P].reshape(P, H * 128) if codec == "nf16" else None,
                                     Ve[b, :P].reshape(P, H * 128) if codec == "nf16" else None)
                kh, vh = ol.dequant(r, h)
            qo.append(r)
            # the recent window holds the fp16 values themselves
            kh_all.append(np.concatenate([kh, Ke[b, P:, h].astype(np.float64)]))
            vh_all.append(np.concatenate([vh, Ve[b, P:, h].astype(np.float64)]))
        refs.append((qo, np.stack(kh_all), np.stack(vh_all)))
    print(f"[{wname} T={T}] oracle quantized", flush=True)
    if temper:
        # choose sigma so that the logits' standard deviation is about 2 (softmax blends)
        qb = Q[0].astype(np.float64)
        lg = np.concatenate([refs[0][1][h // w.group] @ qb[h] for h in range(Hq)])
        sigma = float(2.0 / lg.std())

    info = cache.layer_info(0)
    cap = info.capacity
    if check_codes:
        kw = cache.read(0, kvq.PART_K_CODES, np.uint32).reshape(B, H, cap, info.k_row_words)
        vw = cache.read(0, kvq.PART_V_CODES, np.uint32).reshape(B, H, cap // 128, 512, info.v_dim_words // 4)
        kscale = cache.read(0, kvq.PART_K_SCALES, np.uint16)
        vscale = cache.read(0, kvq.PART_V_SCALES, np.uint16)
        if codec == "nf16":
            kscale = kscale.reshape(B, cap, -1)
            vscale = vscale.reshape(B, cap, -1)
        elif codec == "kivi":
            kscale = kscale.reshape(B, H, cap // 128, 64, 4)
            vscale = vscale.reshape(B, H, cap // 128, 2, 128)
        else:
            kscale = kscale.reshape(B, H, cap)
            vscale = vscale.reshape(B, H, cap)
        nt = (P + 127) // 128
        vb = 4 if codec == "nf16" else v_bits
        assert info.packed_len == P
        for b in range(B):
            for h in range(H):
                r = refs[b][0][h]
                if P == 0:
                    break
                rows = slice(None) if sample_rows is None else sample_rows
                assert np.array_equal(kw[b, h, :P][rows], r["k_words"][rows]), f"K words differ b={b} h={h}"
                assert np.array_equal(vw[b, h, :nt], lay.pack_v_tiles(r["v_codes"], vb)), f"V tiles differ b={b} h={h}"
                if codec == "nf16":
                    assert np.array_equal(kscale[b, :P], r["k_scale_blocks"].view(np.uint16))
                    assert np.array_equal(vscale[b, :P], r["v_scale_blocks"].view(np.uint16))
                elif codec == "kivi":
                    assert np.array_equal(kscale[b, h, :nt], r["k_params"].view(np.uint16)), f"K params b={b} h={h}"
                    assert np.array_equal(vscale[b, h, :nt], r["v_params"].view(np.uint16)), f"V params b={b} h={h}"
                else:
                    assert np.array_equal(kscale[b, h, :P], r["k_s16"].view(np.uint16)), f"K scales b={b} h={h}"
                    assert np.array_equal(vscale[b, h, :P], r["v_s16"].view(np.uint16)), f"V scales b={b} h={h}"
        ring = info.ring_slots          # R, or R + 128 with KIVI
        assert ring == recent + (128 if codec == "kivi" else 0)
        if ring > 0:
            kr = cache.read(0, kvq.PART_K_RECENT, np.float16).reshape(B, ring, H, 128)
            # values: dim-major 128-slot tiles [B][H][ring/128][128][128] -> [B][ring][H][128]
            vr = cache.read(0, kvq.PART_V_RECENT, np.float16).reshape(B, H, ring // 128, 128, 128)
            vr = vr.transpose(0, 2, 4, 1, 3).reshape(B, ring, H, 128)
            pos = np.arange(P, T)
            assert np.array_equal(kr[:, pos % ring].view(np.uint16), Ke[:, P:].astype(np.float16).view(np.uint16))
            assert np.array_equal(vr[:, pos % ring].view(np.uint16), Ve[:, P:].astype(np.float16).view(np.uint16))

    Qt = torch.from_numpy(Q).to(dev)
    out = cache.decode_attn(0, Qt, scale=sigma, n_splits=n_splits)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = np.stack([at.decode_attention(Q[b].astype(np.float64), refs[b][1], refs[b][2],
                                        sigma if sigma > 0 else None) for b in range(B)])
    res = assert_attention_close(got, ref, f"{wname} T={T} K{k_bits}V{v_bits} {codec}")
    if fidelity:
        mae, kl = cache.key_fidelity(0, Qt, Kt, scale=sigma)
        mae, kl = mae.cpu().numpy(), kl.cpu().numpy()
        for b in range(B):
            # the ABI takes the scale as fp32
            rm, rk = fd.logit_fidelity(Q[b], np.transpose(K[b], (1, 0, 2)), refs[b][1],
                                       float(np.float32(sigma)) if sigma > 0 else None)
            assert_fidelity_close(mae[b], rm, f"{wname} T={T} mae b={b}")
            assert_fidelity_close(kl[b], rk, f"{wname} T={T} kl b={b}")
    cache.close()
    return res


FID_REL, FID_ABS = 1e-9, 1e-12


def assert_fidelity_close(gpu, ref, what):
    err = np.abs(np.asarray(gpu) - ref)
    assert np.all(err <= FID_REL * np.abs(ref) + FID_ABS), f"{what}: max err {err.max():.3e} ref {ref}"


def test_tiny_end_to_end():
    w = WORKLOADS["tiny"]
    run_case("tiny", w.T, 4, 4)


def test_tiny_tempered_softmax():
    run_case("tiny", 1024, 4, 4, temper=True)


@pytest.mark.parametrize("pairing", ["half", "interleaved"])
def test_tiny_pairings(pairing):
    run_case("tiny", 700, 3, 2, pairing=pairing)


def test_single_token():
    run_case("tiny", 1, 4, 4)


def test_ragged_appends_cross_tiles():
    run_case("tiny", 1000, 3, 3, chunks=[100, 200, 37, 1, 662])


@pytest.mark.parametrize("kb,vb", [(2, 2), (3, 3), (4, 4)])
def test_llama_layer_budgets(kb, vb):
    run_case("llama8b_32k", 4096, kb, vb, temper=True)


@pytest.mark.parametrize("kb", [1, 5, 8])
def test_extreme_budgets(kb):
    run_case("llama8b_32k", 1000, kb, 8 if kb == 8 else 1)


def test_uniform_codec():
    run_case("llama8b_32k", 3000, 3, 3, codec="uniform", temper=True)


def test_nf16_codec_gauss_and_t5():
    run_case("llama8b_b64", 1500, 4, 4, codec="nf16", batch=3, temper=True)
    run_case("llama8b_b64", 1500, 4, 4, codec="nf16", batch=2, noise="t5", temper=True)


def test_bgtq_batched_t5():
    run_case("llama8b_b64", 2048, 4, 4, batch=4, noise="t5", temper=True)


def test_recent_window_ragged_appends():
    """fp16 recent window of 256 positions: evictions from the ring (with wrap), positions
    that arrive already outside the window, fp32 inputs rounded to fp16 in the window."""
    run_case("tiny", 1000, 3, 3, chunks=[100, 200, 37, 1, 662], recent=256)


def test_recent_window_holds_everything():
    run_case("tiny", 300, 4, 4, chunks=[299, 1], recent=512)


@pytest.mark.parametrize("n_splits", [0, 5])
def test_recent_window_qwen_k3v2(n_splits):
    """Qwen2.5-3B-shaped layer (8 query heads per KV head), asymmetric K3V2, 1024-position
    window, prefill then decode-sized appends."""
    run_case("qwen3b_128k", 20000, 3, 2, chunks=[2048, 17000, 951, 1], recent=1024, temper=True,
             n_splits=n_splits)


def test_recent_window_nf16():
    run_case("llama8b_32k", 3000, 4, 4, codec="nf16", chunks=[1000, 1999, 1], recent=128)


def test_asymmetric_k3v2_qwen_shape():
    """The paper's K3V2 setting (abstract), no recent window, on the Qwen2.5-3B shape."""
    run_case("qwen3b_128k", 20000, 3, 2, temper=True)


def test_query_weighted_allocation():
    """Block weights w_j = E |q_j|^2 from the decode queries, passed to the allocation."""
    run_case("llama8b_32k", 2000, 3, 3, query_weighted=True, temper=True)


@pytest.mark.parametrize("kb", [2, 3])
def test_rotated_uniform_codec(kb):
    """Uniform quantizer on randomly rotated keys (Hadamard rotation with caller signs)."""
    run_case("llama8b_32k", 3000, kb, kb, codec="rot", temper=True, chunks=[1000, 1999, 1])


def test_per_sequence_plans():
    """One plan per (sequence, KV head), each sequence with its own block profile."""
    run_case("llama8b_b64", 1500, 4, 4, batch=4, per_seq=True, temper=True, chunks=[700, 799, 1])


def test_per_sequence_plans_weighted_with_window():
    """Per-sequence plans with per-sequence query weights, a recent window and K3V3 (8 waves)."""
    run_case("qwen3b_128k", 3000, 3, 3, batch=3, per_seq=True, query_weighted=True, recent=512,
             chunks=[2048, 951, 1], temper=True)
    run_case("qwen3b_128k", 2500, 2, 2, batch=2, per_seq=True, n_splits=3, pairing="interleaved")


@pytest.mark.parametrize("kb,vb", [(2, 2), (3, 3), (4, 4), (4, 2)])
def test_kivi_codec(kb, vb):
    """KIVI-style asymmetric integers: whole key tiles from ring and input, the last partial
    tile in fp16."""
    run_case("llama8b_32k", 3000, kb, vb, codec="kivi", temper=True, chunks=[1000, 1999, 1])


def test_kivi_codec_window_and_tile_boundaries():
    """A recent window on top (ring of R + 128 slots), appends ending on and off tile
    boundaries, a context of exactly whole tiles, fp32 inputs, interleaved pairs."""
    run_case("qwen3b_128k", 5000, 3, 3, codec="kivi", chunks=[2048, 2951, 1], recent=256, temper=True)
    run_case("qwen3b_128k", 1024, 2, 2, codec="kivi", chunks=[128, 640, 256], n_splits=3)
    run_case("qwen3b_128k", 300, 3, 3, codec="kivi", chunks=[100, 27, 1, 172], recent=128)
    run_case("tiny", 1000, 4, 4, codec="kivi", chunks=[127, 1, 500, 372], pairing="interleaved")


@pytest.mark.parametrize("kb,noise", [(2, "gauss"), (3, "t5"), (4, "gauss")])
def test_bgtq_group_rotation(kb, noise):
    """Block-GTQ with rotations inside equal-width groups: codes bit-exact, decode and
    fidelity to the usual bars."""
    run_case("llama8b_32k", 3000, kb, kb, codec="bgtq_rot", temper=True, chunks=[1000, 1999, 1], noise=noise)


def test_bgtq_group_rotation_window_and_limits():
    run_case("qwen3b_128k", 5000, 3, 3, codec="bgtq_rot", chunks=[2048, 2951, 1], recent=256, temper=True)
    run_case("qwen3b_128k", 2000, 3, 3, codec="bgtq_rot", b_min=2, b_max=4, pairing="interleaved", n_splits=2)
    run_case("tiny", 1000, 4, 4, codec="bgtq_rot", zero_blocks=(1, 2))


def test_codec_combinations():
    """Per-sequence plans under the group rotation; the KIVI-style codec over a batch with a
    window; the group rotation with fp32 inputs over several appends."""
    run_case("llama8b_b64", 1500, 3, 3, codec="bgtq_rot", batch=3, per_seq=True, chunks=[1000, 499, 1], temper=True)
    run_case("llama8b_b64", 1000, 2, 4, codec="kivi", batch=3, per_seq=True, chunks=[300, 700], recent=128)
    run_case("tiny", 1000, 3, 3, codec="bgtq_rot", chunks=[1, 126, 873])


def test_rotated_uniform_codec_recent_window():
    run_case("qwen3b_128k", 5000, 3, 3, codec="rot", chunks=[2048, 2951, 1], recent=256)


def test_zero_energy_blocks():
    """Blocks that are zero in every key get zero energy, no bits and a zero gain."""
    run_case("llama8b_32k", 1500, 3, 3, zero_blocks=(0, 5, 63), temper=True)


def test_largest_recent_window():
    run_case("qwen3b_128k", 6000, 3, 3, chunks=[2048, 3951, 1], recent=4096)


def test_b_min_b_max_limits():
    run_case("llama8b_32k", 600, 3, 3, b_min=1, b_max=5)


def test_split_count_invariance_and_determinism():
    torch = _torch()
    kvq = _kvq()
    w = WORKLOADS["qwen3b_128k"]
    T = 5000
    k, v = gen_layer(w, 0, 0, T)
    q = gen_query(w, 0, T)
    cache = kvq.Cache(kvq.Config(1, w.n_kv, w.n_q, 1, T, 3, 3))
    dev = torch.device("cuda:0")
    cache.alloc_bits(0, torch.from_numpy(k[:2048]).to(dev))
    cache.quantize_append(0, torch.from_numpy(k[None]).to(dev), torch.from_numpy(v[None]).to(dev))
    qt = torch.from_numpy(q[None]).to(dev)
    outs = [cache.decode_attn(0, qt, n_splits=s).cpu().numpy() for s in (1, 2, 7, 40)]
    for o in outs[1:]:
        assert np.allclose(o, outs[0], rtol=2e-6, atol=2e-6)
    a = cache.decode_attn(0, qt).cpu().numpy()
    b = cache.decode_attn(0, qt).cpu().numpy()
    assert np.array_equal(a, b)
    cache.close()


def test_error_states():
    torch = _torch()
    kvq = _kvq()
    dev = torch.device("cuda:0")
    cache = kvq.Cache(kvq.Config(2, 2, 16, 1, 300, 3, 3))
    x = torch.zeros(1, 10, 2, 128, dtype=torch.float16, device=dev)
    q = torch.zeros(1, 16, 128, dtype=torch.float16, device=dev)
    with pytest.raises(kvq.KvqError) as e:
        cache.quantize_append(0, x, x)                       # no plan yet
    assert e.value.status == kvq.KVQ_ESTATE
    with pytest.raises(kvq.KvqError) as e:
        cache.alloc_bits(0, torch.zeros(0, 2, 128, dtype=torch.float16, device=dev))
    assert e.value.status == kvq.KVQ_EINVAL
    cache.alloc_bits(0, torch.randn(64, 2, 128, device=dev).half())
    with pytest.raises(kvq.KvqError) as e:
        cache.decode_attn(0, q)                               # empty layer
    assert e.value.status == kvq.KVQ_ESTATE
    st = torch.zeros(2, dtype=torch.float64, device=dev)
    assert kvq.lib.kvq_key_fidelity(cache.handle, 0, q.data_ptr(), x.data_ptr(), kvq.KVQ_F16, 0.0,
                                    st.data_ptr(), st.data_ptr(), None) == kvq.KVQ_ESTATE   # empty layer
    cache.quantize_append(0, x[:, :0].contiguous(), x[:, :0].contiguous())   # n_new = 0 is a no-op
    assert cache.seq_len(0) == 0
    cache.quantize_append(0, x, x)
    with pytest.raises(kvq.KvqError) as e:
        cache.alloc_bits(0, torch.randn(64, 2, 128, device=dev).half())   # re-alloc after append
    assert e.value.status == kvq.KVQ_ESTATE
    big = torch.zeros(1, 291, 2, 128, dtype=torch.float16, device=dev)
    with pytest.raises(kvq.KvqError) as e:
        cache.quantize_append(0, big, big)                    # 10 + 291 > 300
    assert e.value.status == kvq.KVQ_ECAPACITY
    assert cache.seq_len(0) == 10
    with pytest.raises(kvq.KvqError) as e:
        cache.decode_attn(5, q)
    assert e.value.status == kvq.KVQ_EINVAL
    out = cache.decode_attn(0, q)
    assert torch.isfinite(out).all()
    raw = torch.zeros(1 * 10 * 2 * 128 + 1, dtype=torch.float16, device=dev)
    assert kvq.lib.kvq_key_fidelity(cache.handle, 0, q.data_ptr(), raw.data_ptr() + 2, kvq.KVQ_F16, 0.0,
                                    out.data_ptr(), out.data_ptr(), None) == kvq.KVQ_EINVAL   # misaligned keys
    mae, kl = cache.key_fidelity(0, q, x)
    assert torch.isfinite(mae).all() and torch.isfinite(kl).all()
    cache.close()


def test_codec_error_states():
    """Rotation signs: required before the first append, only +-1, only for rotating codecs,
    not after an append.  KIVI below one tile: everything in fp16, decode still works."""
    torch = _torch()
    kvq = _kvq()
    dev = torch.device("cuda:0")
    x = torch.randn(1, 200, 2, 128, device=dev).half()
    q = torch.randn(1, 16, 128, device=dev).half()
    rc = kvq.Cache(kvq.Config(1, 2, 16, 1, 300, 3, 3, codec=kvq.CODEC_BGTQ_ROT))
    rc.alloc_bits(0, x[0, :64].contiguous())
    with pytest.raises(kvq.KvqError) as e:
        rc.quantize_append(0, x, x)                           # no signs yet
    assert e.value.status == kvq.KVQ_ESTATE
    bad = np.ones((2, 128), np.int8)
    bad[1, 7] = 2
    with pytest.raises(kvq.KvqError) as e:
        rc.set_rotation(0, bad)
    assert e.value.status == kvq.KVQ_EINVAL
    rc.set_rotation(0, np.ones((2, 128), np.int8))
    rc.quantize_append(0, x, x)
    with pytest.raises(kvq.KvqError) as e:
        rc.set_rotation(0, np.ones((2, 128), np.int8))         # after an append
    assert e.value.status == kvq.KVQ_ESTATE
    assert torch.isfinite(rc.decode_attn(0, q)).all()
    rc.close()
    bc = kvq.Cache(kvq.Config(1, 2, 16, 1, 300, 3, 3))
    with pytest.raises(kvq.KvqError) as e:
        bc.set_rotation(0, np.ones((2, 128), np.int8))         # codec does not rotate
    assert e.value.status == kvq.KVQ_EINVAL
    bc.close()
    pc = kvq.Cache(kvq.Config(1, 2, 16, 2, 300, 3, 3, per_sequence_plans=1))
    with pytest.raises(ValueError):
        pc.alloc_bits(0, x[0, :64].contiguous())             # needs [batch, n_tok, heads, dim]
    pc.close()
    kc = kvq.Cache(kvq.Config(1, 2, 16, 1, 300, 2, 2, codec=kvq.CODEC_KIVI))
    kc.alloc_bits(0)
    kc.quantize_append(0, x[:, :100].contiguous(), x[:, :100].contiguous())
    info = kc.layer_info(0)
    assert info.packed_len == 0 and info.ring_slots == 128 and info.len == 100
    assert torch.isfinite(kc.decode_attn(0, q)).all()
    kc.close()


def test_headline_layer_full_size():
    """Qwen2.5-3B-shaped layer at 131072 tokens, K3V3: sampled K rows, all V tiles and
    scales bit-exact; decode (auto split count, as benchmarked) vs fp64 oracle."""
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(131072, 4096, replace=False))
    run_case("qwen3b_128k", 131072, 3, 3, layer=5, sample_rows=rows)


def test_kivi_codec_full_size():
    """The KIVI-style codec at the headline shape (131072 positions, K3V3): 1024 key tiles."""
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(131072, 4096, replace=False))
    run_case("qwen3b_128k", 131072, 3, 3, codec="kivi", layer=5, sample_rows=rows)


@pytest.mark.timeout(600)
def test_longest_context_layer_full_size():
    """512K context, K2V2, one layer; decode with the automatic split-K."""
    run_case("qwen3b_512k", 524288, 2, 2, layer=0, check_codes=False)
