"""GPU (HIP, gfx950) vs oracle parity through the C ABI.

Plans, codes, packed words and scales must be bit-exact; decode attention
must match the oracle's fp64 attention over its own dequantized cache within
max-abs 2e-3 and relative L2 1e-3.  The key-fidelity diagnostics (fp64 on both
sides, the same exact products, sums in another order) must match the oracle's
within 1e-9 relative + 1e-12 absolute.
"""
import concurrent.futures
import os

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


def _gen_batch(w, layer, T, B, noise, pairing, per_seq):
    """Keys, values [B, T, H, d] and queries [B, Hq, d] of every sequence (threads: the
    generator's numpy work releases the interpreter lock)."""
    def one(b):
        sig = seq_block_sigmas(w, layer, b) if per_seq else None
        k, v = gen_layer(w, layer, 0, T, seq=b, noise=noise, pairing=pairing, sigmas=sig)
        return k, v, gen_query(w, layer, T, seq=b, noise=noise, pairing=pairing, sigmas=sig)
    with concurrent.futures.ThreadPoolExecutor(min(8, B)) as ex:
        res = list(ex.map(one, range(B)))
    return (np.stack([r[0] for r in res]), np.stack([r[1] for r in res]), np.stack([r[2] for r in res]))


def run_case(wname, T, k_bits, v_bits, codec="bgtq", pairing="half", batch=None, layer=0,
             chunks=None, n_splits=0, noise="gauss", temper=False, check_codes=True, sample_rows=None,
             b_min=0, b_max=8, fidelity=True, recent=0, query_weighted=False, zero_blocks=(),
             per_seq=False, sample_seqs=None, steps=0):
    """Quantize T tokens of one layer on the GPU and in the oracle; compare everything.

    recent > 0: the last `recent` positions stay in the fp16 window.  A position that was inside
    the window at the end of its append went through fp16 (fp32 inputs are rounded), and the
    packed storage holds positions 0 .. T - recent - 1.

    per_seq: every sequence draws its own block profile and gets plans of its own from its own
    calibration keys (and its own query-energy weights).

    sample_seqs: the GPU runs the whole batch; the oracle quantizes, and the comparisons cover,
    only these sequences (the plan is still compared in full).

    steps > 0: the last `steps` positions arrive one at a time through decode_step (append, then
    attend), on this cache and, as append + decode_attn, on a twin cache: every step's output
    and, at the end, every stored byte must be equal between the two."""
    torch = _torch()
    kvq = _kvq()
    w = WORKLOADS[wname]
    B = w.batch if batch is None else batch
    H, Hq = w.n_kv, w.n_q
    seqs = list(range(B)) if sample_seqs is None else list(sample_seqs)
    assert not (per_seq and sample_seqs is not None)
    K, V, Q = _gen_batch(w, layer, T, B, noise, pairing, per_seq)   # [B, T, H, d], [B, Hq, d]
    if zero_blocks:
        # degenerate blocks: both coordinates zero in every key (zero energy, zero gain)
        p0, p1 = al.block_pairs(128, pairing)
        for j in zero_blocks:
            K[..., p0[j]] = 0
            K[..., p1[j]] = 0
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

    T0 = T - steps
    bounds = [0, T0] if chunks is None else [0, *np.cumsum(chunks).tolist()]
    assert bounds[-1] == T0
    bounds += list(range(T0 + 1, T + 1))
    grp = 128 if codec == "kivi" else 1                   # KIVI packs whole key tiles only
    P = wn.packed_len(T, recent, grp)                     # packed positions
    # the rows each position is stored from (fp16 copies where it went through the window)
    Ke = {b: wn.stored_rows(K[b], bounds, recent, grp) for b in seqs}
    Ve = {b: wn.stored_rows(V[b], bounds, recent, grp) for b in seqs}
    Kt = torch.from_numpy(K).to(dev)
    Vt = torch.from_numpy(V).to(dev)
    twin = None
    if steps:
        twin = kvq.Cache(cfg)
        twin.alloc_bits(0, torch.from_numpy(np.ascontiguousarray(calib)).to(dev) if alloc else None,
                        block_weight=torch.from_numpy(bw).to(dev) if bw is not None else None)
        if signs is not None:
            twin.set_rotation(0, signs)
    for a, z in zip(bounds[:-1], bounds[1:]):
        if a >= T0:
            break
        cache.quantize_append(0, Kt[:, a:z].contiguous(), Vt[:, a:z].contiguous())
        if twin is not None:
            twin.quantize_append(0, Kt[:, a:z].contiguous(), Vt[:, a:z].contiguous())
    if steps:
        Qd = torch.from_numpy(Q).to(dev)
        for st in range(steps):
            p = T0 + st
            qs = torch.roll(Qd, st, dims=1).contiguous()   # a different query for every step
            got_s = cache.decode_step(0, Kt[:, p].contiguous(), Vt[:, p].contiguous(), qs)
            twin.quantize_append(0, Kt[:, p:p + 1].contiguous(), Vt[:, p:p + 1].contiguous())
            want_s = twin.decode_attn(0, qs)
            torch.cuda.synchronize()
            assert torch.equal(got_s, want_s), f"decode_step output differs from append + decode at position {p}"
        for part, dt in ((kvq.PART_K_CODES, np.uint32), (kvq.PART_V_CODES, np.uint32),
                         (kvq.PART_K_SCALES, np.uint16), (kvq.PART_V_SCALES, np.uint16)):
            assert np.array_equal(cache.read(0, part, dt), twin.read(0, part, dt)), f"decode_step storage differs: part {part}"
        if recent:
            for part in (kvq.PART_K_RECENT, kvq.PART_V_RECENT):
                assert np.array_equal(cache.read(0, part, np.uint16), twin.read(0, part, np.uint16))
        twin.close()
        print(f"[{wname} T={T}] {steps} decode steps equal to append + decode", flush=True)
    assert cache.seq_len(0) == T

    sigma = 0.0
    refs = {}
    for b in seqs:
        kh_all, vh_all, qo = [], [], []
        ol = ols[b]
        for h in range(H):
            kh = np.zeros((0, 128))
            vh = np.zeros((0, 128))
            r = None
            if P > 0:
                r = ol.quantize_head(Ke[b][:P, h], Ve[b][:P, h], h,
                                     Ke[b][:P].reshape(P, H * 128) if codec == "nf16" else None,
                                     Ve[b][:P].reshape(P, H * 128) if codec == "nf16" else None)
                kh, vh = ol.dequant(r, h)
            qo.append(r)
            # the recent window holds the fp16 values themselves
            kh_all.append(np.concatenate([kh, Ke[b][P:, h].astype(np.float64)]))
            vh_all.append(np.concatenate([vh, Ve[b][P:, h].astype(np.float64)]))
        refs[b] = (qo, np.stack(kh_all), np.stack(vh_all))
    print(f"[{wname} T={T}] oracle quantized", flush=True)
    if temper:
        # choose sigma so that the logits' standard deviation is about 2 (softmax blends)
        b0 = seqs[0]
        qb = Q[b0].astype(np.float64)
        lg = np.concatenate([refs[b0][1][h // w.group] @ qb[h] for h in range(Hq)])
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
        for b in seqs:
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
            for b in seqs:
                assert np.array_equal(kr[b, pos % ring].view(np.uint16), Ke[b][P:].astype(np.float16).view(np.uint16))
                assert np.array_equal(vr[b, pos % ring].view(np.uint16), Ve[b][P:].astype(np.float16).view(np.uint16))

    Qt = torch.from_numpy(Q).to(dev)
    out = cache.decode_attn(0, Qt, scale=sigma, n_splits=n_splits)
    torch.cuda.synchronize()
    got = out.cpu().numpy()[seqs]
    ref = np.stack([at.decode_attention(Q[b].astype(np.float64), refs[b][1], refs[b][2],
                                        sigma if sigma > 0 else None) for b in seqs])
    res = assert_attention_close(got, ref, f"{wname} T={T} K{k_bits}V{v_bits} {codec}")
    if fidelity:
        mae, kl = cache.key_fidelity(0, Qt, Kt, scale=sigma)
        mae, kl = mae.cpu().numpy(), kl.cpu().numpy()
        for b in seqs:
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


def test_decode_step_appends():
    """Decode-sized appends (one to four positions per call, the latency path) after a prefill,
    crossing 32-position V segments and 128-position tiles; fp32 and fp16 inputs, per-sequence
    plans, the uniform codec; codes bit-exact and decode to the usual bar."""
    run_case("tiny", 400, 3, 3, chunks=[300] + [1] * 50 + [2, 3, 4] * 5 + [5])
    run_case("llama8b_b64", 600, 4, 3, batch=3, per_seq=True, chunks=[500] + [1] * 30 + [3] * 10 + [4] * 10,
             temper=True)
    run_case("llama8b_32k", 700, 2, 2, codec="uniform", chunks=[600] + [1] * 100)


def test_decode_step_fused_append():
    """decode_step (the new position quantized inside the decode launch) against append +
    decode_attn: outputs of every step and all stored bytes equal, then codes and the final
    decode against the oracle.  Steps cross 32-position V segments and 128-position tiles; one
    query head per KV head (fp32), 8 (two waves per SIMD), 4 with per-sequence plans, the uniform
    codec, value widths 2 and 5 (codes straddling words), and the paths that fall back to two
    calls (recent window, 256-value codec)."""
    run_case("tiny", 300, 3, 3, chunks=[100, 26], steps=174)
    run_case("qwen3b_128k", 2100, 3, 3, chunks=[2040], steps=60, temper=True)
    run_case("llama8b_b64", 700, 4, 3, batch=3, per_seq=True, chunks=[630], steps=70, temper=True)
    run_case("llama8b_32k", 400, 2, 2, codec="uniform", chunks=[380], steps=20)
    run_case("llama8b_32k", 300, 3, 5, chunks=[250], steps=50, temper=True)
    run_case("tiny", 400, 3, 3, chunks=[300], steps=100, recent=128)
    run_case("llama8b_32k", 600, 4, 4, codec="nf16", chunks=[590], steps=10)
    run_case("gqa2_8k", 700, 3, 3, chunks=[650], steps=50, temper=True)   # two query heads per KV head


def test_decode_step_from_empty_cache():
    """Every position through decode_step, from an empty cache: the first launches have one
    split and one partly filled tile (the appended position is its last), then the splits grow
    past the first tiles; outputs and stored bytes equal to append + decode_attn at every step."""
    run_case("tiny", 200, 3, 3, steps=200)
    run_case("qwen3b_128k", 300, 3, 3, steps=300, temper=True)


def test_decode_step_fused_append_separate_merge():
    """32 sequences x 8 KV heads = 256 (sequence, head) units: the decode step's launch is followed by
    the separate merge kernel."""
    run_case("llama8b_b64", 400, 3, 3, batch=32, chunks=[380], steps=20, sample_seqs=(0, 17, 31))


def test_decode_step_fused_append_full_size():
    """The headline layer (Qwen2.5-3B shape, K3V3) grown to 131072 positions by decode steps
    from 131000: the fused launch at the bench's full size and split count."""
    run_case("qwen3b_128k", 131072, 3, 3, layer=5, chunks=[2048, 128952], steps=72)


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


def test_several_tiles_per_wave():
    """Launches whose waves walk several 128-position tiles (few splits over many tiles): each
    later tile's K rows, scales and V words are loaded inside the tile loop.  Block-GTQ with a
    window and a one-position last append, the KIVI-style codec, the 256-value codec at four
    query heads per KV head over a batch, and one split per head (no merge) with a ragged last
    tile."""
    run_case("qwen3b_128k", 6000, 3, 3, chunks=[2048, 3951, 1], n_splits=2, recent=256, temper=True)
    run_case("qwen3b_128k", 5000, 3, 3, codec="kivi", chunks=[2048, 2952], n_splits=2)
    run_case("llama8b_b64", 3000, 4, 4, codec="nf16", batch=2, n_splits=1, temper=True)
    run_case("llama8b_32k", 4000, 2, 2, n_splits=1)

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


def _boundary_rows(bits, rng):
    """fp32 rows whose scale is exactly 1 (so u = x) and which hold every boundary of the width,
    and the fp32 numbers just above and below it: ties take the lower code."""
    from oracle import codebooks as cbk
    from oracle import quantize as qz
    bd = cbk.boundaries(bits)[: 2 ** bits - 1].astype(np.float32)
    probes = np.concatenate([bd, np.nextafter(bd, np.float32(np.inf)), np.nextafter(bd, np.float32(-np.inf)),
                             np.float32([0.0, -0.0])])
    probes = probes[rng.permutation(len(probes))]
    rows, i = [], 0
    while i < len(probes):
        row = np.zeros(128, np.float32)
        n = 0
        while i < len(probes) and n < 100 and float(np.sum(row[:n].astype(np.float64) ** 2) + probes[i] ** 2) < 90.0:
            row[n] = probes[i]
            n += 1
            i += 1
        energy = float(np.sum(row[:n].astype(np.float64) ** 2))
        row[n:] = np.float32(np.sqrt((128.0 - energy) / (128 - n)))
        row = row[rng.permutation(128)]
        # the oracle's scale of the row must be exactly 1 (then u = x exactly)
        s16, _ = qz.row_scale(row[None])
        assert s16[0] == np.float16(1.0), s16
        rows.append(row)
    return np.stack(rows)


@pytest.mark.parametrize("kb,vb", [(2, 8), (3, 3), (8, 5), (5, 1)])
def test_codes_on_boundaries(kb, vb):
    """Values exactly on a boundary, and one fp32 step on either side, in rows of scale 1 (the
    uniform codec, fp32 input): codes bit-exact against the oracle through the many-position
    append, the few-position append and the decode step."""
    torch = _torch()
    kvq = _kvq()
    rng = np.random.default_rng(11 + kb + 10 * vb)
    Kr = _boundary_rows(kb, rng)
    Vr = _boundary_rows(vb, rng)
    N = max(len(Kr), len(Vr)) + 40
    pad = lambda x: np.concatenate([x, x[rng.integers(0, len(x), N - len(x))]])   # noqa: E731
    Kr, Vr = pad(Kr), pad(Vr)
    dev = torch.device("cuda:0")
    cache = kvq.Cache(kvq.Config(n_layers=1, n_kv_heads=1, n_q_heads=1, batch=1, max_tokens=N, k_bits=kb,
                                 v_bits=vb, codec=CODEC["uniform"]))
    cache.alloc_bits(0, None)
    Kt = torch.from_numpy(Kr[None, :, None]).to(dev)   # [1, N, 1, 128] fp32
    Vt = torch.from_numpy(Vr[None, :, None]).to(dev)
    q = torch.zeros(1, 1, 128, dtype=torch.float32, device=dev)
    n_bulk = N - 12
    cache.quantize_append(0, Kt[:, :n_bulk].contiguous(), Vt[:, :n_bulk].contiguous())
    for p in range(n_bulk, N - 6):
        cache.quantize_append(0, Kt[:, p:p + 1].contiguous(), Vt[:, p:p + 1].contiguous())
    for p in range(N - 6, N):
        cache.decode_step(0, Kt[:, p].contiguous(), Vt[:, p].contiguous(), q)
    torch.cuda.synchronize()
    ol = OracleLayer(np.zeros((1, 1, 128)), kb, vb, "uniform")
    r = ol.quantize_head(Kr.astype(np.float32), Vr.astype(np.float32), 0)
    assert np.all(r["k_s16"].view(np.uint16) == 0x3C00) and np.all(r["v_s16"].view(np.uint16) == 0x3C00)
    info = cache.layer_info(0)
    kw = cache.read(0, kvq.PART_K_CODES, np.uint32).reshape(info.capacity, info.k_row_words)[:N]
    vw = cache.read(0, kvq.PART_V_CODES, np.uint32).reshape(info.capacity // 128, 512, vb)[:(N + 127) // 128]
    assert np.array_equal(kw, r["k_words"]), "K words differ"
    assert np.array_equal(vw, lay.pack_v_tiles(r["v_codes"], vb)), "V tiles differ"
    cache.close()


def test_decode_step_error_states():
    """kvq_decode_step validates like the two calls it stands for and appends nothing on an error:
    no plan, a full cache, misaligned rows or output, a NaN scale, a bad layer."""
    torch = _torch()
    kvq = _kvq()
    dev = torch.device("cuda:0")
    cache = kvq.Cache(kvq.Config(1, 2, 16, 1, 130, 3, 3))
    q = torch.randn(1, 16, 128, device=dev).half()
    row = torch.randn(1, 2, 128, device=dev).half()
    with pytest.raises(kvq.KvqError) as e:
        cache.decode_step(0, row, row, q)                      # no plan yet
    assert e.value.status == kvq.KVQ_ESTATE
    cache.alloc_bits(0, torch.randn(64, 2, 128, device=dev).half())
    out = cache.decode_step(0, row, row, q)                    # the first position, one launch
    assert cache.seq_len(0) == 1 and torch.isfinite(out).all()
    raw = torch.zeros(2 * 128 + 8, dtype=torch.float16, device=dev)
    h = cache.handle
    assert kvq.lib.kvq_decode_step(h, 0, raw.data_ptr() + 2, row.data_ptr(), q.data_ptr(), kvq.KVQ_F16, 0.0,
                                   out.data_ptr(), None) == kvq.KVQ_EINVAL            # misaligned k_new
    assert kvq.lib.kvq_decode_step(h, 0, row.data_ptr(), row.data_ptr(), q.data_ptr(), kvq.KVQ_F16, 0.0,
                                   out.data_ptr() + 4, None) == kvq.KVQ_EINVAL        # misaligned out
    assert kvq.lib.kvq_decode_step(h, 0, row.data_ptr(), row.data_ptr(), q.data_ptr(), kvq.KVQ_F16,
                                   float("nan"), out.data_ptr(), None) == kvq.KVQ_EINVAL
    assert kvq.lib.kvq_decode_step(h, 3, row.data_ptr(), row.data_ptr(), q.data_ptr(), kvq.KVQ_F16, 0.0,
                                   out.data_ptr(), None) == kvq.KVQ_EINVAL            # bad layer
    assert kvq.lib.kvq_decode_step(h, 0, None, row.data_ptr(), q.data_ptr(), kvq.KVQ_F16, 0.0,
                                   out.data_ptr(), None) == kvq.KVQ_EINVAL
    assert cache.seq_len(0) == 1                                # nothing appended by the failures
    for _ in range(129):
        cache.decode_step(0, row, row, q)
    assert cache.seq_len(0) == 130
    with pytest.raises(kvq.KvqError) as e:
        cache.decode_step(0, row, row, q)                      # full
    assert e.value.status == kvq.KVQ_ECAPACITY
    assert cache.seq_len(0) == 130
    with pytest.raises(ValueError):
        cache.decode_step(0, row.float(), row, q)               # dtype differs from q's
    torch.cuda.synchronize()
    assert torch.isfinite(cache.decode_attn(0, q)).all()
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
    """Qwen2.5-3B-shaped layer at 131072 tokens, K3V3: every K row, V tile and scale
    bit-exact; decode (auto split count, as benchmarked) vs fp64 oracle."""
    run_case("qwen3b_128k", 131072, 3, 3, layer=5)


def test_kivi_codec_full_size():
    """The KIVI-style codec at the headline shape (131072 positions, K3V3): 1024 key tiles."""
    run_case("qwen3b_128k", 131072, 3, 3, codec="kivi", layer=5)


@pytest.mark.timeout(600)
def test_longest_context_layer_full_size():
    """512K context, K2V2, one layer: every K row, V tile and scale bit-exact; decode with the
    automatic split-K."""
    run_case("qwen3b_512k", 524288, 2, 2, layer=0)


# sequences of the batch-64 shape the oracle checks one by one (first, last and a spread)
C5_SAMPLE = (0, 1, 22, 41, 63)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("codec,noise", [("bgtq", "gauss"), ("bgtq", "t5"), ("nf16", "gauss"), ("nf16", "t5")])
def test_batched_decode_full_shape(codec, noise):
    """The batch-64 x 8192 Llama-shaped K4V4 decode at its full size and in the launch the bench
    times (automatic split count: one split per (sequence, KV head), direct output at G = 4),
    for Block-GTQ and the 256-value absmax codec, Gaussian and Student-t(5) inputs.  The plan
    (from all 64 sequences' calibration keys) is compared in full; codes, scales and decode
    outputs of sampled sequences."""
    run_case("llama8b_b64", 8192, 4, 4, codec=codec, noise=noise, sample_seqs=C5_SAMPLE,
             temper=noise == "t5")


@pytest.mark.parametrize("recent,n_splits", [(0, 0), (512, 3)])
def test_two_query_heads_per_kv_head(recent, n_splits):
    """Grouped-query ratio 2 (4 KV heads, 8 query heads)."""
    run_case("gqa2_8k", 8192, 3, 3, temper=True, recent=recent, n_splits=n_splits, chunks=[2048, 6143, 1])


def test_llama_layer_full_context():
    """One Llama-3.1-8B-shaped layer at its full 32768 positions, K3V3 (auto splits)."""
    run_case("llama8b_32k", 32768, 3, 3, temper=True)


@pytest.mark.parametrize("kb", [2, 4])
def test_uniform_codec_budgets(kb):
    run_case("llama8b_32k", 4096, kb, kb, codec="uniform", temper=True)


@pytest.mark.parametrize("vb", [5, 6, 7])
def test_wide_value_widths(vb):
    run_case("llama8b_32k", 1000, 3, vb, temper=True, chunks=[500, 499, 1])


def test_as_many_units_as_compute_units_with_window():
    """32 sequences x 8 KV heads = 256 (sequence, head) units with a recent window: the packed
    split and the window tile of each unit are merged by the separate merge kernel."""
    run_case("llama8b_b64", 1024, 4, 4, batch=32, recent=128, chunks=[896, 127, 1], temper=True)
    run_case("llama8b_b64", 1024, 3, 2, batch=40, recent=256, sample_seqs=(0, 17, 39))


def _hip_copy_to_host(dev_ptr, nbytes):
    """hipMemcpy through the HIP runtime's C API (no torch tensor wraps the library's memory)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.restype = ctypes.c_int
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    buf = np.empty(nbytes, dtype=np.uint8)
    assert hip.hipMemcpy(buf.ctypes.data, dev_ptr, nbytes, 2) == 0    # device to host
    return buf


def test_cache_view_reads_the_storage_in_place():
    torch = _torch()
    kvq = _kvq()
    w = WORKLOADS["qwen3b_128k"]
    T = 3000
    k, v = gen_layer(w, 1, 0, T)
    dev = torch.device("cuda:0")
    cache = kvq.Cache(kvq.Config(2, w.n_kv, w.n_q, 1, 4096, 3, 3, recent_window=256))
    for layer in (0, 1):
        cache.alloc_bits(layer, torch.from_numpy(k[:2048]).to(dev))
        cache.quantize_append(layer, torch.from_numpy(k[None]).to(dev), torch.from_numpy(v[None]).to(dev))
    torch.cuda.synchronize()
    v0, v1 = cache.view(0), cache.view(1)
    info = cache.layer_info(1)
    assert v1.len == T and v1.packed_len == info.packed_len == T - 256 and v1.capacity == info.capacity
    assert v1.k_codes - v0.k_codes == info.k_codes_bytes and v1.v_codes - v0.v_codes == info.v_codes_bytes
    cap, kw = info.capacity, info.k_row_words
    assert tuple(v1.k_codes_strides) == (w.n_kv * cap * kw, cap * kw, kw)
    assert tuple(v1.scale_strides) == (w.n_kv * cap, cap, 1)
    # every part read through the view equals the synchronizing dump
    for ptr, part, nbytes in ((v1.k_codes, kvq.PART_K_CODES, info.k_codes_bytes),
                              (v1.v_codes, kvq.PART_V_CODES, info.v_codes_bytes),
                              (v1.k_scales, kvq.PART_K_SCALES, info.k_scales_bytes),
                              (v1.v_scales, kvq.PART_V_SCALES, info.v_scales_bytes),
                              (v1.k_recent, kvq.PART_K_RECENT, info.recent_bytes),
                              (v1.v_recent, kvq.PART_V_RECENT, info.recent_bytes)):
        assert np.array_equal(_hip_copy_to_host(ptr, nbytes), cache.read(1, part, np.uint8))
    # the plan records: block widths, gains and field order as the host copy and the oracle give them
    assert v1.n_plans == w.n_kv and v1.plan_bytes == kvq.PLAN_BYTES
    raw = _hip_copy_to_host(v1.plans, v1.n_plans * v1.plan_bytes).reshape(v1.n_plans, v1.plan_bytes)
    bits, gains = cache.get_plan(1)
    ol = OracleLayer(k[:2048], 3, 3)
    for h in range(w.n_kv):
        rec = raw[h]
        bw = rec[kvq.PLAN_OFF_BLOCK_WIDTH:kvq.PLAN_OFF_BLOCK_WIDTH + 64].view(np.int8)
        assert np.array_equal(bw, bits[h]) and np.array_equal(bw, ol.widths[h])
        g = rec[kvq.PLAN_OFF_GAIN:kvq.PLAN_OFF_GAIN + 512].view(np.float32)
        assert np.array_equal(g[:64], gains[h])
        nf = int(rec[kvq.PLAN_OFF_N_FIELDS:kvq.PLAN_OFF_N_FIELDS + 4].view(np.int32)[0])
        dims, ws = ol.fields(h)
        assert nf == len(dims)
        assert np.array_equal(rec[kvq.PLAN_OFF_FIELD_DIM:kvq.PLAN_OFF_FIELD_DIM + nf], dims)
        assert np.array_equal(rec[kvq.PLAN_OFF_FIELD_WIDTH:kvq.PLAN_OFF_FIELD_WIDTH + nf], ws)
    cache.close()


@pytest.mark.parametrize("batch", [1, 32])
def test_merge_that_gives_up_is_reported(batch):
    """A split merger whose bounded wait gives up (bound set to zero polls from the host, so every
    kernel still ends at once) writes NaN and sets the device status word; kvq_cache_status
    reports it once and clears it.  batch 1: mergers inside the decode kernel; batch 32 x 8 KV
    heads with a window: the separate merge kernel."""
    torch = _torch()
    kvq = _kvq()
    dev = torch.device("cuda:0")
    wname = "qwen3b_128k" if batch == 1 else "llama8b_b64"
    w = WORKLOADS[wname]
    T = 5000 if batch == 1 else 600
    recent = 0 if batch == 1 else 128
    k, v = gen_layer(w, 0, 0, T)
    K = torch.from_numpy(np.repeat(k[None], batch, axis=0)).to(dev)
    V = torch.from_numpy(np.repeat(v[None], batch, axis=0)).to(dev)
    q = torch.from_numpy(np.repeat(gen_query(w, 0, T)[None], batch, axis=0)).to(dev)
    cfg = kvq.Config(1, w.n_kv, w.n_q, batch, T, 3, 3, recent_window=recent)
    os.environ["KVQ_MERGE_POLL_LIMIT"] = "0"
    try:
        bad = kvq.Cache(cfg)
    finally:
        del os.environ["KVQ_MERGE_POLL_LIMIT"]
    good = kvq.Cache(cfg)
    for c in (bad, good):
        c.alloc_bits(0, K[0, :2048].contiguous())
        c.quantize_append(0, K, V)
    ref = good.decode_attn(0, q).cpu()
    assert torch.isfinite(ref).all()
    good.status()                                   # nothing to report
    out = bad.decode_attn(0, q).cpu()
    assert torch.isnan(out).all()
    with pytest.raises(kvq.KvqError) as e:
        bad.status()
    assert e.value.status == kvq.KVQ_EHIP and "gave up" in str(e.value)
    bad.status()                                    # reported once, then cleared
    # one split needs no merge: exact again on the same cache
    one = bad.decode_attn(0, q, n_splits=1).cpu() if batch == 1 else None
    if one is not None:
        assert torch.allclose(one, ref, rtol=2e-6, atol=2e-6)
    bad.status()
    bad.close()
    good.close()
