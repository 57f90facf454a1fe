#!/usr/bin/env python3
"""Packed-KV decode attention benchmark on one MI355X.

Workload (default): Qwen2.5-3B-shaped decode attention step, 36 layers, 2 KV
heads, 16 query heads, head_dim 128, 131072 cached tokens per layer, batch 1,
Block-GTQ K3V3 packed cache.  Synthetic RoPE'd Gaussian keys with per-block
log-normal deviations (2 outlier blocks per head at 10x) and Gaussian values
are drawn on the GPU; each layer is calibrated on its first 2048 tokens,
then all but the last 24 tokens are appended at once, and the last 24 by
decode steps (kvq_decode_step: the append and the attention in one launch per
layer), timed as `decode_step_with_append`.

A step = one kvq_decode_attn call per layer (36 launches, one query each),
inputs resident in HBM.  `value` is the step's algorithmic bytes over its time
(effective GB/s); tokens/s and % of the 8 TB/s peak are reported beside it.
The roofline entry divides the timed region (HIP events on the launch stream,
which carries nothing but the decode launches) by the number of launches, and
sets it against the per-launch read ceiling measured in the same run: a plain
streaming-read kernel (kvq_probe_stream_read) over 36 buffers of one launch's
bytes, best of several grid sizes.

Beside the headline (skipped with --decode-only): the 524288-token K2V2 step
(36 layers), one Llama-shaped layer at K2V2/K3V3/K4V4 for Block-GTQ and the
uniform codec (12 copies cycled so the 256 MB last-level cache holds none),
batched decode at 64 x 8192 for Block-GTQ and the 256-value absmax codec,
codec variants of the headline layer, append rates from back-to-back launches,
the single-head 1024-position fp32 K4V4 decode (latency-bound, in us),
the decode step with each layer first appending the new position (one fused
launch per layer, and as two calls), the key fidelity diagnostics, and a
quality side-report (logit MAE, softmax KL, output error) at the default and a
tempered softmax scale.

The CPU baseline times the fp64 oracle's decode (unpack, dequantize,
attention) of layer 0, repeated for at least 10 s of host time on one thread,
and scales the per-layer time to a step.  --traffic-probe runs one plain
256 MiB copy and one decode launch for the HBM byte counters (rocprofv3 --pmc
FETCH_SIZE, then WRITE_SIZE); their per-launch figure is reported only while
the decode kernel's sources hash to the value recorded beside it.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--decode-only] [--traffic-probe]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PLAN_BYTES_PER_HEAD = 1024   # field dims/widths/offsets and gains read by each decode launch
APPEND_STEPS = 24               # new positions per append-and-attend variant (2 warm-up + 22 timed)
SINGLE_APPENDS = 200            # one-position appends timed back to back
BULK_CACHES = 4                 # layers whose 98304-position appends are timed back to back
CPU_SAMPLE_S = 10.0          # lower bound on the host time spent timing the oracle
DECODE_SOURCES = ["decode_mfma.h", "decode_mfma.hip", "decode_mfma_g1.hip", "decode_mfma_g2.hip",
                  "decode_mfma_g4.hip", "decode_mfma_g8.hip", "kvq_internal.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_mfma_qwen3b_128k_k3v3_traffic.json")


def decode_source_hash() -> str:
    """sha256 over the decode kernel's sources: the HBM counters are valid for this text only."""
    import hashlib
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, "rope_aware_bit_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic():
    """Per-launch HBM bytes measured by rocprofv3 counters for the current kernel text, else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != decode_source_hash():
        return None
    return rec.get("bytes_per_launch")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_description():
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


def cpu_baseline(k0, v0, q0, calib, kb, vb, n_layers, bytes_per_step):
    """Time the oracle's decode of one layer (host cores, BLAS limited to one thread)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import allocation as al
    from oracle import attention as at
    from oracle import layout as lay
    from tests.parity import OracleLayer

    H = k0.shape[1]
    with threadpool_limits(limits=1):
        t_a = time.perf_counter()
        ol = OracleLayer(calib, kb, vb)         # allocation from the calibration keys
        t_q = time.perf_counter()
        packed = []
        for h in range(H):                      # quantize + pack every position (the appends)
            r = ol.quantize_head(k0[:, h], v0[:, h], h)
            packed.append((r["k_words"], r["k_s16"], lay.pack_v_tiles(r["v_codes"], vb), r["v_s16"]))
        t_e = time.perf_counter()
    T = k0.shape[0]

    def one_layer():
        kh, vh = [], []
        for h in range(H):
            kw, ks, vw, vs = packed[h]
            dims, ws = ol.fields(h)
            kc = lay.unpack_k_rows(kw, dims, ws, 128)
            kh.append(at.dequant_k(kc, ks, al.dim_widths(ol.widths[h], 128), al.dim_values(ol.g[h], 128)))
            vh.append(at.dequant_v(lay.unpack_v_tiles(vw, vb, T), vs, vb))
        return at.decode_attention(q0.astype(np.float64), np.stack(kh), np.stack(vh))

    with threadpool_limits(limits=1):
        reps, t0 = 0, time.perf_counter()
        while True:
            out = one_layer()
            reps += 1
            if time.perf_counter() - t0 >= CPU_SAMPLE_S or reps >= n_layers:
                break
        dt = (time.perf_counter() - t0) / reps
    assert np.all(np.isfinite(out))
    step_s = dt * n_layers
    return {
        "value": round(bytes_per_step / step_s / 1e9, 4),
        "unit": "GB/s",
        "tokens_per_s": round(1.0 / step_s, 5),
        "cores": 1,
        "kind": "oracle",
        "host": host_description(),
        "alloc_s_per_layer": round(t_q - t_a, 3),
        "quantize_s_per_layer": round(t_e - t_q, 3),
        "sample": f"layer 0 of {n_layers} ({H} KV heads x {T} tokens), decoded {reps} times on one "
                  f"thread: unpack + fp64 dequantize + fp64 attention took {dt:.2f} s per layer; "
                  f"scaled x{n_layers} to one step",
    }


class Timer:
    """HIP events on one stream around a region of enqueued work."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def ms(self, fn, reps, warm=2):
        torch = self.torch
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(self.stream)
        for _ in range(reps):
            fn()
        z.record(self.stream)
        torch.cuda.synchronize()
        return a.elapsed_time(z) / reps


def read_ceiling(torch, kvq, timer, nbytes, n_buffers, dev):
    """Best per-launch time of a plain streaming read of nbytes, cycling n_buffers distinct buffers
    (their total exceeds the last-level cache, as the decode step's layers do)."""
    nb = (int(nbytes) + 15) // 16 * 16
    bufs = [torch.full((nb,), i % 251, dtype=torch.uint8, device=dev) for i in range(n_buffers)]
    sink = torch.zeros(65536, dtype=torch.int32, device=dev)
    best = None
    for n_blocks in (256, 512, 1024, 2048, 4096):
        ms = timer.ms(lambda: [kvq.probe_stream_read(b, n_blocks, sink) for b in bufs], 5)
        us = ms * 1e3 / n_buffers
        if best is None or us < best[0]:
            best = (us, n_blocks)
    del bufs
    return {"us_per_launch": round(best[0], 3), "GB/s": round(nb / (best[0] * 1e-6) / 1e9, 1),
            "bytes_per_launch": nb, "buffers": n_buffers, "workgroups": best[1]}


def decode_bytes(B, H, Hq, T, kb, vb):
    """Algorithmic bytes of one decode launch: packed cache + two fp16 scales per token-head,
    fp16 query, fp32 output, the plan."""
    return B * H * T * ((kb + vb) * 128 / 8 + 4) + B * Hq * 128 * 2 + B * Hq * 128 * 4 + H * PLAN_BYTES_PER_HEAD


def long_context_step(torch, kvq, timer, dev, WORKLOADS, TorchLayerGen):
    """The 524288-token K2V2 decode step: 36 layers, 2 KV / 16 query heads, batch 1."""
    w = WORKLOADS["qwen3b_512k"]
    kb, vb = w.budgets[0]
    L, H, Hq, T = w.n_layers, w.n_kv, w.n_q, w.T
    cache = kvq.Cache(kvq.Config(L, H, Hq, 1, T, kb, vb))
    gen = TorchLayerGen(w, dev)
    for layer in range(L):
        k, v = gen.layer(layer)
        cache.alloc_bits(layer, k[:w.calib_tokens])
        cache.quantize_append(layer, k[None], v[None])
        del k, v
    qs = [gen.query(layer)[None].contiguous() for layer in range(L)]
    outs = [torch.empty(1, Hq, 128, dtype=torch.float32, device=dev) for _ in range(L)]
    torch.cuda.synchronize()

    def step():
        for layer in range(L):
            cache.decode_attn(layer, qs[layer], out=outs[layer])

    ms = timer.ms(step, 10)
    for o in outs:
        assert torch.isfinite(o).all()
    cache.close()
    byts = L * decode_bytes(1, H, Hq, T, kb, vb)
    return {"workload": f"{L} layers x {H} KV heads, {Hq} query heads, {T} tokens, batch 1, Block-GTQ K{kb}V{vb}",
            "ms_per_step": round(ms, 4), "GB/s": round(byts / (ms * 1e-3) / 1e9, 2),
            "frac_of_hbm_peak": round(byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "tokens_per_s": round(1.0 / (ms * 1e-3), 2), "bytes_per_step": int(byts),
            "us_per_launch": round(ms * 1e3 / L, 2),
            "fp16_cache_GB_estimate": round(2 * 2 * 128 * H * L * T / 1e9, 2)}


def llama_layer_budgets(torch, kvq, timer, dev, WORKLOADS, TorchLayerGen):
    """One Llama-3.1-8B-shaped layer (8 KV / 32 query heads, 32768 tokens) at K2V2, K3V3, K4V4, for
    Block-GTQ and the uniform codec; 12 copies of the layer are cycled so the last-level cache
    holds none of them when read."""
    w = WORKLOADS["llama8b_32k"]
    H, Hq, T = w.n_kv, w.n_q, w.T
    n_copies = 12
    gen = TorchLayerGen(w, dev)
    k, v = gen.layer(0)
    q = gen.query(0)[None].contiguous()
    out = torch.empty(1, Hq, 128, dtype=torch.float32, device=dev)
    res = {}
    for kb in (2, 3, 4):
        for name, codec in (("bgtq", kvq.CODEC_BGTQ), ("uniform", kvq.CODEC_UNIFORM)):
            c = kvq.Cache(kvq.Config(n_copies, H, Hq, 1, T, kb, kb, codec=codec))
            for layer in range(n_copies):
                c.alloc_bits(layer, k[:w.calib_tokens] if codec == kvq.CODEC_BGTQ else None)
                c.quantize_append(layer, k[None], v[None])
            ms = timer.ms(lambda: [c.decode_attn(layer, q, out=out) for layer in range(n_copies)], 10)
            us = ms * 1e3 / n_copies
            byts = decode_bytes(1, H, Hq, T, kb, kb)
            res[f"{name}_K{kb}V{kb}"] = {"us_per_launch": round(us, 2), "GB/s": round(byts / (us * 1e-6) / 1e9, 2),
                                         "frac_of_hbm_peak": round(byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                         "bytes_per_launch": int(byts)}
            c.close()
    return {"workload": f"one layer, {H} KV / {Hq} query heads, {T} tokens, batch 1 ({n_copies} copies cycled)", **res}


def tiny_decode(torch, kvq, timer, dev, WORKLOADS, TorchLayerGen):
    """The single-head case (one KV head, one query head, 1024 positions, fp32 keys, values and
    query, K4V4): its 135 KB take 0.02 us at the HBM peak, so the launch is latency-bound and is
    reported in us.  Back-to-back launches queued behind a spin kernel, so the time is the GPU's,
    not the host's per-call overhead."""
    w = WORKLOADS["tiny"]
    kb, vb = w.budgets[0]
    gen = TorchLayerGen(w, dev)
    k, v = gen.layer(0, dtype=torch.float32)
    q = gen.query(0, dtype=torch.float32)[None].contiguous()
    out = torch.empty(1, w.n_q, 128, dtype=torch.float32, device=dev)
    c = kvq.Cache(kvq.Config(1, w.n_kv, w.n_q, 1, w.T, kb, vb))
    c.alloc_bits(0, k[:w.calib_tokens])
    c.quantize_append(0, k[None], v[None])
    n = 200
    for _ in range(5):
        c.decode_attn(0, q, out=out)
    torch.cuda.synchronize()
    a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(20_000_000)
    a.record(timer.stream)
    for _ in range(n):
        c.decode_attn(0, q, out=out)
    z.record(timer.stream)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    us = a.elapsed_time(z) * 1e3 / n
    c.close()
    return {"workload": f"{w.n_kv} KV / {w.n_q} query head, {w.T} positions, batch 1, fp32 inputs, K{kb}V{vb}",
            "us_per_launch": round(us, 2), "launches": n,
            "bytes_per_launch": int(decode_bytes(1, w.n_kv, w.n_q, w.T, kb, vb))}


def batched_decode(torch, kvq, timer, dev, WORKLOADS, TorchLayerGen, gen_query_np, np):
    """Batched decode at the Llama-3.1-8B KV shape, 64 sequences x 8192 tokens, K4V4: Block-GTQ and
    the 256-value absmax codec (every sequence holds the same synthetic keys and values)."""
    wb = WORKLOADS["llama8b_b64"]
    gb = TorchLayerGen(wb, dev)
    kb0, vb0 = gb.layer(0)
    qb = torch.from_numpy(np.stack([np.asarray(gen_query_np(wb, 0, wb.T, seq=i)) for i in range(wb.batch)])).to(dev)
    ob = torch.empty(wb.batch, wb.n_q, 128, dtype=torch.float32, device=dev)
    kx = kb0[None].expand(wb.batch, -1, -1, -1).contiguous()
    vx = vb0[None].expand(wb.batch, -1, -1, -1).contiguous()
    res = {}
    for label, codec in (("bgtq_K4V4", kvq.CODEC_BGTQ), ("nf16_K4V4", kvq.CODEC_NF16_B256)):
        bc = kvq.Cache(kvq.Config(1, wb.n_kv, wb.n_q, wb.batch, wb.T, 4, 4, codec=codec))
        bc.alloc_bits(0, kb0[:wb.calib_tokens] if codec == kvq.CODEC_BGTQ else None)
        bc.quantize_append(0, kx, vx)
        us = timer.ms(lambda: bc.decode_attn(0, qb, out=ob), 20, warm=5) * 1e3
        assert torch.isfinite(ob).all()
        if codec == kvq.CODEC_NF16_B256:   # 4-bit codes and one fp16 scale per 256 values, K and V
            cache_b = wb.batch * wb.T * wb.n_kv * 2 * (64 + 2 * 128 / 256)
        else:
            cache_b = wb.batch * wb.n_kv * wb.T * (8 * 16 + 4)
        byts = cache_b + wb.batch * wb.n_q * 128 * 6 + wb.n_kv * PLAN_BYTES_PER_HEAD
        res[label] = {"us_per_launch": round(us, 2), "GB/s": round(byts / (us * 1e-6) / 1e9, 2),
                      "frac_of_hbm_peak": round(byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                      "tokens_per_s": round(wb.batch / (us * 1e-6), 1), "bytes_per_launch": int(byts)}
        bc.close()
    return {"workload": f"batch {wb.batch} x {wb.T} tokens, {wb.n_kv} KV / {wb.n_q} query heads, one layer", **res}


def append_rates(torch, kvq, timer, dev, WORKLOADS, TorchLayerGen, kb, vb):
    """Kernel-side append rates of the headline shape (2 KV heads, K3V3), each from back-to-back
    launches: appends of 2048 positions, appends of the rest of a 131072-token layer (one per
    layer of BULK_CACHES layers, after their first 32768 positions), and one-position appends
    (the decode step's).  The small appends are queued behind a spin kernel, so their time is
    the GPU's, not the host's per-call overhead."""
    w = WORKLOADS["qwen3b_128k"]
    H, T = w.n_kv, w.T
    gen = TorchLayerGen(w, dev)
    k, v = gen.layer(0)
    per_pos = H * (2 * 128 * 2 + (kb + vb) * 16 + 4)      # fp16 K and V in, packed rows and scales out

    def hold_gpu():
        # a spin kernel of several ms ahead of the timed launches, so that the host has enqueued
        # them all before the GPU reaches the first: small appends then run back to back on the
        # GPU instead of waiting for the host's per-call overhead
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(20_000_000)
    res = {}
    n_chunks = 16
    c = kvq.Cache(kvq.Config(1, H, w.n_q, 1, T + SINGLE_APPENDS + 8, kb, vb))
    c.alloc_bits(0, k[:w.calib_tokens])
    chunks = [(k[None, i * 2048:(i + 1) * 2048].contiguous(), v[None, i * 2048:(i + 1) * 2048].contiguous())
              for i in range(n_chunks)]
    torch.cuda.synchronize()
    a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hold_gpu()
    a.record(timer.stream)
    for kc_, vc_ in chunks:
        c.quantize_append(0, kc_, vc_)
    z.record(timer.stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(z) * 1e3 / n_chunks
    res["chunk_2048"] = {"us_per_append": round(us, 2), "GB/s": round(2048 * per_pos / (us * 1e-6) / 1e9, 2),
                         "appends": n_chunks}
    rest = T - n_chunks * 2048
    kr, vr = k[None, n_chunks * 2048:].contiguous(), v[None, n_chunks * 2048:].contiguous()
    c.quantize_append(0, kr, vr)
    # the same append on further layers, back to back (each layer first holds 32768 positions)
    bc = kvq.Cache(kvq.Config(BULK_CACHES, H, w.n_q, 1, T, kb, vb))
    k0, v0 = k[None, :n_chunks * 2048].contiguous(), v[None, :n_chunks * 2048].contiguous()
    for layer in range(BULK_CACHES):
        bc.alloc_bits(layer, k[:w.calib_tokens])
        bc.quantize_append(layer, k0, v0)
    torch.cuda.synchronize()
    a.record(timer.stream)
    for layer in range(BULK_CACHES):
        bc.quantize_append(layer, kr, vr)
    z.record(timer.stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(z) * 1e3 / BULK_CACHES
    assert all(bc.seq_len(layer) == T for layer in range(BULK_CACHES))
    bc.close()
    res["bulk"] = {"positions": rest, "us": round(us, 2), "appends": BULK_CACHES,
                   "GB/s": round(rest * per_pos / (us * 1e-6) / 1e9, 2),
                   "frac_of_hbm_peak": round(rest * per_pos / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    g = torch.Generator(device=dev).manual_seed(3)
    ones = [(torch.randn(1, 1, H, 128, device=dev, generator=g).half(),
             torch.randn(1, 1, H, 128, device=dev, generator=g).half()) for _ in range(SINGLE_APPENDS)]
    torch.cuda.synchronize()
    hold_gpu()
    a.record(timer.stream)
    for kk, vv in ones:
        c.quantize_append(0, kk, vv)
    z.record(timer.stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(z) * 1e3 / SINGLE_APPENDS
    res["single_position"] = {"us_per_append": round(us, 2), "appends": SINGLE_APPENDS}
    assert c.seq_len(0) == T + SINGLE_APPENDS
    c.close()
    return res


def quality_report(torch, kvq, dev, WORKLOADS, gen_layer_np, gen_query_np, np):
    """Each codec on one Llama-3.1-8B-shaped layer (8 KV / 32 query heads, all 32768 positions,
    Gaussian and Student-t(5) noise), at the default softmax scale 1/sqrt(128) and at a tempered
    scale that makes the unquantized logits' standard deviation 2: logit MAE and softmax KL of
    the stored keys (the library's diagnostics) and the decode output's relative L2 error against
    fp64 attention over the unquantized keys and values (torch, fp64)."""
    wq = WORKLOADS["llama8b_32k"]
    Tq, Hk, Hqq = wq.T, wq.n_kv, wq.n_q
    codecs = (("bgtq_K2V2", kvq.CODEC_BGTQ, 2), ("uniform_K2V2", kvq.CODEC_UNIFORM, 2),
              ("uniform_rotated_K2V2", kvq.CODEC_UNIFORM_ROT, 2), ("kivi_K2V2", kvq.CODEC_KIVI, 2),
              ("bgtq_K3V3", kvq.CODEC_BGTQ, 3), ("uniform_K3V3", kvq.CODEC_UNIFORM, 3),
              ("uniform_rotated_K3V3", kvq.CODEC_UNIFORM_ROT, 3),
              ("bgtq_group_rotated_K3V3", kvq.CODEC_BGTQ_ROT, 3), ("kivi_K3V3", kvq.CODEC_KIVI, 3),
              ("bgtq_K4V4", kvq.CODEC_BGTQ, 4), ("nf16_K4V4", kvq.CODEC_NF16_B256, 4))
    out = {"workload": f"llama8b_32k layer 0, {Tq} positions, {Hk} KV / {Hqq} query heads"}
    for noise in ("gauss", "t5"):
        kq_np, vq_np = gen_layer_np(wq, 0, 0, Tq, noise=noise)
        qq_np = gen_query_np(wq, 0, Tq, noise=noise)
        kq = torch.from_numpy(kq_np).to(dev)[None].contiguous()
        vq = torch.from_numpy(vq_np).to(dev)[None].contiguous()
        qq = torch.from_numpy(qq_np).to(dev)[None].contiguous()
        k64, v64, q64 = kq[0].double(), vq[0].double(), qq[0].double()
        raw = torch.stack([k64[:, hq // wq.group].contiguous() @ q64[hq] for hq in range(Hqq)])   # [Hq, T]
        scales = {"default": 1.0 / float(np.sqrt(128.0)), "tempered": float(2.0 / raw.std())}
        for sl, sigma in scales.items():
            ref = torch.stack([torch.softmax(sigma * raw[hq], dim=0) @ v64[:, hq // wq.group].contiguous()
                               for hq in range(Hqq)])
            rows = {"softmax_scale": float(f"{sigma:.6g}"),
                    "logit_std": float(f"{float((sigma * raw).std()):.4g}")}
            for label, codec, bits in codecs:
                qc = kvq.Cache(kvq.Config(1, Hk, Hqq, 1, Tq, bits, bits, codec=codec))
                qc.alloc_bits(0, kq[0, :wq.calib_tokens].contiguous()
                              if codec in (kvq.CODEC_BGTQ, kvq.CODEC_BGTQ_ROT) else None)
                if codec in (kvq.CODEC_UNIFORM_ROT, kvq.CODEC_BGTQ_ROT):
                    qc.set_rotation(0, np.random.default_rng(11).choice([-1, 1], size=(Hk, 128)).astype(np.int8))
                qc.quantize_append(0, kq, vq)
                o = qc.decode_attn(0, qq, scale=sigma)
                mae_q, kl_q = qc.key_fidelity(0, qq, kq, scale=sigma)
                torch.cuda.synchronize()
                err = float(torch.linalg.norm(o[0].double() - ref) / torch.linalg.norm(ref))
                rows[label] = {"logit_mae": float(f"{float(mae_q.mean()):.5g}"),
                               "softmax_kl": float(f"{float(kl_q.mean()):.5g}"),
                               "out_rel_l2": float(f"{err:.4g}")}
                qc.close()
            out[f"{noise}_{sl}"] = rows
        del kq, vq, qq, k64, v64, q64, raw
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3b_128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the headline step (and the read ceiling): for kernel traces of the step's "
                         "decode launches alone")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run one plain copy of known size and one decode launch, then exit "
                         "(for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the packed decode path "
              "is single-GPU and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from rope_aware_bit_amd import kvq
    from synth import WORKLOADS
    from synth import gen_layer as gen_layer_np
    from synth import gen_query as gen_query_np
    from synth.torch_gen import TorchLayerGen

    w = WORKLOADS[args.workload]
    kb, vb = w.budgets[0]
    L, H, Hq, B, T = w.n_layers, w.n_kv, w.n_q, w.batch, w.T
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    timer = Timer(torch, stream)

    # capacity for the T cached positions plus the new ones of the append-and-attend steps past T
    cache = kvq.Cache(kvq.Config(L, H, Hq, B, T + 2 * APPEND_STEPS, kb, vb))
    gen = TorchLayerGen(w, dev)
    chunk = min(w.calib_tokens, T)
    keep = None
    t_setup = time.perf_counter()
    # every layer holds T positions: the first T - APPEND_STEPS appended at once, the last
    # APPEND_STEPS by decode steps (below, timed), each appending one position and attending
    n_pre = T if args.traffic_probe else T - APPEND_STEPS
    tails = []
    for layer in range(1 if args.traffic_probe else L):
        k, v = gen.layer(layer)
        cache.alloc_bits(layer, k[:chunk])
        cache.quantize_append(layer, k[None, :n_pre].contiguous(), v[None, :n_pre].contiguous())
        tails.append((k[n_pre:].contiguous(), v[n_pre:].contiguous()))
        torch.cuda.synchronize()
        if layer == 0:
            keep = (k.cpu().numpy(), v.cpu().numpy(), k[:chunk].cpu().numpy())
            keys0 = k[None].contiguous()        # layer 0's keys as given, for the fidelity diagnostics
        del k, v
    qs = [gen.query(layer)[None].contiguous() for layer in range(L)]
    if args.traffic_probe:
        keep = keys0 = None
    outs = [torch.empty(B, Hq, 128, dtype=torch.float32, device=dev) for _ in range(L)]
    torch.cuda.synchronize()
    log(f"setup {time.perf_counter() - t_setup:.1f} s")

    if args.traffic_probe:
        # a plain copy of 256 MiB (its counters give the bytes-per-count factor), then one decode
        src = torch.empty(64 << 20, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        cache.decode_attn(0, qs[0], out=outs[0])
        torch.cuda.synchronize()
        log(f"traffic probe: copy {src.numel() * 4} bytes read + written, one decode launch of layer 0")
        cache.close()
        return

    bytes_launch = decode_bytes(B, H, Hq, T, kb, vb)
    bytes_step = bytes_launch * L

    # the decode step as a model runs it, over the last APPEND_STEPS positions (T - 23 .. T): every
    # layer appends the new position's K and V and attends over the cache holding it, in one launch
    # (kvq_decode_step); 2 warm-up steps, the rest timed
    pos = [0]

    def step_fused_tail():
        i = pos[0]
        for layer in range(L):
            cache.decode_step(layer, tails[layer][0][i][None], tails[layer][1][i][None], qs[layer], out=outs[layer])
        pos[0] += 1

    ms_app_tail = timer.ms(step_fused_tail, APPEND_STEPS - 2, warm=2)
    assert pos[0] == APPEND_STEPS and cache.seq_len(0) == T
    del tails

    def step():
        for layer in range(L):
            cache.decode_attn(layer, qs[layer], out=outs[layer])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    for o in outs:
        assert torch.isfinite(o).all()
    log(f"headline step {ms_step:.4f} ms")
    # spread of single steps (a second pass, each step between its own events)
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, z in step_ev:
        a.record(stream)
        step()
        z.record(stream)
    torch.cuda.synchronize()
    step_ms = np.array([a.elapsed_time(z) for a, z in step_ev])

    # the per-launch read ceiling: a streaming read of one launch's bytes, 36 distinct buffers
    ceiling = read_ceiling(torch, kvq, timer, bytes_launch, L, dev)
    log(f"read ceiling {ceiling}")

    variants, extra = {}, {}
    if not args.decode_only:
        # codec variants of the headline layer's data (one layer each), timed like the step
        k0d = keys0[0]
        v0d = torch.from_numpy(keep[1]).to(dev)
        for label, vk, vv, R, codec in (("K3V2", 3, 2, 0, kvq.CODEC_BGTQ),
                                        ("K3V3_recent1024", 3, 3, 1024, kvq.CODEC_BGTQ),
                                        ("K3V3_uniform_rotated", 3, 3, 0, kvq.CODEC_UNIFORM_ROT),
                                        ("K3V3_kivi", 3, 3, 0, kvq.CODEC_KIVI),
                                        ("K3V3_bgtq_group_rotated", 3, 3, 0, kvq.CODEC_BGTQ_ROT)):
            vc = kvq.Cache(kvq.Config(1, H, Hq, B, T, vk, vv, recent_window=R, codec=codec))
            allocates = codec in (kvq.CODEC_BGTQ, kvq.CODEC_BGTQ_ROT)
            vc.alloc_bits(0, k0d[:chunk] if allocates else None)
            if codec in (kvq.CODEC_UNIFORM_ROT, kvq.CODEC_BGTQ_ROT):
                vc.set_rotation(0, np.random.default_rng(11).choice([-1, 1], size=(H, 128)).astype(np.int8))
            vc.quantize_append(0, k0d[None], v0d[None])
            vo = torch.empty(B, Hq, 128, dtype=torch.float32, device=dev)
            us = timer.ms(lambda: vc.decode_attn(0, qs[0], out=vo), 50, warm=5) * 1e3
            # packed positions (KIVI: whole 128-position tiles) with 4 B of scales each (KIVI: 8 B,
            # 2 fp16 per channel per tile and 2 per position), the rest fp16 K and V
            P = vc.layer_info(0).packed_len
            par = 8 if codec == kvq.CODEC_KIVI else 4
            vbytes = B * H * (P * ((vk + vv) * 128 / 8 + par) + (T - P) * 512) + B * Hq * 128 * 6 + H * PLAN_BYTES_PER_HEAD
            variants[label] = {"k_bits": vk, "v_bits": vv, "recent_window": R, "codec": int(codec),
                               "us_per_launch": round(us, 2),
                               "GB/s": round(vbytes / (us * 1e-6) / 1e9, 2)}
            vc.close()
        del v0d
        log("variants done")
        extra["batched_decode"] = batched_decode(torch, kvq, timer, dev, WORKLOADS, TorchLayerGen, gen_query_np, np)
        log("batched done")
        extra["long_context_step"] = long_context_step(torch, kvq, timer, dev, WORKLOADS, TorchLayerGen)
        log("long context done")
        extra["llama_layer_budgets"] = llama_layer_budgets(torch, kvq, timer, dev, WORKLOADS, TorchLayerGen)
        log("budgets done")
        extra["append"] = append_rates(torch, kvq, timer, dev, WORKLOADS, TorchLayerGen, kb, vb)
        log("append done")
        extra["tiny_decode"] = tiny_decode(torch, kvq, timer, dev, WORKLOADS, TorchLayerGen)
        log("tiny done")
        extra["quality"] = quality_report(torch, kvq, dev, WORKLOADS, gen_layer_np, gen_query_np, np)
        log("quality done")

    # key-fidelity diagnostics of layer 0 (logit MAE and softmax KL against the given keys)
    fid = None
    if not args.decode_only:
        reps = 5
        mae, kl = cache.key_fidelity(0, qs[0], keys0)
        us = timer.ms(lambda: cache.key_fidelity(0, qs[0], keys0), reps, warm=1) * 1e3
        mae, kl = cache.key_fidelity(0, qs[0], keys0)
        torch.cuda.synchronize()
        fid_bytes = B * T * H * (128 * 2 + kb * 16 + 2) + B * Hq * 128 * 2
        fid_flops = 2 * 2 * 128 * B * T * Hq          # two fp64 dot products per (position, query head)
        fid = {"layer": 0, "us_per_layer": round(us, 2), "GB/s": round(fid_bytes / (us * 1e-6) / 1e9, 2),
               "fp64_TFLOP/s": round(fid_flops / (us * 1e-6) / 1e12, 2),
               "logit_mae_mean": round(float(mae.mean()), 6), "softmax_kl_mean": float(f"{float(kl.mean()):.6g}")}
    del keys0

    # the decode step as a model runs it: every layer first appends the new position's K and V
    # (one position per sequence), then attends over the cache holding it.  decode_step does both
    # in one launch; the second figure is the two calls (quantize_append, then decode_attn)
    step_app = None
    if not args.decode_only:
        g = torch.Generator(device=dev).manual_seed(5)
        new_kv = [(torch.randn(B, 1, H, 128, device=dev, generator=g).half(),
                   torch.randn(B, 1, H, 128, device=dev, generator=g).half()) for _ in range(L)]

        def step_fused():
            for layer in range(L):
                cache.decode_step(layer, new_kv[layer][0][:, 0], new_kv[layer][1][:, 0], qs[layer], out=outs[layer])

        def step_two_calls():
            for layer in range(L):
                cache.quantize_append(layer, new_kv[layer][0], new_kv[layer][1])
                cache.decode_attn(layer, qs[layer], out=outs[layer])

        # past T (T + 1 .. T + 24 positions: one more, nearly empty, tile per head than at T): the
        # same fused step, attention alone at that length, and the two calls
        ms_app = timer.ms(step_fused, APPEND_STEPS - 2, warm=2)
        ms_same = timer.ms(step, APPEND_STEPS - 2, warm=2)
        ms_two = timer.ms(step_two_calls, APPEND_STEPS - 2, warm=2)
        step_app = {"positions": f"{T - APPEND_STEPS + 1}..{T}", "ms_per_step": round(ms_app_tail, 5),
                    "tokens_per_s": round(B / (ms_app_tail * 1e-3), 2), "steps": APPEND_STEPS - 2,
                    "vs_attention_only": round(ms_app_tail / ms_step, 3),
                    "append_us_per_layer": round((ms_app_tail - ms_step) * 1e3 / L, 2),
                    "past_T": {"positions": f"{T + 1}..{T + APPEND_STEPS}", "ms_per_step": round(ms_app, 5),
                               "attention_only_same_len_ms": round(ms_same, 5),
                               "vs_attention_only_same_len": round(ms_app / ms_same, 3)},
                    "two_calls": {"positions": f"{T + APPEND_STEPS + 1}..{T + 2 * APPEND_STEPS}",
                                  "ms_per_step": round(ms_two, 5), "vs_attention_only": round(ms_two / ms_step, 3),
                                  "append_us_per_layer": round((ms_two - ms_same) * 1e3 / L, 2)}}

    # average decode-launch duration: the timed region holds only decode launches on this stream
    launch_us = ms_step * 1e3 / L

    value = bytes_step / (ms_step * 1e-3) / 1e9
    achieved = bytes_launch / (launch_us * 1e-6) / 1e9
    res = {
        "metric": "packed-KV decode attn: effective HBM GB/s (% of peak) + tokens/s at 128K K3V3",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_p10_p50_p90": [round(float(np.percentile(step_ms, p)), 5) for p in (10, 50, 90)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16-mfma/f32",
        "data": "synthetic",
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(B / (ms_step * 1e-3), 2),
        "config": {
            "workload": f"packed decode attention, Qwen2.5-3B shape: {L} layers x {H} KV heads, "
                        f"{Hq} query heads, head_dim 128, {T} tokens, batch {B}, Block-GTQ K{kb}V{vb}",
            "layers": L, "kv_heads": H, "q_heads": Hq, "head_dim": 128, "context": T, "batch": B,
            "k_bits": kb, "v_bits": vb, "codec": "bgtq", "launches_per_step": L,
            "bytes_per_step": int(bytes_step), "hip_graph": False,
        },
        "decode_step_with_append": step_app,
        "variants": variants,
        **extra,
        "fidelity": fid,
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_mfma",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(),
            "launch_us": round(launch_us, 3),
            "bytes_per_launch": int(bytes_launch),
            "read_ceiling": ceiling,
            "frac_of_read_ceiling": round(achieved / ceiling["GB/s"], 4),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        k0, v0, calib = keep
        res["cpu_baseline"] = cpu_baseline(k0, v0, qs[0][0].cpu().numpy(), calib, kb, vb, L, bytes_step)
    cache.close()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
