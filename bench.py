#!/usr/bin/env python3
"""Packed-KV decode attention benchmark on one MI355X.

Workload (default): Qwen2.5-3B-shaped decode attention step, 36 layers, 2 KV
heads, 16 query heads, head_dim 128, 131072 cached tokens per layer, batch 1,
Block-GTQ K3V3 packed cache.  Synthetic RoPE'd Gaussian keys with per-block
log-normal deviations (2 outlier blocks per head at 10x) and Gaussian values
are drawn on the GPU; each layer is calibrated on its first 2048 tokens,
then all tokens are appended.

A step = one kvq_decode_attn call per layer (36 launches, one query each),
inputs resident in HBM.  `value` is the step's algorithmic bytes over its time
(effective GB/s); tokens/s and % of the 8 TB/s peak are reported beside it.
The roofline entry divides the timed region (HIP events on the launch stream,
which carries nothing but the decode launches) by the number of launches.  The CPU baseline times the fp64 oracle's decode (unpack, dequantize,
attention) of layer 0, repeated for at least 10 s of host time, and scales the
per-layer time to a step.  --traffic-probe runs one plain 256 MiB copy and one
decode launch for the HBM byte counters (rocprofv3 --pmc FETCH_SIZE, then
WRITE_SIZE); their per-launch figure is reported only while the decode kernel's
sources hash to the value recorded beside it.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--traffic-probe]
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
APPEND_STEPS = 24               # new positions of the append-and-attend steps (2 warm-up + 22 timed)
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
        "alloc_s_per_layer": round(t_q - t_a, 3),
        "quantize_s_per_layer": round(t_e - t_q, 3),
        "sample": f"layer 0 of {n_layers} ({H} KV heads x {T} tokens), decoded {reps} times: unpack + "
                  f"fp64 dequantize + fp64 attention took {dt:.2f} s per layer; scaled x{n_layers} "
                  f"to one step",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3b_128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="skip the K3V2 / recent-window variants and the fidelity diagnostics "
                         "(for kernel traces of the step's decode launches alone)")
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

    # capacity for the T cached positions plus the new ones of the append-and-attend steps
    cache = kvq.Cache(kvq.Config(L, H, Hq, B, T + APPEND_STEPS, kb, vb))
    gen = TorchLayerGen(w, dev)
    chunk = min(w.calib_tokens, T)
    app_ms = []
    keep = None
    t_setup = time.perf_counter()
    for layer in range(1 if args.traffic_probe else L):
        k, v = gen.layer(layer)
        cache.alloc_bits(layer, k[:chunk])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        cache.quantize_append(layer, k[None, :chunk], v[None, :chunk])
        e1.record(stream)
        if T > chunk:
            cache.quantize_append(layer, k[None, chunk:], v[None, chunk:])
        torch.cuda.synchronize()
        app_ms.append(e0.elapsed_time(e1))
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

    bytes_cache_layer = B * H * T * ((kb + vb) * 128 / 8 + 4)
    bytes_launch = bytes_cache_layer + B * Hq * 128 * 2 + B * Hq * 128 * 4 + H * PLAN_BYTES_PER_HEAD
    bytes_step = bytes_launch * L

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
    # spread of single steps (a second pass, each step between its own events)
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, z in step_ev:
        a.record(stream)
        step()
        z.record(stream)
    torch.cuda.synchronize()
    step_ms = np.array([a.elapsed_time(z) for a, z in step_ev])

    # variants on layer 0's data (one layer each): the asymmetric K3V2 budget, and an fp16 recent
    # window of 1024 positions; decode launches timed like the step
    variants = {}
    k0d = keys0[0]
    v0d = torch.from_numpy(keep[1]).to(dev) if keep is not None and not args.decode_only else None
    if v0d is not None:
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
            for _ in range(5):
                vc.decode_attn(0, qs[0], out=vo)
            torch.cuda.synchronize()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            for _ in range(50):
                vc.decode_attn(0, qs[0], out=vo)
            a1.record(stream)
            torch.cuda.synchronize()
            us = a0.elapsed_time(a1) * 1e3 / 50
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

    # batched decode at the Llama-3.1-8B shape of the batch-64 workload (64 x 8192 tokens,
    # 8 KV / 32 query heads, K4V4): one layer, every sequence holding the same synthetic data
    if not args.decode_only:
        wb = WORKLOADS["llama8b_b64"]
        gb = TorchLayerGen(wb, dev)
        kb0, vb0 = gb.layer(0)
        bc = kvq.Cache(kvq.Config(1, wb.n_kv, wb.n_q, wb.batch, wb.T, 4, 4))
        bc.alloc_bits(0, kb0[:wb.calib_tokens])
        bc.quantize_append(0, kb0[None].expand(wb.batch, -1, -1, -1).contiguous(),
                           vb0[None].expand(wb.batch, -1, -1, -1).contiguous())
        del kb0, vb0
        qb = torch.from_numpy(np.stack([np.asarray(gen_query_np(wb, 0, wb.T, seq=i)) for i in range(wb.batch)])).to(dev)
        ob = torch.empty(wb.batch, wb.n_q, 128, dtype=torch.float32, device=dev)
        for _ in range(5):
            bc.decode_attn(0, qb, out=ob)
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(20):
            bc.decode_attn(0, qb, out=ob)
        a1.record(stream)
        torch.cuda.synchronize()
        us = a0.elapsed_time(a1) * 1e3 / 20
        bbytes = wb.batch * wb.n_kv * wb.T * (8 * 16 + 4) + wb.batch * wb.n_q * 128 * 6 + wb.n_kv * PLAN_BYTES_PER_HEAD
        variants["llama8b_b64_K4V4"] = {"batch": wb.batch, "context": wb.T, "us_per_launch": round(us, 2),
                                        "GB/s": round(bbytes / (us * 1e-6) / 1e9, 2),
                                        "frac_of_hbm_peak": round(bbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        bc.close()

    # quality side-report: each codec on one Llama-3.1-8B-shaped layer (8 KV / 32 query heads,
    # 8192 positions, Gaussian and Student-t(5) noise): logit MAE and softmax KL of the stored
    # keys (the library's diagnostics) and the decode output's relative L2 error against fp64
    # attention over the unquantized keys and values (torch, fp64)
    quality = None
    if not args.decode_only:
        quality = {}
        wq = WORKLOADS["llama8b_32k"]
        Tq, Hk, Hqq = 8192, wq.n_kv, wq.n_q
        codecs = (("bgtq_K3V3", kvq.CODEC_BGTQ, 3), ("uniform_K3V3", kvq.CODEC_UNIFORM, 3),
                  ("uniform_rotated_K3V3", kvq.CODEC_UNIFORM_ROT, 3),
                  ("bgtq_group_rotated_K3V3", kvq.CODEC_BGTQ_ROT, 3), ("kivi_K3V3", kvq.CODEC_KIVI, 3),
                  ("bgtq_K4V4", kvq.CODEC_BGTQ, 4), ("nf16_K4V4", kvq.CODEC_NF16_B256, 4))
        for noise in ("gauss", "t5"):
            kq_np, vq_np = gen_layer_np(wq, 0, 0, Tq, noise=noise)
            qq_np = gen_query_np(wq, 0, Tq, noise=noise)
            kq = torch.from_numpy(kq_np).to(dev)[None].contiguous()
            vq = torch.from_numpy(vq_np).to(dev)[None].contiguous()
            qq = torch.from_numpy(qq_np).to(dev)[None].contiguous()
            k64, v64, q64 = kq[0].double(), vq[0].double(), qq[0].double()
            ref = torch.empty(Hqq, 128, dtype=torch.float64, device=dev)
            for hq in range(Hqq):
                lg = (k64[:, hq // wq.group].contiguous() @ q64[hq]) / float(np.sqrt(128.0))
                ref[hq] = torch.softmax(lg, dim=0) @ v64[:, hq // wq.group].contiguous()
            rows = {}
            for label, codec, bits in codecs:
                qc = kvq.Cache(kvq.Config(1, Hk, Hqq, 1, Tq, bits, bits, codec=codec))
                qc.alloc_bits(0, kq[0, :wq.calib_tokens].contiguous()
                              if codec in (kvq.CODEC_BGTQ, kvq.CODEC_BGTQ_ROT) else None)
                if codec in (kvq.CODEC_UNIFORM_ROT, kvq.CODEC_BGTQ_ROT):
                    qc.set_rotation(0, np.random.default_rng(11).choice([-1, 1], size=(Hk, 128)).astype(np.int8))
                qc.quantize_append(0, kq, vq)
                o = qc.decode_attn(0, qq)
                mae_q, kl_q = qc.key_fidelity(0, qq, kq)
                torch.cuda.synchronize()
                err = float(torch.linalg.norm(o[0].double() - ref) / torch.linalg.norm(ref))
                rows[label] = {"logit_mae": round(float(mae_q.mean()), 5),
                               "softmax_kl": float(f"{float(kl_q.mean()):.5g}"),
                               "out_rel_l2": float(f"{err:.4g}")}
                qc.close()
            quality[noise] = rows
            del kq, vq, qq, k64, v64, q64, ref

    # key-fidelity diagnostics of layer 0 (logit MAE and softmax KL against the given keys)
    fid_reps = 0 if args.decode_only else 5
    fid_us, mae, kl = float("nan"), torch.full((1,), float("nan")), torch.full((1,), float("nan"))
    if fid_reps:
        cache.key_fidelity(0, qs[0], keys0)
        torch.cuda.synchronize()
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record(stream)
        for _ in range(fid_reps):
            mae, kl = cache.key_fidelity(0, qs[0], keys0)
        f1.record(stream)
        torch.cuda.synchronize()
        fid_us = f0.elapsed_time(f1) * 1e3 / fid_reps
    fid_bytes = B * T * H * (128 * 2 + kb * 16 + 2) + B * Hq * 128 * 2
    fid_flops = 2 * 2 * 128 * B * T * Hq          # two fp64 dot products per (position, query head)
    del keys0

    # the decode step as a model runs it: every layer first appends the new position's K and V
    # (one quantize_append of one position per sequence), then attends over the cache holding it
    step_app = None
    if not args.decode_only:
        g = torch.Generator(device=dev).manual_seed(5)
        new_kv = [(torch.randn(B, 1, H, 128, device=dev, generator=g).half(),
                   torch.randn(B, 1, H, 128, device=dev, generator=g).half()) for _ in range(L)]

        def step_with_append():
            for layer in range(L):
                cache.quantize_append(layer, new_kv[layer][0], new_kv[layer][1])
                cache.decode_attn(layer, qs[layer], out=outs[layer])

        n_warm, n_timed = 2, APPEND_STEPS - 2
        for _ in range(n_warm):
            step_with_append()
        torch.cuda.synchronize()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for _ in range(n_timed):
            step_with_append()
        s1.record(stream)
        torch.cuda.synchronize()
        ms_app = s0.elapsed_time(s1) / n_timed
        step_app = {"ms_per_step": round(ms_app, 5), "tokens_per_s": round(B / (ms_app * 1e-3), 2),
                    "steps": n_timed, "append_us_per_layer": round((ms_app - ms_step) * 1e3 / L, 2)}

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
        "append": {
            "tokens_per_layer": chunk,
            "us_per_layer": round(float(np.mean(app_ms)) * 1e3, 2),
            "GB/s": round((B * H * chunk * (2 * 128 * 2 + (kb + vb) * 16 + 4)) /
                          (float(np.mean(app_ms)) * 1e-3) / 1e9, 2),
        },
        "decode_step_with_append": step_app,
        "quality": None if quality is None else {"workload": "llama8b_32k layer 0, 8192 positions", **quality},
        "variants": variants,
        "fidelity": None if not fid_reps else {
            "layer": 0,
            "us_per_layer": round(fid_us, 2),
            "GB/s": round(fid_bytes / (fid_us * 1e-6) / 1e9, 2),
            "fp64_TFLOP/s": round(fid_flops / (fid_us * 1e-6) / 1e12, 2),
            "logit_mae_mean": round(float(mae.mean()), 6),
            "softmax_kl_mean": float(f"{float(kl.mean()):.6g}"),
        },
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
