"""Fast seeded synthetic K/V/Q drawn on the GPU with torch (bench-sized workloads).

Same recipe as ``workloads.gen_layer`` (per-block log-normal deviations with
outlier blocks from ``block_sigmas``, Gaussian noise, RoPE at positions
0..T-1, the query at position T), but the Gaussian noise comes from torch's
Philox generator on the device, seeded per (workload, layer, sequence), and
the rotation is applied in fp32 with cos/sin tables computed in fp64 on the
host.  It therefore produces different numbers than ``gen_layer`` and is used
where a whole 36-layer cache must be filled quickly; any oracle comparison
made on such data copies the very same tensors to the host.
"""
from __future__ import annotations

import numpy as np

from .workloads import SEED_BASE, Workload, block_index, block_sigmas, rope_frequencies


class TorchLayerGen:
    def __init__(self, w: Workload, device, pairing: str = "half"):
        import torch
        self.torch = torch
        self.w, self.dev, self.pairing = w, device, pairing
        d = w.head_dim
        ang = np.arange(w.T + 1, dtype=np.float64)[:, None] * rope_frequencies(d, w.theta)[None, :]
        self.cos = torch.from_numpy(np.cos(ang).astype(np.float32)).to(device)   # [T+1, d/2]
        self.sin = torch.from_numpy(np.sin(ang).astype(np.float32)).to(device)
        self.jidx = torch.from_numpy(block_index(d, pairing)).to(device)

    def _gen(self, layer: int, seq: int, stream: int):
        g = self.torch.Generator(device=self.dev)
        g.manual_seed(SEED_BASE * 1000 + self.w.index * 100000 + layer * 1000 + seq * 10 + stream)
        return g

    def _rope(self, x, pos0: int):
        # x [n, H, d] fp32, rows at positions pos0 .. pos0 + n - 1
        n = x.shape[0]
        c = self.cos[pos0:pos0 + n][:, None, :]
        s = self.sin[pos0:pos0 + n][:, None, :]
        nb = x.shape[-1] // 2
        out = self.torch.empty_like(x)
        if self.pairing == "half":
            a, b = x[..., :nb], x[..., nb:]
            out[..., :nb] = a * c - b * s
            out[..., nb:] = a * s + b * c
        else:
            a, b = x[..., 0::2], x[..., 1::2]
            out[..., 0::2] = a * c - b * s
            out[..., 1::2] = a * s + b * c
        return out

    def layer(self, layer: int, seq: int = 0, dtype=None):
        """(k, v) [T, n_kv, d] on the device (fp16 unless dtype is given)."""
        torch = self.torch
        w = self.w
        dtype = torch.float16 if dtype is None else dtype
        sig = torch.from_numpy(block_sigmas(w, layer).astype(np.float32)).to(self.dev)[:, self.jidx]
        zk = torch.randn((w.T, w.n_kv, w.head_dim), generator=self._gen(layer, seq, 0), device=self.dev)
        zv = torch.randn((w.T, w.n_kv, w.head_dim), generator=self._gen(layer, seq, 1), device=self.dev)
        k = self._rope(zk * sig[None], 0).to(dtype)
        return k.contiguous(), zv.to(dtype).contiguous()

    def query(self, layer: int, seq: int = 0, dtype=None):
        """q [n_q, d] at position T."""
        torch = self.torch
        w = self.w
        dtype = torch.float16 if dtype is None else dtype
        sig = torch.from_numpy(block_sigmas(w, layer).astype(np.float32)).to(self.dev)[:, self.jidx]
        kv_of_q = torch.arange(w.n_q, device=self.dev) // w.group
        z = torch.randn((w.n_q, w.head_dim), generator=self._gen(layer, seq, 2), device=self.dev)
        q = self._rope((z * sig[kv_of_q])[None], w.T)[0]
        return q.to(dtype).contiguous()
