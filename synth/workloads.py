"""Seeded synthetic K/V/Q generators shaped like the workloads of the pages.

Keys are drawn before RoPE as independent Gaussians whose standard deviation
is constant inside each two-dimensional RoPE frequency block and log-normal
across blocks (some blocks get a 10x outlier multiplier), then rotated with
the standard rotary embedding.  Values are standard Gaussians (or Student-t
with 5 degrees of freedom for the heavy-tail stress case).  Each query head
is drawn like the keys of its KV head and rotated at the position that
follows the cached context.

Every stream is keyed by ``SeedSequence(20261203 + workload index,
spawn_key=(stream, layer, sequence, chunk))`` so any token range of any layer
can be regenerated on its own, in any order, bit-for-bit.  Tokens are drawn
in chunks of ``CHUNK`` = 2048 positions.

Nothing here implements the quantization method: this module only draws
random numbers, multiplies them by the per-block deviations and applies RoPE.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SEED_BASE = 20261203
CHUNK = 2048
HEAD_DIM = 128

# stream identifiers for SeedSequence spawn keys
_S_SIGMA, _S_OUTLIER, _S_K, _S_V, _S_Q = range(5)


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    n_layers: int
    n_kv: int
    n_q: int
    batch: int
    T: int
    theta: float
    dtype: str                 # "f16" or "f32" input precision
    budgets: tuple             # ((k_bits, v_bits), ...)
    n_outliers: int            # outlier 2-D blocks per (layer, KV head)
    outlier_mult: float
    calib_tokens: int          # prefill chunk used for calibration, per sequence
    head_dim: int = HEAD_DIM

    @property
    def group(self) -> int:
        return self.n_q // self.n_kv


WORKLOADS = {
    # tiny single head, fp32, K4V4
    "tiny": Workload(0, "tiny", 1, 1, 1, 1, 1024, 1.0e4, "f32", ((4, 4),), 0, 10.0, 1024),
    # one Llama-3.1-8B-shaped layer at 32K
    "llama8b_32k": Workload(1, "llama8b_32k", 1, 8, 32, 1, 32768, 5.0e5, "f16",
                            ((2, 2), (3, 3), (4, 4)), 2, 10.0, 2048),
    # Qwen2.5-3B-shaped decode at 128K, packed K3V3 (the headline workload)
    "qwen3b_128k": Workload(2, "qwen3b_128k", 36, 2, 16, 1, 131072, 1.0e6, "f16",
                            ((3, 3),), 2, 10.0, 2048),
    # same shape at 512K, K2V2, split-K
    "qwen3b_512k": Workload(3, "qwen3b_512k", 36, 2, 16, 1, 524288, 1.0e6, "f16",
                            ((2, 2),), 2, 10.0, 2048),
    # batched decode, Llama-3.1-8B KV shape, 64 x 8192, K4V4
    "llama8b_b64": Workload(4, "llama8b_b64", 1, 8, 32, 64, 8192, 5.0e5, "f16",
                            ((4, 4),), 2, 10.0, 2048),
    # two query heads per KV head (a grouped-query ratio the library accepts that none of the
    # workloads above has), same key recipe, for parity only
    "gqa2_8k": Workload(5, "gqa2_8k", 1, 4, 8, 1, 8192, 1.0e6, "f16",
                        ((3, 3),), 2, 10.0, 2048),
}


def _rng(w: Workload, stream: int, layer: int, seq: int = 0, chunk: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(SEED_BASE + w.index, spawn_key=(stream, layer, seq, chunk))
    return np.random.Generator(np.random.PCG64(ss))


def block_index(head_dim: int, pairing: str) -> np.ndarray:
    """Block j of every dim i: half-split pairs (j, j+d/2); interleaved pairs (2j, 2j+1)."""
    i = np.arange(head_dim)
    if pairing == "half":
        return i % (head_dim // 2)
    if pairing == "interleaved":
        return i // 2
    raise ValueError(pairing)


def block_sigmas(w: Workload, layer: int) -> np.ndarray:
    """Per-(KV head, block) standard deviations: exp(N(0,1)), outlier blocks x outlier_mult."""
    nb = w.head_dim // 2
    sig = np.exp(_rng(w, _S_SIGMA, layer).standard_normal((w.n_kv, nb)))
    if w.n_outliers:
        r = _rng(w, _S_OUTLIER, layer)
        for h in range(w.n_kv):
            idx = r.choice(nb, size=w.n_outliers, replace=False)
            sig[h, idx] *= w.outlier_mult
    return sig


def seq_block_sigmas(w: Workload, layer: int, seq: int) -> np.ndarray:
    """Block deviations of one sequence in a batch whose sequences differ in kind: sequence 0
    has the layer's own (block_sigmas); sequence s > 0 an independent draw of the same law."""
    if seq == 0:
        return block_sigmas(w, layer)
    nb = w.head_dim // 2
    sig = np.exp(_rng(w, _S_SIGMA, layer, seq).standard_normal((w.n_kv, nb)))
    if w.n_outliers:
        r = _rng(w, _S_OUTLIER, layer, seq)
        for h in range(w.n_kv):
            idx = r.choice(nb, size=w.n_outliers, replace=False)
            sig[h, idx] *= w.outlier_mult
    return sig


def rope_frequencies(head_dim: int, theta: float) -> np.ndarray:
    j = np.arange(head_dim // 2, dtype=np.float64)
    return theta ** (-2.0 * j / head_dim)


def apply_rope(x: np.ndarray, positions: np.ndarray, theta: float, pairing: str = "half") -> np.ndarray:
    """Rotate x[..., t, (h,) d] by angle position*omega_j in each 2-D block, in float64.

    ``x`` has shape [n_pos, ..., d] where the leading axis matches ``positions``.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    nb = d // 2
    ang = np.asarray(positions, dtype=np.float64)[:, None] * rope_frequencies(d, theta)[None, :]
    shape = (ang.shape[0],) + (1,) * (x.ndim - 2) + (nb,)
    c = np.cos(ang).reshape(shape)
    s = np.sin(ang).reshape(shape)
    out = np.empty_like(x)
    if pairing == "half":
        a, b = x[..., :nb], x[..., nb:]
        out[..., :nb] = a * c - b * s
        out[..., nb:] = a * s + b * c
    elif pairing == "interleaved":
        a, b = x[..., 0::2], x[..., 1::2]
        out[..., 0::2] = a * c - b * s
        out[..., 1::2] = a * s + b * c
    else:
        raise ValueError(pairing)
    return out


def _noise(r: np.random.Generator, shape, noise: str) -> np.ndarray:
    if noise == "gauss":
        return r.standard_normal(shape)
    if noise == "t5":
        return r.standard_t(5.0, shape)
    raise ValueError(noise)


def to_input_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float16)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    raise ValueError(dtype)


def gen_layer(w: Workload, layer: int, t0: int, t1: int, seq: int = 0,
              noise: str = "gauss", pairing: str = "half",
              sigmas: Optional[np.ndarray] = None):
    """Keys (post-RoPE) and values for tokens [t0, t1) of one sequence of one layer.

    Returns (k, v) with shape [t1-t0, n_kv, head_dim] in the workload's input dtype.
    """
    d, nkv = w.head_dim, w.n_kv
    sig = block_sigmas(w, layer) if sigmas is None else sigmas
    jidx = block_index(d, pairing)
    sig_dim = sig[:, jidx]                                   # [n_kv, d]
    ks, vs = [], []
    c0, c1 = t0 // CHUNK, (t1 + CHUNK - 1) // CHUNK
    for c in range(c0, c1):
        lo, hi = max(t0, c * CHUNK), min(t1, (c + 1) * CHUNK)
        n = CHUNK
        zk = _noise(_rng(w, _S_K, layer, seq, c), (n, nkv, d), noise)[lo - c * CHUNK: hi - c * CHUNK]
        zv = _noise(_rng(w, _S_V, layer, seq, c), (n, nkv, d), noise)[lo - c * CHUNK: hi - c * CHUNK]
        pos = np.arange(lo, hi)
        ks.append(to_input_dtype(apply_rope(zk * sig_dim[None], pos, w.theta, pairing), w.dtype))
        vs.append(to_input_dtype(zv, w.dtype))
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def gen_query(w: Workload, layer: int, position: int, seq: int = 0, noise: str = "gauss",
              pairing: str = "half", sigmas: Optional[np.ndarray] = None) -> np.ndarray:
    """One decode query [n_q, head_dim] drawn like its KV head's keys, rotated at ``position``."""
    d = w.head_dim
    sig = block_sigmas(w, layer) if sigmas is None else sigmas
    sig_dim = sig[:, block_index(d, pairing)]                # [n_kv, d]
    kv_of_q = np.arange(w.n_q) // w.group
    z = _noise(_rng(w, _S_Q, layer, seq), (w.n_q, d), noise)
    q = apply_rope((z * sig_dim[kv_of_q])[None], np.array([position]), w.theta, pairing)[0]
    return to_input_dtype(q, w.dtype)
