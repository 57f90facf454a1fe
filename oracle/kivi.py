"""KIVI-style asymmetric integer codec (oracle; test infrastructure only).

The leaderboard (KV Cache Quantization on WikiText-2 prompt 2048-token (train)) compares
Block-GTQ and TQ-MSE with KIVI, which the NQKV review's reference list describes as a
streaming, asymmetric quantizer; the review's ablation table (KVQuant row) gives the split
that method family uses: keys quantized per channel, values per token.  The pages
give no formulas.  Readings (the plainest asymmetric min/max integer quantizer):

  For a group of values x (fp32 as given; fp16 inputs are exact) and a width b,
  L = 2^b levels, in this exact order of IEEE operations:
    1. lo = fp16(min x), hi = fp16(max x)            (nearest-even roundings)
    2. d  = fp32(hi) - fp32(lo)                      fp32 subtract
    3. s  = fp16(fp32(d / (L - 1)))                  fp32 divide, then fp16
    4. is = 0 if s == 0 else fp32(1 / s)             correctly rounded fp32 divide
    5. u  = fp32(fp32(x - lo) * is)                  fp32 subtract, fp32 multiply
    6. code = min(max(rint(u), 0), L - 1)            rint: nearest, ties to even
  Reconstruction: x_hat = fp16(lo + s * code), the exact value rounded once to fp16.

  Groups: a key group is one channel over the 128 positions of a 128-position tile
  (position tiles 128 i .. 128 i + 127); a value group is one position's 128 channels.
  A key tile is quantized once all of its positions are known.  Until then ("streaming")
  the positions of the last incomplete tile are held in fp16, as are, with a recent window
  R, the positions after the largest multiple of 128 not above len - R
  (oracle.window.packed_len with group 128).

Stored layout of the parameters (for the parity dumps), fp16, per (sequence, KV head):
  keys   [tile][block j][s(p0), s(p1), lo(p0), lo(p1)]  (p0, p1 = the dims of RoPE block j)
  values [tile][2][128 positions]                       (the tile's s, then its lo)
Codes are packed like the uniform codec's: K rows in the uniform plan's field order, V in
the 128-position tile segments.
"""
from __future__ import annotations

import numpy as np

from . import allocation as al

TILE = 128


def quantize_groups(x: np.ndarray, bits: int):
    """Quantize every row of x [N, n] as one group (steps 1-6).  Returns (codes int64 [N, n],
    s16 [N], lo16 [N])."""
    L = 1 << bits
    x32 = np.asarray(x).astype(np.float32)
    lo16 = x32.min(axis=1).astype(np.float16)
    hi16 = x32.max(axis=1).astype(np.float16)
    d = hi16.astype(np.float32) - lo16.astype(np.float32)
    s16 = (d / np.float32(L - 1)).astype(np.float32).astype(np.float16)
    s32 = s16.astype(np.float32)
    with np.errstate(divide="ignore"):
        is32 = np.where(s32 == 0, np.float32(0), np.float32(1) / np.where(s32 == 0, np.float32(1), s32))
    is32 = is32.astype(np.float32)
    u = ((x32 - lo16.astype(np.float32)[:, None]).astype(np.float32) * is32[:, None]).astype(np.float32)
    codes = np.clip(np.rint(u), 0, L - 1).astype(np.int64)
    return codes, s16, lo16


def reconstruct(codes: np.ndarray, s16: np.ndarray, lo16: np.ndarray) -> np.ndarray:
    """x_hat = fp16(lo + s * code) (exact in fp64, one rounding), returned as fp64.  s16 and
    lo16 broadcast against codes."""
    exact = np.asarray(lo16, dtype=np.float64) + np.asarray(s16, dtype=np.float64) * codes.astype(np.float64)
    return exact.astype(np.float16).astype(np.float64)


def quantize_k_tile(xk: np.ndarray, bits: int):
    """Keys of one complete tile [128 positions, 128 dims]: one group per channel.  Returns
    (codes [128, 128] position-major, s16 [128 dims], lo16 [128 dims])."""
    assert xk.shape[0] == TILE
    c, s16, lo16 = quantize_groups(np.asarray(xk).T, bits)
    return c.T, s16, lo16


def quantize_k(xk: np.ndarray, bits: int):
    """Keys [n_tiles * 128, 128]: tile by tile.  Returns (codes, s16 [n_tiles, 128],
    lo16 [n_tiles, 128])."""
    n = xk.shape[0]
    assert n % TILE == 0
    cs, ss, ls = [], [], []
    for t in range(n // TILE):
        c, s, lo = quantize_k_tile(xk[t * TILE:(t + 1) * TILE], bits)
        cs.append(c)
        ss.append(s)
        ls.append(lo)
    if not cs:
        return np.zeros((0, xk.shape[1]), np.int64), np.zeros((0, xk.shape[1]), np.float16), \
            np.zeros((0, xk.shape[1]), np.float16)
    return np.concatenate(cs), np.stack(ss), np.stack(ls)


def quantize_v(xv: np.ndarray, bits: int):
    """Values [N, 128]: one group per position.  Returns (codes, s16 [N], lo16 [N])."""
    return quantize_groups(xv, bits)


def dequant_k(codes: np.ndarray, s16: np.ndarray, lo16: np.ndarray) -> np.ndarray:
    """Reconstructed keys [n_tiles * 128, 128] from per-tile channel parameters."""
    nt = s16.shape[0]
    out = np.empty(codes.shape, dtype=np.float64)
    for t in range(nt):
        out[t * TILE:(t + 1) * TILE] = reconstruct(codes[t * TILE:(t + 1) * TILE], s16[t][None, :], lo16[t][None, :])
    return out


def dequant_v(codes: np.ndarray, s16: np.ndarray, lo16: np.ndarray) -> np.ndarray:
    return reconstruct(codes, s16[:, None], lo16[:, None])


def k_params_layout(s16: np.ndarray, lo16: np.ndarray, pairing: str = "half") -> np.ndarray:
    """Stored key parameters [n_tiles, 64, 4] fp16 from s16, lo16 [n_tiles, 128]."""
    p0, p1 = al.block_pairs(s16.shape[1], pairing)
    return np.stack([s16[:, p0], s16[:, p1], lo16[:, p0], lo16[:, p1]], axis=-1)


def v_params_layout(s16: np.ndarray, lo16: np.ndarray) -> np.ndarray:
    """Stored value parameters [n_tiles, 2, 128] fp16 from per-position s16, lo16 [n_tiles * 128]."""
    nt = s16.shape[0] // TILE
    return np.stack([s16.reshape(nt, TILE), lo16.reshape(nt, TILE)], axis=1)


def bytes_per_token_head(k_bits: int, v_bits: int, head_dim: int = 128) -> float:
    """Packed codes plus parameters: keys' 2 fp16 per channel per 128 positions, values'
    2 fp16 per position."""
    return (k_bits + v_bits) * head_dim / 8 + 2 * 2 * head_dim / TILE + 2 * 2
