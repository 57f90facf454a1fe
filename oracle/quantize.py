"""Row quantizers (oracle; test infrastructure only).

Block-GTQ / TQ-MSE-style codec (reading of "RoPE-Aware Bit Allocation for
KV-Cache Quantization", abstract: a TQ-MSE-based quantizer with a per-token
scale, codebook lookup and per-block integer widths).  For one token row x of
one KV head, in this exact order of IEEE operations:

  1. x -> fp32 (exact for fp16 / fp32 input)
  2. y_i = x_i * ig_{j(i)}                       fp32 multiply (ig = 1 for V)
  3. ss  = sum_i y_i^2, i ascending              fp64 (squares exact)
  4. s16 = fp16(fp32(sqrt(ss / d)))              fp64 sqrt, then two roundings
  5. is  = 0 if s16 == 0 else fp32(1 / s16)      correctly rounded fp32 divide
  6. u_i = y_i * is                              fp32 multiply
  7. code_i = #{k : beta_{b_i}[k] < u_i}         exact fp32 compares; a u on a
                                                 boundary takes the lower code

NQKV-style codec (Pith review of arXiv 2505.16210, "What carries the
argument" and referee major comment 1; block size 256 from "Assumptions &
free parameters"): per token, each run of 256 consecutive values of the
token's [H_kv * d] vector is scaled by its absolute maximum, with no mean
subtraction, and mapped to the 16-level Gaussian-quantile codebook:

  a = max_i |x_i| (fp32), s16 = fp16(a), is = 0 if s16 == 0 else fp32(1/s16),
  u_i = x_i * is (fp32), code_i = #{k : beta^NF[k] < u_i}.
"""
from __future__ import annotations

import numpy as np

from . import codebooks as cbk


def row_scale(y32: np.ndarray):
    """(s16, is32) for rows y32[N, d] (fp32), steps 3-5 above."""
    y64 = y32.astype(np.float64)
    ss = np.zeros(y32.shape[0], dtype=np.float64)
    for i in range(y32.shape[1]):
        ss = ss + y64[:, i] * y64[:, i]
    s32 = np.sqrt(ss / y32.shape[1]).astype(np.float32)
    s16 = s32.astype(np.float16)
    s16f = s16.astype(np.float32)
    with np.errstate(divide="ignore"):
        is32 = np.where(s16f == 0, np.float32(0), np.float32(1) / s16f).astype(np.float32)
    return s16, is32


def code_of(u: np.ndarray, bounds: np.ndarray) -> np.ndarray:
    """#{k : bounds[k] < u} elementwise."""
    return np.searchsorted(np.asarray(bounds, dtype=np.float32), u.astype(np.float32),
                           side="left").astype(np.uint8)


def quantize_rows(x: np.ndarray, width_dim: np.ndarray, ig_dim=None):
    """Quantize rows x[N, d] with per-dim widths (0..8) and per-dim inverse gains.

    Returns (codes uint8[N, d] with 0 where width is 0, s16 fp16[N], u fp32[N, d]).
    """
    x32 = np.asarray(x).astype(np.float32)
    ig = np.ones(x32.shape[1], np.float32) if ig_dim is None else np.asarray(ig_dim, np.float32)
    y = (x32 * ig[None, :]).astype(np.float32)
    s16, is32 = row_scale(y)
    u = (y * is32[:, None]).astype(np.float32)
    codes = np.zeros(x32.shape, dtype=np.uint8)
    wd = np.asarray(width_dim)
    for i in range(x32.shape[1]):
        if wd[i] > 0:
            codes[:, i] = code_of(u[:, i], cbk.boundaries(int(wd[i])))
    return codes, s16, u


def quantize_nf16(x_tok: np.ndarray, block: int = 256):
    """Absmax NF16 codec over rows x_tok[N, n] (n a multiple of ``block``).

    Returns (codes uint8[N, n], s16 fp16[N, n // block], u fp32[N, n]).
    """
    x32 = np.asarray(x_tok).astype(np.float32)
    N, n = x32.shape
    nblk = n // block
    xb = x32.reshape(N, nblk, block)
    a = np.max(np.abs(xb), axis=2)
    s16 = a.astype(np.float16)
    s16f = s16.astype(np.float32)
    with np.errstate(divide="ignore"):
        is32 = np.where(s16f == 0, np.float32(0), np.float32(1) / s16f).astype(np.float32)
    u = (xb * is32[:, :, None]).astype(np.float32).reshape(N, n)
    codes = code_of(u, cbk.nf16_boundaries())
    return codes, s16, u
