"""Randomized Hadamard rotation of key rows (oracle; test infrastructure only).

RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract: the allocator sits on
top of TurboQuant-MSE (TQ-MSE).  TurboQuant's quantizer first applies a random
orthogonal rotation to the whole vector, so that every coordinate follows nearly
the same law, and then quantizes each coordinate with one scalar codebook.  The
pages do not describe the rotation.  Reading (the flat-vector uniform baseline):
  * R = H D / sqrt(d), with H the d x d Sylvester-Hadamard matrix (entries +-1) and
    D = diag(s) a random sign vector per (layer, KV head), supplied by the caller;
  * stored key input y = fp32(R k) (R k exact in fp64 for fp16 keys, one rounding
    at the division by sqrt(d) and one to fp32), quantized at the uniform width;
  * decode and diagnostics use k_hat = R^T y_hat = D H y_hat / sqrt(d); equivalently
    <q, k_hat> = <R q, y_hat>;
  * values are not rotated.
H x is computed with the fast Walsh-Hadamard transform: log2(d) stages of
butterflies (a, b) -> (a + b, a - b) over pairs at distance 1, 2, 4, ..., d/2.
"""
from __future__ import annotations

import numpy as np


def fwht(x: np.ndarray) -> np.ndarray:
    """H x along the last axis (length a power of two), in fp64, stage by stage."""
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    h = 1
    while h < d:
        v = y.reshape(*y.shape[:-1], d // (2 * h), 2, h)
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        h *= 2
    return y


def rotate(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """R x = H (s * x) / sqrt(d), fp64 (rows on the last axis)."""
    d = x.shape[-1]
    return fwht(np.asarray(x, dtype=np.float64) * np.asarray(signs, dtype=np.float64)) / np.sqrt(float(d))


def rotate_rows_fp32(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """The quantizer's input for rotated keys: fp32(R x)."""
    return rotate(x, signs).astype(np.float32)


def unrotate(y: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """R^T y = s * (H y) / sqrt(d), fp64."""
    d = y.shape[-1]
    return np.asarray(signs, dtype=np.float64) * fwht(y) / np.sqrt(float(d))
