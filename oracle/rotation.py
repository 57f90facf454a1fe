"""Randomized Hadamard rotations of key rows (oracle; test infrastructure only).

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


# ---- Block-GTQ with rotations inside equal-width groups -------------------------------------
# The allocation hands every RoPE block a width; a rotation that mixed blocks of different
# widths would undo it.  Reading (the "rotating within equal-width groups" variant of the
# TQ-MSE element): in the plan's field order (blocks by width descending, then index; p0 then
# p1) the fields of each width form one contiguous run.  Each run of n fields is cut into
# power-of-two chunks, largest first (its binary decomposition), and each chunk of m fields
# with dims d_0 .. d_{m-1} is rotated by H_m D / sqrt(m): y_{d_k} = sum_l H_m[k, l] s_{d_l}
# v_{d_l} / sqrt(m), with the caller's signs s indexed by dim.  The rotated input is the
# gain-normalised key v = fp32(x * ig); the stored input is fp32 of that rotation (fp64
# butterflies stage by stage, then the division by sqrt(m)).  Decode uses
# <q, g * R^T y_hat> = <R (g * q), y_hat>; width-0 blocks are not stored and not rotated.


def group_chunks(fwidths: np.ndarray):
    """Chunks (start, size) of the stored fields (widths in plan order, all > 0)."""
    out = []
    f, n = 0, len(fwidths)
    while f < n:
        e = f
        while e < n and fwidths[e] == fwidths[f]:
            e += 1
        run = e - f
        s = f
        for bit in range(7, -1, -1):
            if run & (1 << bit):
                out.append((s, 1 << bit))
                s += 1 << bit
        f = e
    return out


def rotate_in_groups(v: np.ndarray, signs: np.ndarray, fdims: np.ndarray, fwidths: np.ndarray) -> np.ndarray:
    """R v for rows v [N, 128] (dim layout), fp64; dims of width-0 blocks are passed through."""
    out = np.array(v, dtype=np.float64, copy=True)
    sg = np.asarray(signs, dtype=np.float64)
    for s, m in group_chunks(fwidths):
        d = np.asarray(fdims[s:s + m])
        out[:, d] = fwht(out[:, d] * sg[d]) / np.sqrt(float(m))
    return out


def unrotate_in_groups(y: np.ndarray, signs: np.ndarray, fdims: np.ndarray, fwidths: np.ndarray) -> np.ndarray:
    """R^T y (R is orthogonal: each chunk's inverse is D H_m / sqrt(m)), fp64."""
    out = np.array(y, dtype=np.float64, copy=True)
    sg = np.asarray(signs, dtype=np.float64)
    for s, m in group_chunks(fwidths):
        d = np.asarray(fdims[s:s + m])
        out[:, d] = fwht(out[:, d]) / np.sqrt(float(m)) * sg[d]
    return out
