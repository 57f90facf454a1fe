"""Dequantization and fp64 GQA decode attention (oracle; test infrastructure only).

Decode attention over the packed cache (RoPE-Aware Bit Allocation for
KV-Cache Quantization, abstract: its serving path decodes directly from a
packed K3V3 cache at 128K context).  Readings:

  * the dequantized cache: K x_hat = s16 * g_{j(i)} * CB_{b_i}[code] (0 when
    b_i = 0); V x_hat = s16 * CB_{B_V}[code]; the 256-value absmax codec
    x_hat = s16 * NF[code]; all evaluated in fp64 from the stored integers and
    fp16/fp32 numbers;
  * logits l_{h,t} = sigma * <q_h, x_hat^K_{kv(h),t}> with sigma = 1/sqrt(d)
    unless given, kv(h) = floor(h / G) (contiguous grouped-query mapping);
  * p = softmax over the cached tokens (max subtracted), o_h = sum_t p_t x_hat^V_t.

RoPE block identity (same abstract: the logit splits into per-block terms
that depend on the relative position): with q = R(m) q0 and k = R(n) k0,
q . k = sum_j q0_j^T R((n - m) w_j) k0_j.
"""
from __future__ import annotations

import numpy as np

from . import codebooks as cbk
from .allocation import block_pairs


def dequant_k(codes: np.ndarray, s16: np.ndarray, width_dim: np.ndarray, g_dim: np.ndarray) -> np.ndarray:
    """codes[N, d], s16[N] -> fp64 [N, d]."""
    N, d = codes.shape
    out = np.zeros((N, d), dtype=np.float64)
    s = np.asarray(s16, dtype=np.float16).astype(np.float64)
    g = np.asarray(g_dim, dtype=np.float32).astype(np.float64)
    for i in range(d):
        w = int(width_dim[i])
        if w == 0:
            continue
        cb = cbk.codebook(w).astype(np.float64)
        out[:, i] = s * g[i] * cb[codes[:, i]]
    return out


def dequant_v(codes: np.ndarray, s16: np.ndarray, bits: int) -> np.ndarray:
    cb = cbk.codebook(bits).astype(np.float64)
    s = np.asarray(s16, dtype=np.float16).astype(np.float64)
    return s[:, None] * cb[codes]


def dequant_nf16(codes: np.ndarray, s16: np.ndarray, block: int = 256) -> np.ndarray:
    """codes[N, n], s16[N, n // block] -> fp64 [N, n]."""
    lv = cbk.nf16_levels().astype(np.float64)
    s = np.repeat(np.asarray(s16, dtype=np.float16).astype(np.float64), block, axis=1)
    return s * lv[codes]


def decode_attention(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, scale=None) -> np.ndarray:
    """q[H_q, d]; k_hat, v_hat [H_kv, T, d] (fp64) -> out [H_q, d] fp64."""
    q = np.asarray(q, dtype=np.float64)
    H_q, d = q.shape
    H_kv = k_hat.shape[0]
    G = H_q // H_kv
    sc = 1.0 / np.sqrt(d) if scale is None or scale <= 0 else float(scale)
    out = np.zeros((H_q, d), dtype=np.float64)
    for h in range(H_q):
        kv = h // G
        logits = sc * (k_hat[kv] @ q[h])
        p = np.exp(logits - logits.max())
        p /= p.sum()
        out[h] = p @ v_hat[kv]
    return out


def rope_block_logit(q0: np.ndarray, k0: np.ndarray, m: int, n: int, theta: float,
                     pairing: str = "half") -> float:
    """sum_j q0_j^T R((n - m) w_j) k0_j for pre-rotation q0, k0 [d] (fp64)."""
    d = q0.size
    p0, p1 = block_pairs(d, pairing)
    w = theta ** (-2.0 * np.arange(d // 2) / d)
    total = 0.0
    for j in range(d // 2):
        a = (n - m) * w[j]
        R = np.array([[np.cos(a), -np.sin(a)], [np.sin(a), np.cos(a)]])
        qj = np.array([q0[p0[j]], q0[p1[j]]], dtype=np.float64)
        kj = np.array([k0[p0[j]], k0[p1[j]]], dtype=np.float64)
        total += float(qj @ (R @ kj))
    return total


def bytes_per_token_head(k_bits: int, v_bits: int, head_dim: int = 128) -> float:
    """Packed bytes per cached token per KV head: codes + one fp16 scale each for K and V."""
    return (k_bits + v_bits) * head_dim / 8.0 + 4.0


def nf16_bytes_per_token_head(head_dim: int = 128, block: int = 256) -> float:
    """4-bit codes for K and V plus their share of the per-256-value fp16 scales."""
    return 2 * (head_dim * 4 / 8.0 + 2.0 * head_dim / block)


def compression_ratio(k_bits: int, v_bits: int, head_dim: int = 128) -> float:
    """fp16 K+V bytes over packed bytes, per token and KV head (plan amortised away)."""
    return (2 * 2 * head_dim) / bytes_per_token_head(k_bits, v_bits, head_dim)
