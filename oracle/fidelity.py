"""Key-cache fidelity diagnostics in fp64 (oracle; test infrastructure only).

What is measured, after the pages:
  * RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract: the method is
    judged by how well the stored keys preserve the query-key attention logits,
    as a per-layer mean absolute error (Block-GTQ against uniform TQ-MSE at 2 and
    3 bits per dimension, keys only);
  * KV Cache Quantization on WikiText-2 prompt 2048-token (train), evaluation
    results: the softmax KL divergence between the attention distributions.

Readings (the pages give neither formula):
  * the logit is the attention logit a_t = sigma * <q_h, k_t> with the decode
    path's softmax scale (1/sqrt(d) unless given), against the same with the
    dequantized key k_hat_t;
  * MAE is the mean of |a_t - a_hat_t| over the cached positions t, per query
    head;
  * KL is KL(softmax(a) || softmax(a_hat)): the full-precision distribution is
    the reference;
  * K-only: values play no part.
"""
from __future__ import annotations

import numpy as np


def _log_softmax(x: np.ndarray) -> np.ndarray:
    m = np.max(x)
    z = x - m
    return z - np.log(np.sum(np.exp(z)))


def logit_fidelity(q: np.ndarray, k: np.ndarray, k_hat: np.ndarray, scale=None):
    """q [H_q, d]; k, k_hat [H_kv, T, d] -> (mae [H_q], kl [H_q]) in fp64.

    Query head h reads KV head h // G (G = H_q / H_kv)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    k_hat = np.asarray(k_hat, dtype=np.float64)
    H_q, d = q.shape
    H_kv = k.shape[0]
    G = H_q // H_kv
    sc = 1.0 / np.sqrt(d) if scale is None or scale <= 0 else float(scale)
    mae = np.zeros(H_q)
    kl = np.zeros(H_q)
    for h in range(H_q):
        a = sc * (k[h // G] @ q[h])
        b = sc * (k_hat[h // G] @ q[h])
        mae[h] = np.mean(np.abs(a - b))
        la, lb = _log_softmax(a), _log_softmax(b)
        kl[h] = float(np.sum(np.exp(la) * (la - lb)))
    return mae, kl
