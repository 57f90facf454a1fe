"""Per-head codec compositions (oracle; test infrastructure only).

Each codec of the cache is a short chain of the oracle's pinned steps.  This
module writes every chain out once, in the order of the readings, so that the
parity tests and the smoke run only call it:

Block-GTQ (RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract: the
per-block integer widths of the allocation on top of a TQ-MSE-style scalar
quantizer).  Keys: quantize.quantize_rows with the block widths and inverse
gains spread to dims; dequantized as s16 * g_j * CB_{b_j}[code].  Values: the
same quantizer at the uniform width B_V with unit gains.

Uniform quantizer on randomly rotated keys (same abstract, the TQ-MSE element:
a random rotation of the whole vector before one scalar codebook; reading: a
randomized Sylvester-Hadamard rotation with caller signs).  Keys: y =
rotation.rotate_rows_fp32(x, s), quantized at the uniform width with unit
gains; dequantized as R^T (s16 * CB[code]).

Block-GTQ rotated inside equal-width groups (same element, restricted so that no
rotation mixes blocks of different widths; reading).  Keys: v = fp32(x * ig)
(one fp32 multiply), y = fp32(R_groups v) with R_groups the chunked rotation of
rotation.rotate_in_groups over the plan's field order, then quantize_rows with
the block widths and unit gains; dequantized as g * R_groups^T (s16 * CB[code]).

256-value absmax codec (Pith review of NQKV, "What carries the argument" and
referee major comment 1: one absmax scale per block of 256 values of the
token's [n_kv * 128] vector, 16-level Gaussian-quantile codebook).  A block
spans two KV heads, so head h's 128 values sit in block h // 2 and take that
block's scale; dequantized as s16 * NF[code].
"""
from __future__ import annotations

import numpy as np

from . import allocation as al
from . import attention as at
from . import quantize as qz
from . import rotation as rt

HEAD_DIM = 128
NF_BLOCK = 256


# ---- Block-GTQ (and the unrotated uniform codec: widths all B_K, gains 1) ------------------

def quantize_bgtq_keys(k_rows, widths, ig, pairing="half"):
    """Key rows [N, 128] of one head with block widths [64] and inverse gains [64]:
    (codes uint8 [N, 128], s16 fp16 [N])."""
    wd = al.dim_widths(widths, HEAD_DIM, pairing)
    igd = al.dim_values(np.asarray(ig, np.float32), HEAD_DIM, pairing)
    codes, s16, _ = qz.quantize_rows(k_rows, wd, igd)
    return codes, s16


def dequant_bgtq_keys(codes, s16, widths, g, pairing="half"):
    wd = al.dim_widths(widths, HEAD_DIM, pairing)
    gd = al.dim_values(np.asarray(g, np.float32), HEAD_DIM, pairing)
    return at.dequant_k(codes, s16, wd, gd)


def quantize_values(v_rows, bits):
    """Value rows [N, 128] at the uniform width `bits`, unit gains: (codes, s16)."""
    codes, s16, _ = qz.quantize_rows(v_rows, np.full(HEAD_DIM, int(bits)))
    return codes, s16


def dequant_values(codes, s16, bits):
    return at.dequant_v(codes, s16, int(bits))


# ---- uniform quantizer on randomly rotated keys ------------------------------------------

def quantize_rotated_uniform(k_rows, bits, signs):
    """Stored input fp32(R k), R = H D / sqrt(128), quantized at `bits` with unit gains."""
    y = rt.rotate_rows_fp32(k_rows, signs)
    codes, s16, _ = qz.quantize_rows(y, np.full(HEAD_DIM, int(bits)))
    return codes, s16


def dequant_rotated_uniform(codes, s16, bits, signs):
    y_hat = at.dequant_k(codes, s16, np.full(HEAD_DIM, int(bits)), np.ones(HEAD_DIM, np.float32))
    return rt.unrotate(y_hat, signs)


# ---- Block-GTQ rotated inside equal-width groups -----------------------------------------

def group_rotated_input(k_rows, widths, ig, signs, pairing="half"):
    """The quantizer's input for the group-rotated codec: fp32(R_groups fp32(k * ig))."""
    igd = al.dim_values(np.asarray(ig, np.float32), HEAD_DIM, pairing)
    v = (np.asarray(k_rows).astype(np.float32) * igd.astype(np.float32)[None, :]).astype(np.float32)
    dims, ws = al.field_order(widths, HEAD_DIM, pairing)
    return rt.rotate_in_groups(v.astype(np.float64), signs, dims, ws).astype(np.float32)


def quantize_bgtq_group_rotated(k_rows, widths, ig, signs, pairing="half"):
    y = group_rotated_input(k_rows, widths, ig, signs, pairing)
    codes, s16, _ = qz.quantize_rows(y, al.dim_widths(widths, HEAD_DIM, pairing))
    return codes, s16


def dequant_bgtq_group_rotated(codes, s16, widths, g, signs, pairing="half"):
    wd = al.dim_widths(widths, HEAD_DIM, pairing)
    y_hat = at.dequant_k(codes, s16, wd, np.ones(HEAD_DIM, np.float32))
    dims, ws = al.field_order(widths, HEAD_DIM, pairing)
    gd = al.dim_values(np.asarray(g, np.float32), HEAD_DIM, pairing).astype(np.float64)
    return rt.unrotate_in_groups(y_hat, signs, dims, ws) * gd[None, :]


# ---- 256-value absmax codec, per-head slices -----------------------------------------------

def quantize_nf16_tokens(x_tok):
    """Token vectors [N, n_kv * 128]: (codes [N, n_kv * 128], block scales fp16 [N, n_kv * 128 / 256])."""
    codes, s16, _ = qz.quantize_nf16(x_tok, NF_BLOCK)
    return codes, s16


def nf16_head_slice(codes_tok, s16_blocks, h):
    """Head h's codes [N, 128] and scales [N]: its 128 values lie in 256-value block
    (128 h) // 256 = h // 2 of the token vector."""
    c = np.asarray(codes_tok)[:, h * HEAD_DIM:(h + 1) * HEAD_DIM]
    s = np.asarray(s16_blocks)[:, (h * HEAD_DIM) // NF_BLOCK]
    return c, s


def dequant_nf16_head(codes_h, s16_h):
    """s16 * NF[code] for one head's slice (every value of the slice shares its block's scale)."""
    return at.dequant_nf16(codes_h, np.asarray(s16_h)[:, None], block=HEAD_DIM)
