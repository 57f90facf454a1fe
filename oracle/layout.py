"""Packed-cache bit layout (oracle; test infrastructure only).

The pages state that the cache is stored packed (RoPE-Aware Bit Allocation
for KV-Cache Quantization, abstract) and that the NQKV cache keeps codebook
indices plus block scales (Pith review, "What carries the argument"), but give
no layout.  The layout used here:

K rows.  One row per (sequence, KV head, token): the stored fields in plan
order (allocation.field_order), each field's code written least-significant
bit first into a little-endian stream of 32-bit words; a row is exactly
B_K * d / 32 words (widths sum to B_K * d bits).

V tiles.  Tokens are grouped in tiles of 128 positions.  Inside a tile, the
codes of one dim for 32 consecutive tokens form a segment: an LSB-first stream
of B_V words (token 32g + e of the tile at bit e * B_V).  The 128 dims x 4
token groups = 512 segments are stored in the order (dim // 16, g, dim % 16),
i.e. segment index ((dim // 16) * 4 + g) * 16 + dim % 16, so that 64
consecutive segments are the 16 dims x 4 token groups of one 16-dim slice.
A tile is 512 * B_V words.
"""
from __future__ import annotations

import numpy as np

V_TILE = 128


def _put(words: np.ndarray, col_bit: int, w: int, vals: np.ndarray):
    wi, sh = divmod(col_bit, 32)
    v = vals.astype(np.uint64)
    words[:, wi] |= ((v << np.uint64(sh)) & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    if sh + w > 32:
        words[:, wi + 1] |= (v >> np.uint64(32 - sh)).astype(np.uint32)


def _get(words: np.ndarray, col_bit: int, w: int) -> np.ndarray:
    wi, sh = divmod(col_bit, 32)
    lo = words[:, wi].astype(np.uint64)
    if sh + w > 32:
        lo = lo | (words[:, wi + 1].astype(np.uint64) << np.uint64(32))
    return ((lo >> np.uint64(sh)) & np.uint64((1 << w) - 1)).astype(np.uint8)


def pack_k_rows(codes: np.ndarray, fdims: np.ndarray, fwidths: np.ndarray, n_words: int) -> np.ndarray:
    """codes[N, d] -> words uint32[N, n_words] with fields (fdims, fwidths) in order."""
    N = codes.shape[0]
    words = np.zeros((N, n_words), dtype=np.uint32)
    pos = 0
    for i, w in zip(fdims, fwidths):
        _put(words, pos, int(w), codes[:, int(i)])
        pos += int(w)
    assert pos == 32 * n_words, "fields must fill the row exactly"
    return words


def unpack_k_rows(words: np.ndarray, fdims: np.ndarray, fwidths: np.ndarray, head_dim: int) -> np.ndarray:
    codes = np.zeros((words.shape[0], head_dim), dtype=np.uint8)
    pos = 0
    for i, w in zip(fdims, fwidths):
        codes[:, int(i)] = _get(words, pos, int(w))
        pos += int(w)
    return codes


def _v_segments(codes: np.ndarray):
    """codes[T, 128] -> (segments[nt * 512, 32] in storage order, nt); tokens past T are 0."""
    T, d = codes.shape
    assert d == 128
    nt = (T + V_TILE - 1) // V_TILE
    padded = np.zeros((nt * V_TILE, d), dtype=np.uint8)
    padded[:T] = codes
    x = padded.reshape(nt, 4, 32, 8, 16)             # [tile, g, e, dim//16, dim%16]
    x = x.transpose(0, 3, 1, 4, 2)                    # [tile, dim//16, g, dim%16, e]
    return x.reshape(nt * 512, 32), nt


def pack_v_tiles(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes[T, 128] -> words uint32[ceil(T/128), 512, bits]."""
    seg, nt = _v_segments(codes)
    w = np.zeros((nt * 512, bits), dtype=np.uint32)
    for e in range(32):
        _put(w, e * bits, bits, seg[:, e])
    return w.reshape(nt, 512, bits)


def unpack_v_tiles(words: np.ndarray, bits: int, T: int) -> np.ndarray:
    nt = words.shape[0]
    flat = words.reshape(nt * 512, bits)
    seg = np.zeros((nt * 512, 32), dtype=np.uint8)
    for e in range(32):
        seg[:, e] = _get(flat, e * bits, bits)
    x = seg.reshape(nt, 8, 4, 16, 32).transpose(0, 2, 4, 1, 3)   # [tile, g, e, dim//16, dim%16]
    return x.reshape(nt * V_TILE, 128)[:T]
