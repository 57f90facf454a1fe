"""Packed-cache bit layout (oracle; test infrastructure only).

The pages state that the cache is stored packed (RoPE-Aware Bit Allocation
for KV-Cache Quantization, abstract) and that the NQKV cache keeps codebook
indices plus block scales (Pith review, "What carries the argument"), but give
no layout.  The layout used here:

K rows.  One row per (sequence, KV head, token): the stored fields in plan
order (allocation.field_order), each field's code written least-significant
bit first into a little-endian stream of 32-bit words; a row is exactly
B_K * d / 32 words (widths sum to B_K * d bits).

V tiles.  Tokens are grouped in tiles of 128 positions.  Inside a tile the
codes are dim-major: for dim i, the 128 tokens' B_V-bit codes form one
LSB-first stream of 4 * B_V words (token tau at bit tau * B_V).  A tile is
d * 4 * B_V words.
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


def pack_v_tiles(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes[T, d] -> words uint32[ceil(T/128), d, 4*bits]; tokens past T are zero."""
    T, d = codes.shape
    nt = (T + V_TILE - 1) // V_TILE
    padded = np.zeros((nt * V_TILE, d), dtype=np.uint8)
    padded[:T] = codes
    # [tile, dim, token-in-tile]: each (tile, dim) row is one dim's 128-token stream
    streams = padded.reshape(nt, V_TILE, d).transpose(0, 2, 1).reshape(nt * d, V_TILE)
    w = np.zeros((nt * d, 4 * bits), dtype=np.uint32)
    for tau in range(V_TILE):
        _put(w, tau * bits, bits, streams[:, tau])
    return w.reshape(nt, d, 4 * bits)


def unpack_v_tiles(words: np.ndarray, bits: int, T: int) -> np.ndarray:
    nt, d, nw = words.shape
    flat = words.reshape(nt * d, nw)
    streams = np.zeros((nt * d, V_TILE), dtype=np.uint8)
    for tau in range(V_TILE):
        streams[:, tau] = _get(flat, tau * bits, bits)
    return streams.reshape(nt, d, V_TILE).transpose(0, 2, 1).reshape(nt * V_TILE, d)[:T]
