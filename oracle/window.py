"""The fp16 recent window (oracle; test infrastructure only).

RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract: the paper reports its
results with no fp16 buffer of recent keys, which names the variant where the most recent
tokens are held in fp16 rather than in the low-bit cache; the leaderboard (KV Cache
Quantization on WikiText-2 prompt 2048-token (train)) has a buffer-setting column for it.  The pages do not describe the buffer.  Readings:
  * after every append, the last min(len, R) positions of the sequence are held as
    fp16 copies of their K and V rows (both: the buffer is read as one of recent tokens);
  * a position is quantized when it leaves the window, from its fp16 copy; a
    position that is already outside the window when it is appended is quantized
    from the input as given;
  * decode reads the window's fp16 values as they are (no scale, no codebook).
The KIVI-style codec quantizes keys per channel over whole 128-position tiles, so its
packed storage only ever holds whole tiles (the `group` argument below).
"""
from __future__ import annotations

import numpy as np


def packed_len(length: int, R: int, group: int = 1) -> int:
    """Positions held by the packed cache after `length` appended positions.  With group > 1
    (the KIVI-style codec's 128-position key tiles) only whole groups are packed: the largest
    multiple of `group` not above max(0, length - R)."""
    p = max(0, length - R) if R > 0 else length
    return p // group * group


def through_fp16(bounds, R: int, group: int = 1) -> np.ndarray:
    """Which positions were ever held in fp16, for appends of positions [bounds[i],
    bounds[i+1]): position p of an append ending at z is held in fp16 iff
    p >= packed_len(z, R, group).  Returns a bool array over [0, bounds[-1])."""
    T = bounds[-1]
    mask = np.zeros(T, dtype=bool)
    if R <= 0 and group == 1:
        return mask
    for a, z in zip(bounds[:-1], bounds[1:]):
        mask[max(a, packed_len(z, R, group)):z] = True
    return mask


def stored_rows(x: np.ndarray, bounds, R: int, group: int = 1) -> np.ndarray:
    """The rows each position is stored from: x rounded to fp16 where the position went
    through fp16, x itself elsewhere (x: [..., T, ...] with positions on axis 0)."""
    m = through_fp16(bounds, R, group)
    out = np.array(x, copy=True)
    out[m] = np.asarray(x[m]).astype(np.float16).astype(out.dtype)
    return out
