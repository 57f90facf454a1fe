"""The fp16 recent window (oracle; test infrastructure only).

RoPE-Aware Bit Allocation for KV-Cache Quantization, abstract: the paper's results
are stated "without an fp16 recent-key buffer", i.e. a variant in which the most
recent tokens are held in fp16 rather than in the low-bit cache; the leaderboard
(KV Cache Quantization on WikiText-2 prompt 2048-token (train)) lists this as its
"Buffer Setting".  The pages do not describe the buffer.  Readings:
  * after every append, the last min(len, R) positions of the sequence are held as
    fp16 copies of their K and V rows (both, as "recent tokens");
  * a position is quantized when it leaves the window, from its fp16 copy; a
    position that is already outside the window when it is appended is quantized
    from the input as given;
  * decode reads the window's fp16 values as they are (no scale, no codebook).
"""
from __future__ import annotations

import numpy as np


def packed_len(length: int, R: int) -> int:
    """Positions held by the packed cache after `length` appended positions."""
    return max(0, length - R) if R > 0 else length


def through_fp16(bounds, R: int) -> np.ndarray:
    """Which positions were ever inside the window, for appends of positions
    [bounds[i], bounds[i+1]): position p of an append ending at z enters the window iff
    p >= z - R.  Returns a bool array over [0, bounds[-1])."""
    T = bounds[-1]
    mask = np.zeros(T, dtype=bool)
    if R <= 0:
        return mask
    for a, z in zip(bounds[:-1], bounds[1:]):
        mask[max(a, z - R):z] = True
    return mask


def stored_rows(x: np.ndarray, bounds, R: int) -> np.ndarray:
    """The rows each position is stored from: x rounded to fp16 where the position went
    through the window, x itself elsewhere (x: [..., T, ...] with positions on axis 0)."""
    m = through_fp16(bounds, R)
    out = np.array(x, copy=True)
    out[m] = np.asarray(x[m]).astype(np.float16).astype(out.dtype)
    return out
