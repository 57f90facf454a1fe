"""RoPE-block energy score, per-block gains and greedy bit allocation (oracle).

Source: "RoPE-Aware Bit Allocation for KV-Cache Quantization", abstract.  With
RoPE, the logit a cached key will contribute splits into one term per 2-D
frequency block, each depending on the relative position; the method scores
every block of every (layer, KV head) by its energy, without labels, and hands
out integer widths greedily by marginal gain, so energetic blocks get more bits.

Readings (the pages give no formulas):
  * score: m_j = sum_t (k_{t,p0(j)}^2 + k_{t,p1(j)}^2) / (2T) over the keys the
    caller passes (keys only -> label-free; RoPE-invariant because a rotation
    keeps each block's norm); optional block weights give s_j = w_j m_j.
    Summation order, fixed so results are reproducible bit-for-bit: each
    term is x0*x0 + x1*x1 in fp64 (exact squares, one rounding); terms are
    added in token order inside 256-token chunks, chunk totals in chunk order;
    then one fp64 division by 2T.
  * pairing: half-split (j, j + d/2) by default, interleaved (2j, 2j+1) option.
  * one integer width b_j in [b_min, b_max] per block, shared by both of its
    coordinates; the row costs sum_j 2 b_j = B*d bits exactly.
  * greedy: start at b_min; (B - b_min) d/2 steps; each step raises the
    eligible block with the largest s_j * delta(b_j) (fp64 product of the fp64
    score and the fp32 delta); ties go to the smallest j.
  * gains: g_j = fp32(sqrt(m_j / mbar)), ig_j = fp32(1 / sqrt(m_j / mbar)) with
    mbar = (sum_j m_j, j ascending) / (d/2), all in fp64 before the final
    rounding; mbar = 0 -> g = ig = 1; m_j = 0 -> g_j = ig_j = 0.
  * field (plan) order: blocks by width descending, then j ascending; within a
    block coordinate p0 then p1; zero-width blocks store nothing.
"""
from __future__ import annotations

import numpy as np

ENERGY_CHUNK = 256


def block_pairs(head_dim: int, pairing: str = "half"):
    nb = head_dim // 2
    j = np.arange(nb)
    if pairing == "half":
        return j, j + nb
    if pairing == "interleaved":
        return 2 * j, 2 * j + 1
    raise ValueError(pairing)


def energy(keys: np.ndarray, pairing: str = "half") -> np.ndarray:
    """Per-(KV head, block) mean square m[h, j] of keys[T, H, d] (fp16/fp32 input)."""
    keys = np.asarray(keys)
    T, H, d = keys.shape
    if T == 0:
        raise ValueError("no calibration tokens")
    p0, p1 = block_pairs(d, pairing)
    x = keys.astype(np.float64)
    term = x[:, :, p0] * x[:, :, p0] + x[:, :, p1] * x[:, :, p1]      # [T, H, nb]
    total = np.zeros((H, d // 2), dtype=np.float64)
    for c0 in range(0, T, ENERGY_CHUNK):
        # add.accumulate is a strictly sequential running sum in token order
        chunk_sum = np.add.accumulate(term[c0:c0 + ENERGY_CHUNK], axis=0)[-1]
        total = total + chunk_sum
    return total / (2.0 * T)


def gains(m: np.ndarray):
    """(g, ig) fp32 per block from energies m[..., nb] (fp64)."""
    m = np.asarray(m, dtype=np.float64)
    nb = m.shape[-1]
    s = np.zeros(m.shape[:-1], dtype=np.float64)
    for j in range(nb):
        s = s + m[..., j]
    mbar = s / nb
    g = np.ones(m.shape, dtype=np.float32)
    ig = np.ones(m.shape, dtype=np.float32)
    for idx in np.ndindex(m.shape[:-1]):
        if mbar[idx] == 0.0:
            continue
        for j in range(nb):
            mj = m[idx + (j,)]
            if mj == 0.0:
                g[idx + (j,)] = 0.0
                ig[idx + (j,)] = 0.0
            else:
                r = np.sqrt(mj / mbar[idx])
                g[idx + (j,)] = np.float32(r)
                ig[idx + (j,)] = np.float32(1.0 / r)
    return g, ig


def greedy_allocate(scores: np.ndarray, budget_bits: int, b_min: int, b_max: int,
                    delta: np.ndarray) -> np.ndarray:
    """Integer widths b[nb] with sum 2 b_j = budget_bits * 2 nb, by marginal gain."""
    s = np.asarray(scores, dtype=np.float64)
    nb = s.size
    if not (b_min <= budget_bits <= b_max):
        raise ValueError("budget outside [b_min, b_max]")
    b = np.full(nb, b_min, dtype=np.int64)
    dl = np.asarray(delta, dtype=np.float32).astype(np.float64)
    for _ in range((budget_bits - b_min) * nb):
        gain = np.full(nb, -np.inf)
        ok = b < b_max
        gain[ok] = s[ok] * dl[b[ok]]
        j = int(np.argmax(gain))          # first maximum -> smallest j on ties
        b[j] += 1
    return b


def allocate(keys: np.ndarray, budget_bits: int, b_min: int = 0, b_max: int = 8,
             pairing: str = "half", block_weight=None, delta=None):
    """Full per-layer allocation for keys[T, H, d]: (widths[H, nb], g[H, nb], ig[H, nb], m)."""
    from .codebooks import delta_table
    dl = delta_table() if delta is None else delta
    m = energy(keys, pairing)
    sc = m if block_weight is None else m * np.asarray(block_weight, dtype=np.float64)
    widths = np.stack([greedy_allocate(sc[h], budget_bits, b_min, b_max, dl)
                       for h in range(m.shape[0])])
    g, ig = gains(m)
    return widths, g, ig, m


def field_order(widths: np.ndarray, head_dim: int, pairing: str = "half"):
    """Plan order of the stored fields of one head: (dims[n], widths[n]) for widths > 0."""
    w = np.asarray(widths)
    p0, p1 = block_pairs(head_dim, pairing)
    order = sorted(range(w.size), key=lambda j: (-int(w[j]), j))
    dims, ws = [], []
    for j in order:
        if w[j] == 0:
            continue
        dims += [int(p0[j]), int(p1[j])]
        ws += [int(w[j]), int(w[j])]
    return np.array(dims, dtype=np.int64), np.array(ws, dtype=np.int64)


def dim_widths(widths: np.ndarray, head_dim: int, pairing: str = "half") -> np.ndarray:
    """Width of every dim i (its block's width)."""
    p0, p1 = block_pairs(head_dim, pairing)
    out = np.zeros(head_dim, dtype=np.int64)
    out[p0] = widths
    out[p1] = widths
    return out


def dim_values(per_block: np.ndarray, head_dim: int, pairing: str = "half") -> np.ndarray:
    p0, p1 = block_pairs(head_dim, pairing)
    per_block = np.asarray(per_block)
    out = np.zeros(per_block.shape[:-1] + (head_dim,), dtype=per_block.dtype)
    out[..., p0] = per_block
    out[..., p1] = per_block
    return out
