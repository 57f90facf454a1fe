"""Scalar codebooks of the quantizers (oracle; test infrastructure only).

TQ-MSE-style codebook (reading).  The method's quantizer derives from
TurboQuant-MSE (RoPE-Aware Bit Allocation for KV-Cache Quantization,
abstract), but the pages print no codebook.  The reading taken here is the MSE-optimal
(Lloyd-Max) 2^b-level scalar quantizer for a standard normal, with no random
rotation; its centroids are rounded once to fp16 (round-to-nearest-even) and
those fp16 values *are* the codebook.  Decision boundaries are the fp32
rounding of the exact midpoint of neighbouring fp16 centroids.

Greedy gains (reading).  The allocator raises widths by marginal gain; the gain
of raising a block from b to b+1 bits is taken as delta(b) = c(b) - c(b+1)
rounded once to fp32, where c(b) is the exact N(0,1) mean squared error of the
b-bit codebook above (c(0) = 1: a zero-width block reconstructs 0).

16-level Gaussian-quantile codebook (reading).  The NQKV review describes a
fixed codebook of sixteen standard-normal quantiles, applied after each block
is divided by its absolute maximum ("What carries the argument"; referee major
comment 1).  The level
values are not printed; the reading is the equal-mass bin midpoints
Phi^-1((k + 1/2)/16), divided by Phi^-1(31/32) so the end levels are +-1,
rounded to fp16, with fp32 midpoint boundaries.
"""
from __future__ import annotations

import functools
import math
from statistics import NormalDist

import numpy as np

_SQRT2 = math.sqrt(2.0)
_SQRT2PI = math.sqrt(2.0 * math.pi)
MAX_BITS = 8


def upper_tail(x: float) -> float:
    """Q(x) = P(Z > x) for Z ~ N(0,1); +inf -> 0, -inf -> 1."""
    if x == math.inf:
        return 0.0
    if x == -math.inf:
        return 1.0
    return 0.5 * math.erfc(x / _SQRT2)


def density(x: float) -> float:
    if math.isinf(x):
        return 0.0
    return math.exp(-0.5 * x * x) / _SQRT2PI


def _cell_mass(a: float, b: float) -> float:
    """P(a < Z <= b), evaluated in the tail that keeps precision."""
    if a >= 0.0:
        return upper_tail(a) - upper_tail(b)
    if b <= 0.0:
        return upper_tail(-b) - upper_tail(-a)
    return 1.0 - upper_tail(b) - upper_tail(-a)


def lloyd_max_real(bits: int) -> np.ndarray:
    """fp64 centroids of the 2^bits-level Lloyd-Max quantizer of N(0,1).

    Solves the two optimality conditions (each centroid is the conditional
    mean of its cell; each boundary is the midpoint of its two centroids) by
    Newton's method on F(c) = E[Z | cell(c)] - c, starting from the
    equal-mass quantiles, until the Newton step is below 1e-15.
    """
    L = 1 << bits
    nd = NormalDist()
    c = np.array([nd.inv_cdf((k + 0.5) / L) for k in range(L)], dtype=np.float64)
    for _ in range(200):
        lo = [-math.inf] + [0.5 * (c[k - 1] + c[k]) for k in range(1, L)]
        hi = [0.5 * (c[k] + c[k + 1]) for k in range(L - 1)] + [math.inf]
        F = np.zeros(L)
        J = np.zeros((L, L))
        for k in range(L):
            P = _cell_mass(lo[k], hi[k])
            mu = (density(lo[k]) - density(hi[k])) / P
            F[k] = mu - c[k]
            J[k, k] = -1.0
            # d mu / d lo = dens(lo) (mu - lo) / P ; d mu / d hi = dens(hi) (hi - mu) / P
            if k > 0:
                dlo = density(lo[k]) * (mu - lo[k]) / P
                J[k, k - 1] += 0.5 * dlo
                J[k, k] += 0.5 * dlo
            if k < L - 1:
                dhi = density(hi[k]) * (hi[k] - mu) / P
                J[k, k + 1] += 0.5 * dhi
                J[k, k] += 0.5 * dhi
        step = np.linalg.solve(J, -F)
        c = c + step
        if np.max(np.abs(step)) < 1e-15:
            break
    # exact symmetry of the N(0,1) optimum
    return 0.5 * (c - c[::-1])


@functools.lru_cache(maxsize=None)
def _codebook_cached(bits: int):
    if not 1 <= bits <= MAX_BITS:
        raise ValueError("bits must be in [1, 8]")
    cb = lloyd_max_real(bits).astype(np.float16)        # fp64 -> fp16, RNE, one rounding
    mid = 0.5 * (cb[:-1].astype(np.float64) + cb[1:].astype(np.float64))  # exact in fp64
    bd = mid.astype(np.float32)                          # one RNE rounding to fp32
    cb.setflags(write=False)
    bd.setflags(write=False)
    return cb, bd


def codebook(bits: int) -> np.ndarray:
    """fp16 centroids CB_bits[0 .. 2^bits - 1], ascending."""
    return _codebook_cached(bits)[0]


def boundaries(bits: int) -> np.ndarray:
    """fp32 decision boundaries beta_bits[0 .. 2^bits - 2], ascending."""
    return _codebook_cached(bits)[1]


def mse_of(centroids: np.ndarray, bounds: np.ndarray) -> float:
    """Exact E[(Z - q(Z))^2] for Z ~ N(0,1) and a symmetric scalar quantizer.

    Cell k is (bounds[k-1], bounds[k]] with reconstruction centroids[k].  Uses
    the per-cell closed form
      (1 + c^2) P(cell) - 2 c (dens(a) - dens(b)) + (a dens(a) - b dens(b))
    summed over the non-negative half and doubled (the quantizer is symmetric
    and the middle boundary is 0).
    """
    c = np.asarray(centroids, dtype=np.float64)
    bd = np.asarray(bounds, dtype=np.float64)
    L = c.size
    assert L % 2 == 0 and bd[L // 2 - 1] == 0.0
    total = 0.0
    for k in range(L // 2, L):
        a = bd[k - 1]
        b = bd[k] if k < L - 1 else math.inf
        P = _cell_mass(a, b)
        ea, eb = density(a), density(b)
        xa = a * ea
        xb = 0.0 if math.isinf(b) else b * eb
        total += (1.0 + c[k] * c[k]) * P - 2.0 * c[k] * (ea - eb) + (xa - xb)
    return 2.0 * total


@functools.lru_cache(maxsize=None)
def distortion(bits: int) -> float:
    """c(b): exact N(0,1) MSE of the b-bit fp16 codebook; c(0) = 1."""
    if bits == 0:
        return 1.0
    return mse_of(codebook(bits).astype(np.float64), boundaries(bits).astype(np.float64))


def delta_table() -> np.ndarray:
    """delta(b) = fp32(c(b) - c(b+1)) for b = 0 .. 7 (gain of the (b+1)-th bit)."""
    return np.array([distortion(b) - distortion(b + 1) for b in range(MAX_BITS)],
                    dtype=np.float64).astype(np.float32)


def nf16_real() -> np.ndarray:
    """fp64 levels Phi^-1((k + 1/2)/16) / Phi^-1(31/32), k = 0 .. 15."""
    nd = NormalDist()
    z = nd.inv_cdf(31.0 / 32.0)
    return np.array([nd.inv_cdf((k + 0.5) / 16.0) / z for k in range(16)], dtype=np.float64)


def nf16_levels() -> np.ndarray:
    return nf16_real().astype(np.float16)


def nf16_boundaries() -> np.ndarray:
    lv = nf16_levels().astype(np.float64)
    return (0.5 * (lv[:-1] + lv[1:])).astype(np.float32)
