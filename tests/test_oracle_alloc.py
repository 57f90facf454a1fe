"""Pins of oracle.allocation: budget identity, brute-force optimality, invariants, sum order."""
import itertools
import math

import numpy as np
import pytest

from oracle import allocation as al
from oracle import codebooks as cbk
from synth import apply_rope

DELTA = cbk.delta_table()


def _objective(scores, widths):
    # distortion model implied by the fp32 deltas: C(b) = -sum_{b'<b} delta(b')
    C = np.concatenate([[0.0], -np.cumsum(DELTA.astype(np.float64))])
    return float(np.sum(np.asarray(scores) * C[np.asarray(widths)]))


def _true_objective(scores, widths):
    c = np.array([cbk.distortion(b) for b in range(9)])
    return float(np.sum(np.asarray(scores) * c[np.asarray(widths)]))


@pytest.mark.parametrize("budget,bmin,bmax", [(2, 0, 8), (3, 0, 8), (4, 0, 8), (3, 1, 6), (1, 0, 2), (8, 0, 8), (0, 0, 8)])
def test_budget_identity(budget, bmin, bmax):
    rng = np.random.default_rng(budget * 10 + bmin)
    for _ in range(5):
        s = np.exp(2 * rng.standard_normal(64))
        b = al.greedy_allocate(s, budget, bmin, bmax, DELTA)
        assert int(np.sum(2 * b)) == budget * 128
        assert b.min() >= bmin and b.max() <= bmax


@pytest.mark.parametrize("d", [2, 4, 6, 8, 10])
def test_greedy_equals_brute_force(d):
    nb = d // 2
    rng = np.random.default_rng(d)
    for trial in range(6):
        s = np.exp(2.5 * rng.standard_normal(nb))
        for budget in range(0, 9):
            g = al.greedy_allocate(s, budget, 0, 8, DELTA)
            best, best_sets = math.inf, []
            for combo in itertools.product(range(9), repeat=nb):
                if sum(combo) != budget * nb:
                    continue
                v = _objective(s, combo)
                if v < best - 1e-12 * abs(best if best != math.inf else 1):
                    best, best_sets = v, [combo]
                elif abs(v - best) <= 1e-12 * abs(best):
                    best_sets.append(combo)
            assert _objective(s, g) == pytest.approx(best, rel=1e-12, abs=1e-300)
            assert tuple(int(x) for x in g) in best_sets
            # and within fp32-delta rounding of the true-distortion optimum
            tbest = min(_true_objective(s, c) for c in best_sets)
            assert _true_objective(s, g) == pytest.approx(tbest, rel=1e-6)


def test_greedy_beats_uniform_and_is_monotone():
    rng = np.random.default_rng(11)
    for budget in (2, 3, 4):
        s = np.exp(2 * rng.standard_normal(64))
        b = al.greedy_allocate(s, budget, 0, 8, DELTA)
        assert _true_objective(s, b) <= _true_objective(s, np.full(64, budget)) + 1e-15
        order = np.argsort(-s)
        assert np.all(np.diff(b[order]) <= 0)          # s_i > s_j => b_i >= b_j


def test_equal_scores_give_uniform_widths():
    for budget in range(0, 9):
        b = al.greedy_allocate(np.ones(64), budget, 0, 8, DELTA)
        assert np.all(b == budget)


def test_ties_go_to_smallest_block():
    b = al.greedy_allocate(np.ones(4), 1, 0, 8, DELTA)      # 4 steps, round-robin from j = 0
    assert b.tolist() == [1, 1, 1, 1]
    # scores [1, 5, 5], 3 steps: j=1 (tie with j=2), then j=2, then 5*d(1) on both -> j=1
    b = al.greedy_allocate(np.array([1.0, 5.0, 5.0]), 1, 0, 8, DELTA)
    assert b.tolist() == [0, 2, 1]


def test_permutation_equivariance():
    rng = np.random.default_rng(5)
    s = np.exp(2 * rng.standard_normal(64))
    perm = rng.permutation(64)
    b = al.greedy_allocate(s, 3, 0, 8, DELTA)
    bp = al.greedy_allocate(s[perm], 3, 0, 8, DELTA)
    assert np.array_equal(bp, b[perm])


@pytest.mark.parametrize("pairing", ["half", "interleaved"])
def test_energy_is_rope_invariant(pairing):
    rng = np.random.default_rng(2)
    T, H, d = 700, 2, 128
    k0 = rng.standard_normal((T, H, d)) * np.exp(rng.standard_normal(d))[None, None, :]
    kr = apply_rope(k0, np.arange(T), 5.0e5, pairing)
    m0 = al.energy(k0, pairing)
    m1 = al.energy(kr, pairing)
    assert np.allclose(m0, m1, rtol=1e-12)


def test_energy_scaling_and_fsum():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((600, 3, 128)).astype(np.float32)
    m = al.energy(k)
    for e in (1, 3, -2):
        assert np.array_equal(al.energy(k * np.float32(2.0 ** e)), m * 4.0 ** e)
    p0, p1 = al.block_pairs(128)
    x = k.astype(np.float64)
    for h in range(3):
        for j in (0, 17, 63):
            ref = math.fsum(list(x[:, h, p0[j]] ** 2) + list(x[:, h, p1[j]] ** 2)) / (2 * 600)
            assert m[h, j] == pytest.approx(ref, rel=1e-14)


def test_energy_summation_order():
    # token 0 has term 2^31; tokens 1..255 have term 2^-28 (below half an ulp of 2^31, so the
    # in-chunk running sum drops them); chunk 1 (tokens 256..511) sums exactly to 2^-20.
    # The specified order gives (2^31 + 2^-20) / (2T); exact summation would give more.
    T = 512
    k = np.zeros((T, 1, 2), dtype=np.float16)
    k[0, 0, 0] = k[0, 0, 1] = 2.0 ** 15
    k[1:, 0, 0] = 2.0 ** -14
    m = al.energy(k)
    assert m[0, 0] == (2.0 ** 31 + 2.0 ** -20) / (2 * T)
    exact = (2.0 ** 31 + 511 * 2.0 ** -28) / (2 * T)
    assert m[0, 0] != exact


def test_energy_rejects_empty():
    with pytest.raises(ValueError):
        al.energy(np.zeros((0, 1, 128), np.float32))


def test_gains():
    rng = np.random.default_rng(9)
    m = np.exp(3 * rng.standard_normal((2, 64)))
    g, ig = al.gains(m)
    assert g.dtype == np.float32 and ig.dtype == np.float32
    # sum_j g_j^2 = nb (mean block energy normalised to 1)
    assert np.allclose(np.sum(g.astype(np.float64) ** 2, axis=1), 64, rtol=1e-6)
    assert np.allclose(g.astype(np.float64) * ig.astype(np.float64), 1.0, rtol=1e-6)
    g4, ig4 = al.gains(m * 4.0)
    assert np.array_equal(g4, g) and np.array_equal(ig4, ig)
    ge, ige = al.gains(np.full((1, 64), 3.7))
    assert np.all(ge == 1) and np.all(ige == 1)
    mz = m[:1].copy()
    mz[0, 5] = 0.0
    gz, igz = al.gains(mz)
    assert gz[0, 5] == 0 and igz[0, 5] == 0
    g0, ig0 = al.gains(np.zeros((1, 64)))
    assert np.all(g0 == 1) and np.all(ig0 == 1)


def test_field_order():
    rng = np.random.default_rng(1)
    s = np.exp(2 * rng.standard_normal(64))
    for pairing in ("half", "interleaved"):
        b = al.greedy_allocate(s, 3, 0, 8, DELTA)
        dims, ws = al.field_order(b, 128, pairing)
        assert int(ws.sum()) == 3 * 128
        assert np.all(np.diff(ws) <= 0)
        p0, p1 = al.block_pairs(128, pairing)
        # each stored block contributes p0 then p1, with its own width
        for f in range(0, dims.size, 2):
            j = int(np.where(p0 == dims[f])[0][0])
            assert dims[f + 1] == p1[j] and ws[f] == b[j] == ws[f + 1]
        # blocks of equal width appear in ascending block index
        blocks = [int(np.where(p0 == dims[f])[0][0]) for f in range(0, dims.size, 2)]
        for w in set(ws.tolist()):
            bw = [blk for blk in blocks if b[blk] == w]
            assert bw == sorted(bw)
        assert sorted(blocks) == sorted(int(j) for j in np.where(b > 0)[0])
