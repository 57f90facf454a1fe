"""Pins of the recent-window oracle (oracle/window.py): a step-by-step simulation of the
window, invariants and special cases."""
import numpy as np
import pytest

from oracle import window as wn


def _simulate(chunks, R):
    """Keep the set of positions held in fp16 after each append; record every position
    that was ever held."""
    held, ever, length = [], set(), 0
    for n in chunks:
        for p in range(length, length + n):
            held.append(p)
        length += n
        held = held[-R:] if R > 0 else []
        ever.update(held)
    return ever, length


@pytest.mark.parametrize("seed", range(20))
def test_window_matches_simulation(seed):
    rng = np.random.default_rng(seed)
    chunks = rng.integers(1, 300, size=rng.integers(1, 8)).tolist()
    R = int(rng.choice([0, 1, 7, 64, 256, 1000]))
    ever, T = _simulate(chunks, R)
    bounds = [0, *np.cumsum(chunks).tolist()]
    mask = wn.through_fp16(bounds, R)
    assert set(np.flatnonzero(mask).tolist()) == ever
    assert wn.packed_len(T, R) + min(T, R if R > 0 else 0) == T
    if R > 0:
        assert mask[max(0, T - R):].all()          # the current window


def test_window_special_cases():
    assert not wn.through_fp16([0, 500], 0).any()
    assert wn.through_fp16([0, 100, 300], 512).all()
    assert wn.packed_len(300, 512) == 0 and wn.packed_len(300, 0) == 300


def test_stored_rows_rounds_only_window_positions():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((50, 2, 4)).astype(np.float32)
    out = wn.stored_rows(x, [0, 20, 50], 10)
    m = wn.through_fp16([0, 20, 50], 10)
    assert np.array_equal(out[~m], x[~m])
    assert np.array_equal(out[m], x[m].astype(np.float16).astype(np.float32))
    h = x.astype(np.float16)
    assert np.array_equal(wn.stored_rows(h, [0, 20, 50], 10), h)


def _simulate_grouped(chunks, R, group):
    """The packed prefix only ever grows by whole groups: after each append it advances one
    group at a time while a whole group lies before the last R positions."""
    ever, length, pk = set(), 0, 0
    for n in chunks:
        length += n
        while pk + group <= length - R:
            pk += group
        ever.update(range(pk, length))
    return ever, length, pk


@pytest.mark.parametrize("seed", range(20))
def test_grouped_packing_matches_simulation(seed):
    """Whole 128-position groups only (the KIVI-style codec's key tiles), with and without a
    recent window."""
    rng = np.random.default_rng(100 + seed)
    chunks = rng.integers(1, 400, size=rng.integers(1, 8)).tolist()
    R = int(rng.choice([0, 128, 256, 512]))
    ever, T, pk = _simulate_grouped(chunks, R, 128)
    bounds = [0, *np.cumsum(chunks).tolist()]
    assert wn.packed_len(T, R, 128) == pk
    assert pk % 128 == 0 and 0 <= T - pk - R < 128 or (pk == 0 and T < R + 128)
    mask = wn.through_fp16(bounds, R, 128)
    assert set(np.flatnonzero(mask).tolist()) == ever


def test_grouped_packing_special_cases():
    assert wn.packed_len(127, 0, 128) == 0 and wn.packed_len(128, 0, 128) == 128
    assert wn.packed_len(1000, 0, 128) == 896 and wn.packed_len(1000, 256, 128) == 640
    # one append of a whole number of tiles packs everything from the input
    assert not wn.through_fp16([0, 1024], 0, 128).any()
    assert wn.through_fp16([0, 1000], 0, 128).sum() == 1000 - 896
