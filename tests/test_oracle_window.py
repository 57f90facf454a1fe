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
