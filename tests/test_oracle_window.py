"""Pins of the sliding-window reading: a query attends to the last W
positions of its sequence; blocks wholly before the window may be released
without changing any output."""
import numpy as np
import pytest
import torch

import workloads
from helpers import bits, brute_force, oracle_run
from oracle import allocator as A


def _wl(seed=31, dtype="bf16"):
    return workloads.random_small(seed, S=5, Hq=8, Hkv=2, d=32, dtype=dtype, max_len=90, min_len=1)


@pytest.mark.parametrize("window", [1, 2, 5, 16, 17, 33, 64, 1000])
def test_window_matches_brute_force(window):
    wl = _wl()
    q, k, v = wl.tensors()
    _, out = oracle_run(wl, q, k, v, window=window)
    ref = brute_force(wl, q, k, v, window=window)
    assert np.max(np.abs(out - ref)) <= 1e-13


def test_window_covering_sequence_is_full_attention():
    wl = _wl(32)
    q, k, v = wl.tensors()
    _, full = oracle_run(wl, q, k, v)
    _, win = oracle_run(wl, q, k, v, window=int(wl.lengths.max()))
    assert np.array_equal(full, win)


def test_window_of_one_returns_last_value():
    wl = _wl(33)
    q, k, v = wl.tensors()
    _, out = oracle_run(wl, q, k, v, window=1)
    offs = wl.offsets
    G = wl.Hq // wl.Hkv
    for s in range(wl.S):
        last = v[offs[s + 1] - 1].double().numpy()
        for h in range(wl.Hq):
            assert np.array_equal(out[s, h], last[h // G])


@pytest.mark.parametrize("window", [1, 16, 20, 47])
def test_released_blocks_leave_outputs_unchanged(window):
    wl = _wl(34)
    q, k, v = wl.tensors()
    _, kept = oracle_run(wl, q, k, v, window=window)
    trim = [("window", sid, window) for sid in wl.seq_ids]
    rp, trimmed = oracle_run(wl, q, k, v, window=window, extra_ops=trim)
    assert np.array_equal(kept, trimmed)
    rp.alloc.check_invariants()
    # every block wholly before a window went back to the pool
    for sid, n in zip(wl.seq_ids, rp.lengths()):
        t = rp.alloc.table(sid)
        cut = max(0, n - window) // wl.block
        assert t[:cut] == [A.HOLE] * cut and A.HOLE not in t[cut:]
    live = sum(1 for r in rp.alloc.ref if r > 0)
    assert live == sum(len(t) - t.count(A.HOLE) for t in rp.tables())


def test_gather_refuses_released_block():
    wl = _wl(35)
    q, k, v = wl.tensors()
    trim = [("window", sid, 1) for sid in wl.seq_ids]
    rp, _ = oracle_run(wl, q, k, v, window=1, extra_ops=trim)
    s = int(np.argmax(wl.lengths))
    with pytest.raises(ValueError):
        rp.pool.gather(0, rp.tables()[s], int(rp.lengths()[s]), 0)
