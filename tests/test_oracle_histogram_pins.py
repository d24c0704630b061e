"""Pins of the oracle's slot-update histogram (slot_update_counts).

The papers.ananclaw.com summary (engineering-risks section, risk 3) asks for a
histogram of how often each slot is updated, to catch writes collapsing onto a
few slots.  The pins: brute force by nested loops on small inputs, the total
(every token writes W distinct slots of each head), and the collapsed case where
every token selects the same slots.
"""
import numpy as np
import pytest

from oracle import sdm_oracle as O


def _ids(rng, B, T, H, N, W):
    out = np.empty((B, T, H, W), np.int32)
    for idx in np.ndindex(B, T, H):
        out[idx] = np.sort(rng.choice(N, W, replace=False))
    return out


def test_counts_equal_brute_force():
    rng = np.random.default_rng(31)
    B, T, H, N, W = 2, 9, 3, 20, 4
    ids = _ids(rng, B, T, H, N, W)
    c = O.slot_update_counts(ids, N)
    for h in range(H):
        for s in range(N):
            n = 0
            for b in range(B):
                for t in range(T):
                    n += int(s in ids[b, t, h])
            assert c[h, s] == n


def test_total_is_every_write():
    rng = np.random.default_rng(32)
    B, T, H, N, W = 3, 40, 2, 64, 16
    c = O.slot_update_counts(_ids(rng, B, T, H, N, W), N)
    assert c.shape == (H, N) and np.all(c.sum(axis=1) == B * T * W) and c.min() >= 0


def test_collapsed_selection():
    B, T, H, N, W = 2, 25, 2, 50, 5
    ids = np.broadcast_to(np.array([3, 7, 11, 40, 49], np.int32), (B, T, H, W))
    c = O.slot_update_counts(ids, N)
    want = np.zeros((H, N), np.int64)
    want[:, [3, 7, 11, 40, 49]] = B * T
    assert np.array_equal(c, want)


def _per_batch_only(idx_w, N):  # planted mistake: counts batch entry 0 only
    idx_w = np.asarray(idx_w)
    return _orig(idx_w[:1], N) if idx_w.shape[0] > 1 else _orig(idx_w, N)


def _head_mixed(idx_w, N):      # planted mistake: heads summed together
    c = _orig(idx_w, N)
    return np.broadcast_to(c.sum(0), c.shape).copy()


_orig = O.slot_update_counts


@pytest.mark.parametrize("fn", [_per_batch_only, _head_mixed])
def test_pins_catch_mutant(fn, monkeypatch):
    monkeypatch.setattr(O, "slot_update_counts", fn)
    failed = 0
    for pin in (test_counts_equal_brute_force, test_total_is_every_write, test_collapsed_selection):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1
