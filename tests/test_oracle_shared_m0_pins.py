"""Pins of the oracle's shared-initial-state form (forward_walk_shared).

The learned initial state M0 is one parameter of the layer, shared by every
sequence (section on the learned M0 of the ai-paper-analysis.pages.dev summary;
section 三 of the m.163.com article).  A sequence's memory starts as M0 and a
per-sequence store holds only the rows touched so far.  Pins: a fresh sequence
(nothing touched) equals the plain walk from M0 whatever the store holds; a fully
touched one equals the plain walk from the store; two consecutive calls equal
one call over their tokens; the touched set is the union of the ids read and
written, by brute force.
"""
import numpy as np
import pytest

from oracle import sdm_oracle as O


def _sel(rng, T, N, d_v, W, R):
    return dict(
        idx_w=np.array([np.sort(rng.choice(N, W, replace=False)) for _ in range(T)]),
        wt_w=rng.dirichlet(np.ones(W), T), idx_r=np.array([np.sort(rng.choice(N, R, replace=False))
                                                           for _ in range(T)]),
        wt_r=rng.dirichlet(np.ones(R), T), v=rng.standard_normal((T, d_v)),
        g=rng.uniform(0, 1, (T, d_v)), alpha=rng.uniform(0.3, 1, T), beta=rng.uniform(0, 1, T))


def _cut(sel, a, b):
    return {k: v[a:b] for k, v in sel.items()}


def test_fresh_sequence_is_the_plain_walk_from_m0():
    rng = np.random.default_rng(41)
    T, N, d_v = 50, 64, 8
    sel = _sel(rng, T, N, d_v, 6, 5)
    m0 = rng.standard_normal((N, d_v))
    gam = rng.uniform(0.5, 1.5, d_v)
    store = np.full((N, d_v), np.nan)             # never read while untouched
    out, y, M, touched = O.forward_walk_shared(m0, store, np.zeros(N, bool), sel, gam, 1e-6)
    o2, y2, M2 = O.forward_walk(m0, sel, gam, 1e-6)
    assert np.array_equal(out, o2) and np.array_equal(y, y2) and np.array_equal(M, M2)
    assert np.array_equal(M[~touched], m0[~touched])


def test_fully_touched_is_the_plain_walk_from_the_store():
    rng = np.random.default_rng(42)
    T, N, d_v = 30, 36, 4
    sel = _sel(rng, T, N, d_v, 5, 7)
    m0 = np.full((N, d_v), np.nan)                # never read when every row is touched
    store = rng.standard_normal((N, d_v))
    gam = np.ones(d_v)
    out, y, M, touched = O.forward_walk_shared(m0, store, np.ones(N, bool), sel, gam, 1e-6)
    o2, y2, M2 = O.forward_walk(store, sel, gam, 1e-6)
    assert np.array_equal(out, o2) and np.array_equal(M, M2) and touched.all()


def test_two_calls_equal_one():
    rng = np.random.default_rng(43)
    T, N, d_v = 60, 100, 8
    sel = _sel(rng, T, N, d_v, 8, 8)
    m0 = rng.standard_normal((N, d_v))
    gam = rng.uniform(0.5, 1.5, d_v)
    t0 = np.zeros(N, bool)
    out, _, M, tch = O.forward_walk_shared(m0, np.zeros((N, d_v)), t0, sel, gam, 1e-6)
    o1, _, M1, t1 = O.forward_walk_shared(m0, np.zeros((N, d_v)), t0, _cut(sel, 0, 23), gam, 1e-6)
    store = np.where(t1[:, None], M1, 0.0)        # what a store holds: touched rows only
    o2, _, M2, t2 = O.forward_walk_shared(m0, store, t1, _cut(sel, 23, T), gam, 1e-6)
    assert np.array_equal(np.concatenate([o1, o2]), out)
    assert np.array_equal(M2, M) and np.array_equal(t2, tch)


def test_touched_is_every_slot_read_or_written():
    rng = np.random.default_rng(44)
    T, N, d_v = 20, 90, 2
    sel = _sel(rng, T, N, d_v, 3, 4)
    before = rng.random(N) < 0.1
    _, _, _, touched = O.forward_walk_shared(rng.standard_normal((N, d_v)),
                                             rng.standard_normal((N, d_v)), before, sel,
                                             np.ones(d_v), 1e-6)
    for i in range(N):
        hit = bool(before[i])
        for t in range(T):
            hit = hit or i in sel["idx_w"][t] or i in sel["idx_r"][t]
        assert touched[i] == hit


_orig = O.forward_walk_shared


def _writes_only(m0_h, store_h, touched_h, sel, gamma_h, eps, rule="slot", state="exact"):
    out, y, M, _ = _orig(m0_h, store_h, touched_h, sel, gamma_h, eps, rule, state)
    t = np.asarray(touched_h, bool).copy()
    t[np.asarray(sel["idx_w"]).ravel()] = True
    return out, y, M, t


def _store_always(m0_h, store_h, touched_h, sel, gamma_h, eps, rule="slot", state="exact"):
    return _orig(m0_h, store_h, np.ones(len(touched_h), bool), sel, gamma_h, eps, rule, state)


@pytest.mark.parametrize("fn", [_writes_only, _store_always])
def test_pins_catch_mutant(fn, monkeypatch):
    monkeypatch.setattr(O, "forward_walk_shared", fn)
    failed = 0
    for pin in (test_fresh_sequence_is_the_plain_walk_from_m0,
                test_fully_touched_is_the_plain_walk_from_the_store, test_two_calls_equal_one,
                test_touched_is_every_slot_read_or_written):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1
