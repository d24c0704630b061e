"""Pins of the oracle's chunkwise form (sparse_inner, scan_chunkwise).

The chunkwise form is an exact reordering of the sequential recurrences, so its
result is fixed by scan() and scan_gdn(), which are pinned on their own (hand-worked
fixtures, closed forms, a dense matrix recurrence): for every chunk size, from one
token to more than the whole sequence, y and the final state must agree within fp64
rounding, on slot spaces small enough that tokens of a chunk share many slots.
sparse_inner is checked by brute force over all pairs of positions and against a
dense dot product.  Planted mistakes in the chunkwise form must fail.
"""
import inspect

import numpy as np
import pytest

from oracle import sdm_oracle as O


def _walk(seed, N, T, W, R, dv, alpha=None, beta=None):
    rng = np.random.default_rng(seed)
    ids = lambda k: np.stack([np.sort(rng.choice(N, k, replace=False)) for _ in range(T)])
    return dict(state0=rng.standard_normal((N, dv)), idx_w=ids(W),
                wt_w=rng.dirichlet(np.ones(W), T), idx_r=ids(R),
                wt_r=rng.dirichlet(np.ones(R), T), v=rng.standard_normal((T, dv)),
                alpha=rng.uniform(0.3, 1.0, T) if alpha is None else np.full(T, alpha),
                beta=rng.uniform(0.0, 1.0, T) if beta is None else np.full(T, beta))


SEQ = {"slot": O.scan, "gdn": O.scan_gdn}


def _agree(w, C, rule, fn=None):
    fn = fn or O.scan_chunkwise
    y, M = SEQ[rule](**w)[:2]
    yc, Mc = fn(**w, C=C, rule=rule)
    scale = max(1.0, np.abs(y).max(), np.abs(M).max())
    np.testing.assert_allclose(yc, y, rtol=0, atol=1e-12 * scale, err_msg=f"y C={C} {rule}")
    np.testing.assert_allclose(Mc, M, rtol=0, atol=1e-12 * scale, err_msg=f"M C={C} {rule}")


@pytest.mark.parametrize("rule", ["slot", "gdn"])
@pytest.mark.parametrize("N,T,W,R,dv", [(12, 11, 4, 3, 5),    # most tokens share slots
                                        (6, 9, 6, 6, 2),      # every slot, every token
                                        (64, 20, 5, 7, 3),    # few collisions
                                        (16, 13, 1, 1, 4)])   # one slot per token
def test_chunkwise_equals_sequential(rule, N, T, W, R, dv):
    w = _walk(N * 100 + T, N, T, W, R, dv)
    for C in (1, 2, 3, 4, 5, T - 1, T, T + 7):
        _agree(w, C, rule)


@pytest.mark.parametrize("rule", ["slot", "gdn"])
def test_identity_gates_leave_state_and_read_it(rule):
    # alpha = 1, beta = 0: nothing is written; every read returns the weighted M0 rows
    w = _walk(3, 10, 8, 3, 4, 3, alpha=1.0, beta=0.0)
    y, M = O.scan_chunkwise(**w, C=3, rule=rule)
    np.testing.assert_array_equal(M, w["state0"])
    exp = np.einsum("tk,tkd->td", w["wt_r"], w["state0"][w["idx_r"]])
    np.testing.assert_allclose(y, exp, rtol=0, atol=1e-15)


def test_sparse_inner_brute_force():
    rng = np.random.default_rng(7)
    for _ in range(200):
        N = int(rng.integers(1, 40))
        a = np.sort(rng.choice(N, int(rng.integers(0, N + 1)), replace=False))
        b = np.sort(rng.choice(N, int(rng.integers(0, N + 1)), replace=False))
        va, vb = rng.standard_normal(a.size), rng.standard_normal(b.size)
        got = O.sparse_inner(a, b, lambda p, q: va[p] * vb[q])
        brute = sum(va[p] * vb[q] for p in range(a.size) for q in range(b.size) if a[p] == b[q])
        da, db = np.zeros(N), np.zeros(N)
        da[a], db[b] = va, vb
        assert abs(got - brute) <= 1e-12
        assert abs(got - float(da @ db)) <= 1e-12


# ---- planted mistakes ----------------------------------------------------------------
_SRC = inspect.getsource(O.scan_chunkwise)
_MUTANTS = {
    "decay includes the source token": ("for u in range(s + 1, t + 1):",
                                        "for u in range(max(s, c0), t + 1):"),
    "decay stops before the reading token": ("for u in range(s + 1, t + 1):",
                                             "for u in range(s + 1, t):"),
    "chunk-start rows read undecayed": ("y[t] += wt_r[t, k] * G(int(j), c0 - 1, t) * M0[j]",
                                        "y[t] += wt_r[t, k] * M0[j]"),
    "no triangular solve": ("rhs -= b_ts * x[s]", "pass"),
    "own token's term left out": ("for s in range(c0, t + 1):", "for s in range(c0, t):"),
    "slot decay without the delta factor": ("alpha[u] * (1.0 - beta[u] * wt_w[u, k]) if",
                                            "alpha[u] if"),
}


def _mutant(kind):
    old, new = _MUTANTS[kind]
    assert _SRC.count(old) == 1, kind
    ns = dict(O.__dict__)
    exec(compile(_SRC.replace(old, new), "<mutant>", "exec"), ns)
    return ns["scan_chunkwise"]


def _bad_merge(ids_a, ids_b, term):
    # advances past a match without counting it when the first list's id is not greater
    p = q = 0
    acc = 0.0
    while p < len(ids_a) and q < len(ids_b):
        if ids_a[p] <= ids_b[q]:
            p += 1
        else:
            q += 1
    return acc


@pytest.mark.parametrize("kind", list(_MUTANTS) + ["merge skips matches"])
def test_pins_catch_mutant(kind, monkeypatch):
    if kind == "merge skips matches":
        monkeypatch.setattr(O, "sparse_inner", _bad_merge)
        fn = O.scan_chunkwise
    else:
        fn = _mutant(kind)
    w = _walk(1211, 12, 11, 4, 3, 5)
    with pytest.raises(AssertionError):
        for rule in ("slot", "gdn"):
            _agree(w, 4, rule, fn)
