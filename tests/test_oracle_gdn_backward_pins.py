"""Pins of the oracle's backward for the key-weighted (GDN-form) write rule.

scan_backward(..., rule="gdn") undoes scan_gdn's writes from the rows they replaced
(scan_gdn(..., record=True)), as the m.163.com article's training scheme does for
the per-slot rule (section 八).  It is pinned against central differences of the
forward oracle scan_gdn (itself pinned against a dense matrix-form gated delta
recurrence): for L = <out, P> + <M_T, Q> every input -- v, gate, alpha, beta, both
weight sets, the RMSNorm weight and the initial state -- is perturbed one element at
a time.  The restored initial state must be bit-identical.  Planted mistakes in the
key-weighted terms must fail.
"""
import inspect

import numpy as np
import pytest

from oracle import sdm_oracle as O

EPS = 1e-6


def _case(seed, T=7, N=12, d_v=4, W=3, R=4):
    rng = np.random.default_rng(seed)
    return dict(
        state0=rng.standard_normal((N, d_v)),
        idx_w=np.array([np.sort(rng.choice(N, W, replace=False)) for _ in range(T)]),
        wt_w=rng.dirichlet(np.ones(W), T),
        idx_r=np.array([np.sort(rng.choice(N, R, replace=False)) for _ in range(T)]),
        wt_r=rng.dirichlet(np.ones(R), T),
        v=rng.standard_normal((T, d_v)), gate=rng.uniform(0.1, 1.0, (T, d_v)),
        alpha=rng.uniform(0.3, 1.0, T), beta=rng.uniform(0.05, 0.95, T),
        gamma=rng.uniform(0.5, 1.5, d_v), P=rng.standard_normal((T, d_v)),
        Q=rng.standard_normal((N, d_v)))


def _loss(c):
    y, M = O.scan_gdn(c["state0"], c["idx_w"], c["wt_w"], c["idx_r"], c["wt_r"], c["v"],
                      c["alpha"], c["beta"])
    out = O.rms_norm_gate(y, c["gamma"], c["gate"], EPS)
    return np.sum(out * c["P"]) + np.sum(M * c["Q"])


def _backward(c, fn=None):
    fn = fn or O.scan_backward
    y, M, log = O.scan_gdn(c["state0"], c["idx_w"], c["wt_w"], c["idx_r"], c["wt_r"], c["v"],
                           c["alpha"], c["beta"], record=True)
    return fn(M, log, c["idx_w"], c["wt_w"], c["idx_r"], c["wt_r"], c["v"], c["alpha"],
              c["beta"], y, c["gate"], c["gamma"], EPS, c["P"], c["Q"], rule="gdn")


def _numeric(c, key):
    x = c[key]
    grad = np.zeros_like(x)
    for i in np.ndindex(*x.shape):
        h = 1e-6 * max(1.0, abs(x[i]))
        old = x[i]
        x[i] = old + h
        lp = _loss(c)
        x[i] = old - h
        lm = _loss(c)
        x[i] = old
        grad[i] = (lp - lm) / (2 * h)
    return grad


GRADS = {"v": "d_v", "gate": "d_gate", "alpha": "d_alpha", "beta": "d_beta", "wt_w": "d_wt_w",
         "wt_r": "d_wt_r", "gamma": "d_gamma"}


def _check(c, fn=None):
    g, M0, dM0 = _backward(c, fn)
    for key, name in GRADS.items():
        assert np.allclose(g[name], _numeric(c, key), rtol=1e-6, atol=1e-7), key
    assert np.allclose(dM0, _numeric(c, "state0"), rtol=1e-6, atol=1e-7), "state0"
    assert np.array_equal(M0, c["state0"]), "initial state not restored"


@pytest.mark.parametrize("seed", [61, 62])
def test_gradients_equal_central_differences(seed):
    _check(_case(seed))


def test_slots_written_and_read_by_one_token_and_reused():
    # N = 4 with W = 3, R = 4: every token reads what it writes, slots recur every token
    _check(_case(63, T=6, N=4, d_v=3, W=3, R=4))


def test_every_slot_in_every_write_set():
    # W = N: the prediction couples all rows of the memory at every token
    _check(_case(64, T=5, N=5, d_v=3, W=5, R=2))


def test_one_slot_of_weight_one_matches_the_per_slot_rule():
    # W = 1 (weight k = 1): the two rules give the same update, M' = alpha m + beta (v -
    # alpha m), so every gradient but the weight's agrees.  The weight enters
    # differently -- (1 - beta k) alpha m + beta k v against alpha m + beta k (v - k
    # alpha m) -- so at k = 1 the per-slot rule's d k = beta <G, v - alpha m> becomes
    # beta <G, v - 2 alpha m> = per-slot d k - beta <G, alpha m> for the key-weighted one.
    c = _case(65, T=8, N=6, d_v=3, W=1, R=2)
    g, M0, dM0 = _backward(c)
    y, M, log = O.scan(c["state0"], c["idx_w"], c["wt_w"], c["idx_r"], c["wt_r"], c["v"],
                       c["alpha"], c["beta"], record=True)
    gs, M0s, dM0s = O.scan_backward(M, log, c["idx_w"], c["wt_w"], c["idx_r"], c["wt_r"], c["v"],
                                    c["alpha"], c["beta"], y, c["gate"], c["gamma"], EPS, c["P"],
                                    c["Q"])
    for name in GRADS.values():
        if name != "d_wt_w":
            assert np.allclose(g[name], gs[name], rtol=1e-12, atol=1e-13), name
    assert np.allclose(dM0, dM0s, rtol=1e-12, atol=1e-13)
    # the weight's gradient by the closed form above: G, the gradient of the written
    # row, is the per-slot rule's d_v / beta (d_v = beta k G with k = 1), and m is the
    # logged row (the same forward for both rules)
    G = gs["d_v"] / c["beta"][:, None]
    m = log[:, 0]
    exp = gs["d_wt_w"][:, 0] - c["beta"] * c["alpha"] * np.sum(G * m, axis=1)
    assert np.allclose(g["d_wt_w"][:, 0], exp, rtol=1e-10, atol=1e-12)


# ---- planted mistakes in the key-weighted terms (CPU): each must fail ---------------
_SRC = inspect.getsource(O.scan_backward)
_MUTANTS = {
    "prediction path dropped from dm~": ("dmt = G - np.outer(k, de)", "dmt = G"),
    "prediction path dropped from dk": ("g[\"d_wt_w\"][t] = beta[t] * (G @ e) - mt @ de",
                                        "g[\"d_wt_w\"][t] = beta[t] * (G @ e)"),
    "de without beta": ("de = beta[t] * (k @ G)", "de = k @ G"),
    "alpha gradient from G": ("g[\"d_alpha\"][t] = np.sum(dmt * m)",
                              "g[\"d_alpha\"][t] = np.sum(G * m)"),
    "error term without the forget gate": ("e = v[t] - k @ mt", "e = v[t] - k @ m"),
}


def _mutant(kind):
    old, new = _MUTANTS[kind]
    assert _SRC.count(old) == 1, kind
    ns = dict(O.__dict__)
    exec(compile(_SRC.replace(old, new), "<mutant>", "exec"), ns)
    return ns["scan_backward"]


@pytest.mark.parametrize("kind", list(_MUTANTS))
def test_pins_catch_mutant(kind):
    with pytest.raises(AssertionError):
        _check(_case(61), _mutant(kind))
