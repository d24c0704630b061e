"""Pins of the oracle's scan backward (scan_backward) and its write log.

The training scheme of the m.163.com article (section 八, memory-efficiency
paragraph) applies the sparse update in place and undoes it in backward, keeping
the state plus the rows the writes overwrote.  The backward is pinned against
central differences of the forward oracle (itself pinned elsewhere): for a scalar
loss L = <out, P> + <M_T, Q> with fixed random P and Q, every input of the scan
-- v, gate, alpha, beta, both weight sets, the RMSNorm weight and the initial
state -- is perturbed one element at a time.  The restored initial state must be
bit-identical to the forward's.  Planted mistakes in the reverse walk must fail.
"""
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
    y, M = O.scan(c["state0"], c["idx_w"], c["wt_w"], c["idx_r"], c["wt_r"], c["v"], c["alpha"],
                  c["beta"])
    out = O.rms_norm_gate(y, c["gamma"], c["gate"], EPS)
    return np.sum(out * c["P"]) + np.sum(M * c["Q"])


def _backward(c):
    y, M, log = O.scan(c["state0"], c["idx_w"], c["wt_w"], c["idx_r"], c["wt_r"], c["v"],
                       c["alpha"], c["beta"], record=True)
    return O.scan_backward(M, log, c["idx_w"], c["wt_w"], c["idx_r"], c["wt_r"], c["v"],
                           c["alpha"], c["beta"], y, c["gate"], c["gamma"], EPS, c["P"], c["Q"])


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


@pytest.mark.parametrize("seed", [51, 52])
def test_gradients_equal_central_differences(seed):
    c = _case(seed)
    g, M0, dM0 = _backward(c)
    for key, name in GRADS.items():
        num = _numeric(c, key)
        assert np.allclose(g[name], num, rtol=1e-6, atol=1e-7), key
    assert np.allclose(dM0, _numeric(c, "state0"), rtol=1e-6, atol=1e-7), "state0"


def test_slots_written_and_read_by_one_token_and_reused():
    # N = 4 with W = 3, R = 4: every token reads what it writes, slots recur every token
    c = _case(53, T=6, N=4, d_v=3, W=3, R=4)
    g, _, dM0 = _backward(c)
    for key, name in GRADS.items():
        assert np.allclose(g[name], _numeric(c, key), rtol=1e-6, atol=1e-7), key
    assert np.allclose(dM0, _numeric(c, "state0"), rtol=1e-6, atol=1e-7)


def test_restores_the_initial_state_exactly():
    c = _case(54, T=40, N=30, d_v=8, W=6, R=5)
    _, M0, _ = _backward(c)
    assert np.array_equal(M0, c["state0"])


def test_identity_writes_pass_the_state_gradient_through():
    # alpha = 1, beta = 0: writes change nothing, so dM0 = Q + the reads' q dy terms,
    # and the gradients of v and of the write weights vanish
    c = _case(55)
    c["alpha"][:] = 1.0
    c["beta"][:] = 0.0
    g, _, dM0 = _backward(c)
    assert np.all(g["d_v"] == 0) and np.all(g["d_wt_w"] == 0)
    assert np.allclose(dM0, _numeric(c, "state0"), rtol=1e-6, atol=1e-7)


# ---- planted mistakes in the reverse walk (CPU): each must fail a pin above --------
_orig = O.scan_backward


def _mutant(kind):
    def scan_backward(state_T, log, idx_w, wt_w, idx_r, wt_r, v, alpha, beta, y, gate, gamma_h,
                      eps, d_out, d_state):
        M = np.array(state_T, float, copy=True)
        dM = np.array(d_state, float, copy=True)
        T, d_v = np.shape(y)
        g = dict(d_v=np.zeros((T, d_v)), d_gate=np.zeros((T, d_v)), d_alpha=np.zeros(T),
                 d_beta=np.zeros(T), d_wt_w=np.zeros(np.shape(idx_w)),
                 d_wt_r=np.zeros(np.shape(idx_r)), d_gamma=np.zeros(d_v))
        for t in range(T - 1, -1, -1):
            s = 1.0 / np.sqrt(np.mean(y[t] * y[t]) + eps)
            yhat = y[t] * s
            g["d_gate"][t] = d_out[t] * yhat * gamma_h
            g["d_gamma"] += d_out[t] * yhat * gate[t]
            u = d_out[t] * gamma_h * gate[t]
            dy = s * u if kind == "norm_without_mean" else s * (u - yhat * np.mean(u * yhat))

            def read():
                rows = idx_r[t]
                g["d_wt_r"][t] = M[rows] @ dy
                dM[rows] += wt_r[t][:, None] * dy[None, :]

            def write():
                rows = idx_w[t]
                m = log[t]
                c = beta[t] * wt_w[t]
                G = dM[rows]
                g["d_v"][t] = c @ G
                dc = np.sum(G * (v[t][None, :] - alpha[t] * m), axis=1)
                fac = 1.0 if kind == "alpha_without_1mc" else (1.0 - c)[:, None]
                g["d_alpha"][t] = np.sum(fac * G * m)
                g["d_beta"][t] = wt_w[t] @ dc
                g["d_wt_w"][t] = beta[t] * dc
                if kind != "gradient_not_decayed":
                    dM[rows] = (alpha[t] * (1.0 - c))[:, None] * G
                M[rows] = m

            if kind == "write_before_read":
                write()
                read()
            else:
                read()
                write()
        return g, M, dM
    return scan_backward


@pytest.mark.parametrize("kind", ["norm_without_mean", "alpha_without_1mc", "gradient_not_decayed",
                                  "write_before_read"])
def test_pins_catch_mutant(kind, monkeypatch):
    monkeypatch.setattr(O, "scan_backward", _mutant(kind))
    failed = 0
    for pin in (lambda: test_gradients_equal_central_differences(51),
                test_slots_written_and_read_by_one_token_and_reused,
                test_restores_the_initial_state_exactly,
                test_identity_writes_pass_the_state_gradient_through):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, kind
