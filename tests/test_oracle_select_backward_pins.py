"""Pins of the oracle's selection-pass backward (softmax_backward, pass_a_backward).

The whole layer from x is differentiated by central differences of the forward
oracle (pinned elsewhere): for a scalar loss L = <out, P> + <M_T, Q> with fixed
random P and Q, every element of x, W_proj, A and b_dt is perturbed.  The analytic
gradient chains the scan backward (pinned by its own central differences) into
pass_a_backward and the projection's dx = dY W_proj, dW_proj = dY^T x.  The cases
are drawn so that no selected set changes under the perturbations (the selection is
piecewise constant; its gap to the next slot is checked).  Planted mistakes in the
selection backward must fail.
"""
import numpy as np
import pytest

from oracle import sdm_oracle as O

EPS = 1e-6
SHAPE = dict(H=2, n=4, d_v=3, W=3, R=2)


def _case(seed, gate_act):
    rng = np.random.default_rng(seed)
    H, n, d_v = SHAPE["H"], SHAPE["n"], SHAPE["d_v"]
    B, T, d = 2, 4, 5
    P = 4 * n + 2 * d_v + 2
    return dict(x=rng.standard_normal((B, T, d)), w=rng.standard_normal((H * P, d)) * 0.7,
                A=rng.uniform(0.5, 1.5, H), b_dt=rng.uniform(-2.0, 0.5, H),
                gamma=rng.uniform(0.5, 1.5, (H, d_v)),
                state0=rng.standard_normal((B, H, n * n, d_v)) * 0.5,
                Pm=rng.standard_normal((B, T, H, d_v)),
                Q=rng.standard_normal((B, H, n * n, d_v)), gate_act=gate_act)


def _loss(c):
    out, st, _ = O.forward(c["x"], c["w"], c["A"], c["b_dt"], c["gamma"], c["state0"],
                           eps=EPS, gate_act=c["gate_act"], **SHAPE)
    return np.sum(out * c["Pm"]) + np.sum(st * c["Q"])


def _min_gap(c):
    a = O.pass_a(c["x"], c["w"], c["A"], c["b_dt"], gate_act=c["gate_act"], **SHAPE)
    return min(np.min(a["gap_w"]), np.min(a["gap_r"]))


def _analytic(c):
    H, n, d_v = SHAPE["H"], SHAPE["n"], SHAPE["d_v"]
    a = O.pass_a(c["x"], c["w"], c["A"], c["b_dt"], gate_act=c["gate_act"], **SHAPE)
    B, T = c["x"].shape[:2]
    grads = {k: np.zeros(a[k.replace("d_", "", 1) if k != "d_g" else "g"].shape)
             for k in ("d_wt_w", "d_wt_r", "d_v", "d_g", "d_alpha", "d_beta")}
    for b in range(B):
        for h in range(H):
            w = {k: a[k][b, :, h] for k in ("idx_w", "wt_w", "idx_r", "wt_r", "v", "g",
                                            "alpha", "beta")}
            y, M, log = O.scan(c["state0"][b, h], w["idx_w"], w["wt_w"], w["idx_r"], w["wt_r"],
                               w["v"], w["alpha"], w["beta"], record=True)
            g, _, _ = O.scan_backward(M, log, w["idx_w"], w["wt_w"], w["idx_r"], w["wt_r"],
                                      w["v"], w["alpha"], w["beta"], y, w["g"], c["gamma"][h],
                                      EPS, c["Pm"][b, :, h], c["Q"][b, h])
            for k in ("d_wt_w", "d_wt_r", "d_v", "d_alpha", "d_beta"):
                grads[k][b, :, h] = g[k]
            grads["d_g"][b, :, h] = g["d_gate"]
    return O.pass_a_backward(a, grads, c["A"], c["b_dt"], H, n, d_v, gate_act=c["gate_act"],
                             x=c["x"], w_proj=c["w"])


def _numeric(c, key):
    arr = c[key]
    grad = np.zeros_like(arr)
    for i in np.ndindex(*arr.shape):
        h = 1e-6 * max(1.0, abs(arr[i]))
        old = arr[i]
        arr[i] = old + h
        lp = _loss(c)
        arr[i] = old - h
        lm = _loss(c)
        arr[i] = old
        grad[i] = (lp - lm) / (2 * h)
    return grad


def _check(c):
    assert _min_gap(c) > 1e-3, "case too close to a selection change"
    got = _analytic(c)
    for key, gk in (("x", "dx"), ("w", "dW_proj"), ("A", "dA"), ("b_dt", "db_dt")):
        num = _numeric(c, key)
        scale = max(1.0, float(np.abs(num).max()))
        np.testing.assert_allclose(got[gk], num, rtol=0, atol=2e-6 * scale, err_msg=key)


@pytest.mark.parametrize("gate_act", [O.GATE_SIGMOID, O.GATE_SILU, O.GATE_NONE])
def test_layer_gradients_equal_central_differences(gate_act):
    _check(_case(31 + gate_act, gate_act))


def test_softmax_backward_closed_form():
    # w = softmax(s): dw_i/ds_j = w_i (delta_ij - w_j); with dw = e_k the score gradient
    # is w_k (e_k - w)
    w = O.softmax([0.3, -1.2, 2.0, 0.0])
    for k in range(4):
        dw = np.eye(4)[k]
        np.testing.assert_allclose(O.softmax_backward(w, dw), w[k] * (np.eye(4)[k] - w),
                                   rtol=1e-15, atol=1e-17)
    # a weight vector's gradient along constant dL/dw is zero (the weights sum to 1)
    np.testing.assert_allclose(O.softmax_backward(w, np.full(4, 2.5)), 0.0, atol=1e-15)


# ---- planted mistakes ----------------------------------------------------------------
def _mutant(kind):
    orig_sb, orig_fg = O.softmax_backward, O.forget_gate

    def softmax_no_centering(w, dw):
        return np.asarray(w, float) * np.asarray(dw, float)

    def pab(a, grads, A, b_dt, H, n, d_v, gate_act=O.GATE_SIGMOID, x=None, w_proj=None):
        r = O.__dict__["_orig_pab"](a, grads, A, b_dt, H, n, d_v, gate_act, x, w_proj)
        P = 4 * n + 2 * d_v + 2
        dY = r["dY"].reshape(r["dY"].shape[:-1] + (H, P)).copy()
        if kind == "halves swapped":
            dY[..., 0:n], dY[..., n:2 * n] = dY[..., n:2 * n].copy(), dY[..., 0:n].copy()
        if kind == "forget sign":
            dY[..., 4 * n + 2 * d_v] *= -1.0
        if kind == "input gate":
            dY[..., 4 * n + 2 * d_v + 1] *= 2.0
        r["dY"] = dY.reshape(r["dY"].shape)
        dYf = r["dY"].reshape(-1, H * P)
        r["dx"] = (dYf @ np.asarray(w_proj, float)).reshape(r["dx"].shape)
        r["dW_proj"] = dYf.T @ np.asarray(x, float).reshape(dYf.shape[0], -1)
        if kind == "dA sign":
            r["dA"] = -r["dA"]
        return r

    if kind == "softmax not centred":
        return "softmax_backward", softmax_no_centering
    return "pass_a_backward", pab


@pytest.mark.parametrize("kind", ["softmax not centred", "halves swapped", "forget sign",
                                  "input gate", "dA sign"])
def test_pins_catch_mutant(kind, monkeypatch):
    attr, fn = _mutant(kind)
    monkeypatch.setitem(O.__dict__, "_orig_pab", O.pass_a_backward)
    monkeypatch.setattr(O, attr, fn)
    with pytest.raises(AssertionError):
        _check(_case(31, O.GATE_SIGMOID))
