"""Selection-pass backward (sdm_select_backward) against the oracle's pass_a_backward.

The GPU's selection pass runs first; its selected ids and softmax weights are handed
to the oracle as they are (the selected sets are piecewise constant, so no gradient
flows through the choice, and comparing against the GPU's own sets keeps near-ties
out of the comparison).  The gate pre-activations on the oracle side are x . W_proj
in fp64 from the same stored inputs.  Incoming gradients are seeded normals.

* dY: the value columns are the incoming d_v bit for bit; the half-score columns
  (softmax backward summed over repeated half indices) within 1e-5 of the row's
  scale; the gate, forget and input-gate columns within the fp32 tolerance of the
  stage-A gates (the GPU recomputes the forget pre-gate in fp32).
* dA, db_dt: sums over every token, within 1e-5 of the sum of the terms' magnitudes.
* Two runs are bit-identical (fixed summation orders throughout).
"""
import numpy as np
import pytest
import torch

from oracle import sdm_oracle as O
from sparse_memory_linear_sdm_amd import _lib, dims_for, ops, synth
from tests.gpu_util import RTOL, ATOL, assert_close, host, layer_inputs, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"\n[gpu] {request.node.nodeid}")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    yield
    torch.cuda.synchronize()


def _grads(rng, wl):
    B, T, H = wl.B, wl.T, wl.H
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    return dict(d_wt_w=f(B, T, H, wl.W), d_wt_r=f(B, T, H, wl.R), d_v=f(B, T, H, wl.d_v),
                d_gate=f(B, T, H, wl.d_v), d_alpha=f(B, T, H), d_beta=f(B, T, H))


def _oracle_rows(wl, x_rows, w_proj, A, b_dt, prod_rows, grads_rows):
    """pass_a_backward of the given token rows ([S, d] of x, products and gradients
    [S, H, *]) with the GPU's selections and the fp64 pre-activations."""
    parts = O.split_heads(O.project(x_rows, w_proj), wl.H, wl.n, wl.d_v)
    a = dict(idx_w=prod_rows["idx_w"], wt_w=prod_rows["wt_w"].astype(np.float64),
             idx_r=prod_rows["idx_r"], wt_r=prod_rows["wt_r"].astype(np.float64),
             alpha=O.forget_gate(parts["a"], np.asarray(A, np.float64),
                                 np.asarray(b_dt, np.float64)),
             a_pre=parts["a"], b_pre=parts["b"], g_pre=parts["g"])
    g = {k: np.asarray(v, np.float64) for k, v in grads_rows.items()}
    g["d_g"] = g.pop("d_gate")
    return O.pass_a_backward(a, g, A, b_dt, wl.H, wl.n, wl.d_v, gate_act=wl.gate_act)


def _check_rows(wl, dy_rows, exp, grads_rows, prod_rows):
    """Column-block checks of dY rows [S, H*P] against the oracle's."""
    n, dv, H = wl.n, wl.d_v, wl.H
    P = 4 * n + 2 * dv + 2
    got = dy_rows.reshape(-1, H, P).astype(np.float64)
    ex = exp.reshape(-1, H, P)
    o = 4 * n
    # value columns: copied
    assert np.array_equal(dy_rows.reshape(-1, H, P)[..., o:o + dv],
                          grads_rows["d_v"].reshape(-1, H, dv)), "d_v columns"
    # half-score columns: per (token, head, role), scale = sum_k |w_k| (|dw_k| + |sum w dw|)
    for role, (o1, o2) in (("w", (0, n)), ("r", (2 * n, 3 * n))):
        w = prod_rows[f"wt_{role}"].reshape(-1, H, getattr(wl, role.upper())).astype(np.float64)
        dw = grads_rows[f"d_wt_{role}"].reshape(w.shape).astype(np.float64)
        s = np.abs(np.sum(w * dw, -1, keepdims=True))
        scale = np.sum(np.abs(w) * (np.abs(dw) + s), -1)[..., None] + 1e-30
        for lo in (o1, o2):
            err = np.abs(got[..., lo:lo + n] - ex[..., lo:lo + n])
            worst = float((err / scale).max())
            assert worst <= 1e-5, f"half-score columns of role {role} at {lo}: {worst:.3e}"
    assert_close(got[..., o + dv:o + 2 * dv], ex[..., o + dv:o + 2 * dv], "gate columns")
    assert_close(got[..., o + 2 * dv], ex[..., o + 2 * dv], "forget pre-gate column")
    assert_close(got[..., o + 2 * dv + 1], ex[..., o + 2 * dv + 1], "input pre-gate column")


def _sums_close(got, exp, terms_abs, what):
    err = np.abs(np.asarray(got, np.float64) - exp)
    assert np.all(err <= 1e-5 * terms_abs + 1e-30), f"{what}: err {err} vs {terms_abs}"


def _term_magnitudes(wl, x2, w_proj, A, b_dt, d_alpha):
    """sum over tokens of |dA term| and |db_dt term| per head (for the tolerance)."""
    P = wl.P
    rows = [h * P + 4 * wl.n + 2 * wl.d_v for h in range(wl.H)]
    z = x2.astype(np.float64) @ np.asarray(w_proj, np.float64)[rows].T + b_dt
    alpha = O.forget_gate(z - b_dt, np.asarray(A, np.float64), np.asarray(b_dt, np.float64))
    da = d_alpha.reshape(-1, wl.H).astype(np.float64)
    tA = np.sum(np.abs(da * O.softplus(z) * alpha), 0)
    tb = np.sum(np.abs(da * A * alpha * O.sigmoid(z)), 0)
    return tA, tb


def _run(wl, d, grads_h, prod=None):
    dm = dims_for(wl)
    if prod is None:
        prod = ops.select(dm, d["x"], d["w_proj"], d["A"], d["b_dt"])
    gd = {k: to_dev(v) for k, v in grads_h.items()}
    out = ops.select_backward(dm, prod, d["x"], d["w_proj"], d["A"], d["b_dt"], gd)
    torch.cuda.synchronize()
    return prod, out


CASES = [
    synth.WORKLOADS["tiny"],
    synth.small("tiny", gate_act=O.GATE_NONE, B=2, T=37),
    synth.small("tiny", gate_act=O.GATE_SILU, T=50),
    synth.small("layer1p4b", B=1, T=40, d_model=512, H=2, n=40, W=16, R=16, d_v=64,
                gate_act=O.GATE_SILU),
    synth.small("layer1p4b", B=2, T=160, d_model=256, n=40, W=16, R=16, d_v=32),
    # n = 12: 128 of 144 slots written, every half index repeated about ten times
    synth.small("layer1p4b", B=1, T=48, d_model=128, H=3, n=12, W=128, R=100, d_v=64,
                gate_act=O.GATE_NONE),
    synth.small("layer1p4b", B=1, T=200, d_model=2048, H=2, n=362, W=64, R=64, d_v=128),
    # the largest counts and half size: 128 entries per role, a 4354-column head row
    synth.small("layer1p4b", B=1, T=24, d_model=256, H=2, n=1024, W=128, R=128, d_v=128),
]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: f"{w.name}-B{w.B}T{w.T}n{w.n}W{w.W}g{w.gate_act}")
def test_select_backward_matches_oracle(wl):
    h, d = layer_inputs(wl, seed=3, with_state=False)
    rng = np.random.default_rng(5)
    grads = _grads(rng, wl)
    prod, (dy, dA, db) = _run(wl, d, grads)
    ph = {k: host(prod[k]) for k in ("idx_w", "wt_w", "idx_r", "wt_r")}
    x2 = h["x"].reshape(-1, wl.d_model)
    flat = lambda a: a.reshape((-1,) + a.shape[2:])
    exp = _oracle_rows(wl, x2, h["w_proj"], h["A"], h["b_dt"], {k: flat(v) for k, v in ph.items()},
                       {k: flat(v) for k, v in grads.items()})
    _check_rows(wl, host(dy).reshape(-1, wl.H * wl.P), exp["dY"], {k: flat(v) for k, v in grads.items()},
                {k: flat(v) for k, v in ph.items()})
    tA, tb = _term_magnitudes(wl, x2, h["w_proj"], h["A"], h["b_dt"], grads["d_alpha"])
    _sums_close(host(dA), exp["dA"], tA, "dA")
    _sums_close(host(db), exp["db_dt"], tb, "db_dt")
    # deterministic: a second call gives the same bits
    _, (dy2, dA2, db2) = _run(wl, d, grads, prod)
    for a, b, what in ((dy, dy2, "dY"), (dA, dA2, "dA"), (db, db2, "db_dt")):
        assert torch.equal(a, b), f"{what} differs between two calls"


def test_select_backward_full_size_sampled():
    """The 1.4B-like layer at full size (B=8, T=4096, H=4, N=131072): sampled rows of
    dY, and dA / db_dt over all 32768 tokens."""
    wl = synth.WORKLOADS["layer1p4b"]
    h, d = layer_inputs(wl, seed=0, with_state=False)
    rng = np.random.default_rng(11)
    grads = _grads(rng, wl)
    prod, (dy, dA, db) = _run(wl, d, grads)
    M = wl.tokens
    rows = np.unique(np.concatenate([[0, 1, M - 1], rng.integers(0, M, 61)]))
    say(f"  checking {rows.size} sampled token rows of {M}")
    x2 = h["x"].reshape(M, wl.d_model)
    pick = lambda t: host(t).reshape((M,) + tuple(t.shape[2:]))[rows]
    ph = {k: pick(prod[k]) for k in ("idx_w", "wt_w", "idx_r", "wt_r")}
    gr = {k: v.reshape((M,) + v.shape[2:])[rows] for k, v in grads.items()}
    exp = _oracle_rows(wl, x2[rows], h["w_proj"], h["A"], h["b_dt"], ph, gr)
    _check_rows(wl, host(dy).reshape(M, -1)[rows], exp["dY"], gr, ph)
    # the per-head sums over every token
    P = wl.P
    cols = [hh * P + 4 * wl.n + 2 * wl.d_v for hh in range(wl.H)]
    z = x2.astype(np.float64) @ np.asarray(h["w_proj"], np.float64)[cols].T + h["b_dt"]
    A = np.asarray(h["A"], np.float64)
    alpha = np.exp(-A * O.softplus(z))
    da = grads["d_alpha"].reshape(M, wl.H).astype(np.float64)
    eA = np.sum(da * (-O.softplus(z) * alpha), 0)
    eb = np.sum(da * (-A * alpha * O.sigmoid(z)), 0)
    tA, tb = _term_magnitudes(wl, x2, h["w_proj"], h["A"], h["b_dt"], grads["d_alpha"])
    _sums_close(host(dA), eA, tA, "dA")
    _sums_close(host(db), eb, tb, "db_dt")
