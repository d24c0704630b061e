"""Pins of the oracle's chunkwise backward (scan_backward_chunkwise).

The chunkwise backward reorders the reverse walk's arithmetic: per chunk, the
key-weighted rule's de comes from the transposed triangular system, and every slot
the chunk touches is then walked back on its own.  So its results are fixed by
scan_backward(), which is pinned on its own by central differences of the forward
(tests/test_oracle_backward_pins.py, tests/test_oracle_gdn_backward_pins.py): for
every chunk size, from one token to more than the whole sequence, every gradient,
the restored state and the initial-state gradient must agree within fp64 rounding,
on slot spaces small enough that the tokens of a chunk share many slots and read
slots that other tokens write.  Planted mistakes in the chunkwise form must fail.
"""
import inspect

import numpy as np
import pytest

from oracle import sdm_oracle as O

SEQ = {"slot": O.scan, "gdn": O.scan_gdn}


def _case(seed, N, T, W, R, dv, rule, alpha=None, beta=None):
    rng = np.random.default_rng(seed)
    ids = lambda k: np.stack([np.sort(rng.choice(N, k, replace=False)) for _ in range(T)])
    w = dict(idx_w=ids(W), wt_w=rng.dirichlet(np.ones(W), T), idx_r=ids(R),
             wt_r=rng.dirichlet(np.ones(R), T), v=rng.standard_normal((T, dv)),
             alpha=rng.uniform(0.3, 1.0, T) if alpha is None else np.full(T, alpha),
             beta=rng.uniform(0.0, 1.0, T) if beta is None else np.full(T, beta))
    m0 = rng.standard_normal((N, dv))
    y, MT, log = SEQ[rule](m0, **w, record=True)
    rest = dict(y=y, gate=rng.uniform(0.2, 1.0, (T, dv)), gamma_h=rng.uniform(0.5, 1.5, dv),
                eps=1e-6, d_out=rng.standard_normal((T, dv)), d_state=rng.standard_normal((N, dv)))
    return dict(state_T=MT, log=log, **w, **rest), m0


def _agree(case, C, rule, fn=None):
    fn = fn or O.scan_backward_chunkwise
    g1, M1, dM1 = O.scan_backward(**case, rule=rule)
    g2, M2, dM2 = fn(**case, C=C, rule=rule)
    for k in g1:
        scale = max(1.0, np.abs(g1[k]).max())
        np.testing.assert_allclose(g2[k], g1[k], rtol=0, atol=1e-12 * scale,
                                   err_msg=f"{k} C={C} {rule}")
    np.testing.assert_array_equal(M2, M1)
    scale = max(1.0, np.abs(dM1).max())
    np.testing.assert_allclose(dM2, dM1, rtol=0, atol=1e-12 * scale, err_msg=f"dM C={C} {rule}")


@pytest.mark.parametrize("rule", ["slot", "gdn"])
@pytest.mark.parametrize("N,T,W,R,dv", [(12, 11, 4, 3, 5),    # most tokens share slots
                                        (6, 9, 6, 6, 2),      # every slot, every token
                                        (64, 20, 5, 7, 3),    # few collisions
                                        (16, 13, 1, 1, 4)])   # one slot per token
def test_chunkwise_backward_equals_reverse_walk(rule, N, T, W, R, dv):
    case, m0 = _case(N * 100 + T, N, T, W, R, dv, rule)
    for C in (1, 2, 3, 4, 5, T - 1, T, T + 7):
        _agree(case, C, rule)
    # the restored state is the forward's initial state, bit for bit
    np.testing.assert_array_equal(O.scan_backward_chunkwise(**case, C=4, rule=rule)[1], m0)


@pytest.mark.parametrize("rule", ["slot", "gdn"])
def test_identity_gates_pass_gradients_through(rule):
    # alpha = 1, beta = 0: nothing is written, so dL/dM0 is dL/dM_T plus every read's
    # q dy on its row, and no gradient reaches v
    case, _ = _case(5, 10, 8, 3, 4, 3, rule, alpha=1.0, beta=0.0)
    g, _, dM = O.scan_backward_chunkwise(**case, C=3, rule=rule)
    dy = O._norm_gate_backward(case["y"], case["gate"], case["gamma_h"], 1e-6, case["d_out"])[0]
    exp = case["d_state"].copy()
    for t in range(8):
        for k, j in enumerate(case["idx_r"][t]):
            exp[j] += case["wt_r"][t, k] * dy[t]
    np.testing.assert_allclose(dM, exp, rtol=0, atol=1e-13)
    assert not g["d_v"].any()


# ---- planted mistakes ----------------------------------------------------------------
_SRC = inspect.getsource(O.scan_backward_chunkwise)
_MUTANTS = {
    "reads' gradients left out of h": ("hu += a_tu * dy[t]", "pass"),
    "h from its own token's reads only": ("for t in range(u, end + 1):",
                                          "for t in range(u, u + 1):"),
    "end gradient undecayed in h": ("hu += wt_w[u, k] * G(int(j), u, end) * dM[j]",
                                    "hu += wt_w[u, k] * dM[j]"),
    "no back substitution": ("rhs -= b_tu * de[t]", "pass"),
    "de left out of the slot walk": ("D = alpha[t] * (D - wt_w[t, k] * de[t])",
                                     "D = alpha[t] * D"),
    "reads see the chunk-end row": ("F = log[t, k]", "pass"),
    "slot decay without the delta factor": ("D = alpha[t] * (1.0 - beta[t] * wt_w[t, k]) * D",
                                            "D = alpha[t] * D"),
    "decay includes the writing token": ("for u in range(s + 1, t + 1):",
                                         "for u in range(s, t + 1):"),
}


def _mutant(kind):
    old, new = _MUTANTS[kind]
    assert _SRC.count(old) == 1, kind
    ns = dict(O.__dict__)
    exec(compile(_SRC.replace(old, new), "<mutant>", "exec"), ns)
    return ns["scan_backward_chunkwise"]


@pytest.mark.parametrize("kind", list(_MUTANTS))
def test_pins_catch_mutant(kind):
    fn = _mutant(kind)
    with pytest.raises(AssertionError):
        for rule in ("slot", "gdn"):
            case, _ = _case(1211, 12, 11, 4, 3, 5, rule)
            _agree(case, 4, rule, fn)
