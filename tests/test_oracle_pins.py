"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each test checks the oracle against one of: a hand-worked fixture in
tests/golden/ (derivation and citation inside the file), a closed form, exact
rational arithmetic of the pages' literal formulas, or brute force.  Together
they are chosen so that a dropped term, a wrong sign, a transposed operand or
index, a read before the write, or a decay of unselected rows fails at least
one test.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import sdm_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _sym(s):
    """Evaluate the few symbolic constants the fixtures use."""
    env = {"ln3": math.log(3.0), "e": math.e, "ln": math.log}
    s = s.replace("ln(e-1)", "ln(e-1)")
    if "/" in s and all(p.strip().lstrip("-").isdigit() for p in s.split("/")):
        return float(Fraction(s))
    if s == "3/4 ln3":
        return 0.75 * math.log(3.0)
    if s == "1/e":
        return 1.0 / math.e
    return float(eval(s, {"__builtins__": {}}, env))


# --------------------------------------------------------------------------
# Hand-worked fixtures
# --------------------------------------------------------------------------
def test_golden_selection_ids_scores_gap():
    g = _load("pkm_select.json")
    for case in g["cases"]:
        ids, sc, gap = O.top_slots(case["half1"], case["half2"], case["count"])
        assert ids.tolist() == case["ids"], case["name"]
        assert sc.tolist() == case["scores"], case["name"]
        assert gap == case["gap"], case["name"]


def test_golden_selection_weights():
    g = _load("pkm_select.json")
    for case in g["weights"]:
        h2 = [_sym(s) for s in case["half2_symbolic"]]
        ids, wt, _ = O.select(case["half1"], h2, case["count"])
        assert ids.tolist() == case["ids"]
        np.testing.assert_allclose(wt, case["weights"], rtol=1e-15, atol=0)


def test_golden_projection_layout():
    g = _load("projection_layout.json")
    d, s = g["d"], g["shift"]
    w = np.zeros((d, d))
    for p in range(d):
        w[p, (p + s) % d] = 1.0
    x = np.arange(d, dtype=np.float64)[None, :]
    parts = O.split_heads(O.project(x, w), g["H"], g["n"], g["d_v"])
    for h, exp in enumerate(g["heads"]):
        for k in ("kw1", "kw2", "kr1", "kr2", "v", "g"):
            assert parts[k][0, h].tolist() == exp[k], (h, k)
        assert parts["a"][0, h] == exp["a"] and parts["b"][0, h] == exp["b"]


def test_golden_gates():
    g = _load("gates.json")
    for c in g["alpha"]:
        a = _sym(c["a"]) if c["a"] != "ln(e-1)" else math.log(math.e - 1.0)
        got = O.forget_gate(a, _sym(c["A"]), _sym(c["b_dt"]))
        assert got == pytest.approx(_sym(c["alpha"]), rel=1e-15, abs=0)
    for c in g["beta"]:
        assert O.input_gate(_sym(c["b"])) == pytest.approx(_sym(c["beta"]), rel=1e-15)
    ga = g["gate_activation"]
    for c in ga["sigmoid"]:
        assert O.gate_activation(_sym(c["g"]), O.GATE_SIGMOID) == pytest.approx(_sym(c["out"]), rel=1e-15)
    for c in ga["silu"]:
        assert O.gate_activation(_sym(c["g"]), O.GATE_SILU) == pytest.approx(_sym(c["out"]), rel=1e-15)


def test_golden_scan_worked_example():
    g = _load("scan_worked.json")
    y, M = O.scan(g["state0"], g["idx_w"], g["wt_w"], g["idx_r"], g["wt_r"], g["v"],
                  g["alpha"], g["beta"])
    # every value is dyadic, so fp64 reproduces the hand derivation exactly
    assert y.tolist() == [[float(Fraction(s)) for s in r] for r in g["y"]]
    assert M.tolist() == [[float(Fraction(s)) for s in r] for r in g["state_final"]]


def test_golden_norm_gate():
    g = _load("norm_gate.json")
    for c in g["cases"]:
        out = O.rms_norm_gate(g["y"], g["gamma"], g["gate"], float(Fraction(c["eps"])))
        np.testing.assert_allclose(out, [float(Fraction(s)) for s in c["out"]], rtol=1e-15, atol=1e-15)


# --------------------------------------------------------------------------
# Selection: brute force and the product-key theorem
# --------------------------------------------------------------------------
def _brute_force_python(h1, h2, count):
    """Pure-Python definition: sort every (score, id) pair, keep the best `count`."""
    n = len(h1)
    pairs = [(-(float(h1[i]) + float(h2[j])), i * n + j) for i in range(n) for j in range(n)]
    pairs.sort()
    return sorted(p[1] for p in pairs[:count])


def _product_key_select(h1, h2, count):
    """The product-key shortcut as the pages describe it: best k of each half,
    then the k*k outer-sum combinations, then the best `count` of those."""
    n = len(h1)
    k = min(count, n)
    top1 = sorted(range(n), key=lambda i: (-float(h1[i]), i))[:k]
    top2 = sorted(range(n), key=lambda j: (-float(h2[j]), j))[:k]
    cands = [(-(float(h1[i]) + float(h2[j])), i * n + j) for i in top1 for j in top2]
    cands.sort()
    return sorted(c[1] for c in cands[:count]), len(cands)


@pytest.mark.parametrize("n,count", [(4, 1), (4, 3), (5, 8), (8, 8), (8, 20), (16, 8), (6, 36)])
def test_selection_equals_python_brute_force(n, count):
    rng = np.random.default_rng(100 + n * 7 + count)
    for trial in range(30):
        if trial % 3 == 0:      # heavy ties: a few quantised levels
            h1 = rng.integers(-2, 3, n).astype(np.float64) * 0.5
            h2 = rng.integers(-2, 3, n).astype(np.float64) * 0.5
        else:
            h1 = rng.standard_normal(n)
            h2 = rng.standard_normal(n)
        ids, sc, _ = O.top_slots(h1, h2, count)
        assert ids.tolist() == _brute_force_python(h1, h2, count)
        np.testing.assert_array_equal(sc, [h1[i // n] + h2[i % n] for i in ids])


@pytest.mark.parametrize("n,count", [(16, 8), (32, 8), (24, 64), (64, 64), (40, 128)])
def test_product_key_shortcut_reaches_oracle_set(n, count):
    """The shortcut's set equals the oracle's full-N selection, ties included."""
    rng = np.random.default_rng(7 * n + count)
    for trial in range(12):
        if trial % 2:
            h1 = rng.integers(-3, 4, n).astype(np.float64)
            h2 = rng.integers(-3, 4, n).astype(np.float64)
        else:
            h1 = rng.standard_normal(n).astype(np.float32).astype(np.float64)
            h2 = rng.standard_normal(n).astype(np.float32).astype(np.float64)
        ids, _, _ = O.top_slots(h1, h2, count)
        pk, ncand = _product_key_select(h1, h2, count)
        assert ids.tolist() == pk
        assert ncand == min(count, n) ** 2


def test_candidate_count_matches_page_example():
    g = _load("pkm_select.json")["candidate_count"]
    rng = np.random.default_rng(3)
    h1, h2 = rng.standard_normal(362), rng.standard_normal(362)
    _, ncand = _product_key_select(h1, h2, g["k"])
    assert ncand == g["candidates"]


def test_selection_gap_and_near_ties():
    h1 = np.array([0.0, 1e-7])
    h2 = np.array([0.0, 1.0])
    ids, _, gap = O.top_slots(h1, h2, 2)     # scores 0, 1, 1e-7, 1+1e-7
    assert ids.tolist() == [1, 3]
    assert gap == pytest.approx(1.0 - 1e-7, rel=1e-12)
    _, _, gap1 = O.top_slots(h1, h2, 1)
    assert gap1 == pytest.approx(1e-7, rel=1e-6)
    _, _, gapN = O.top_slots(h1, h2, 4)
    assert gapN == float("inf")


def test_selection_rejects_bad_count():
    with pytest.raises(ValueError):
        O.top_slots([0.0, 1.0], [0.0, 1.0], 5)
    with pytest.raises(ValueError):
        O.top_slots([0.0, 1.0], [0.0, 1.0], 0)


def test_softmax_weights_invariants():
    rng = np.random.default_rng(11)
    for count in (1, 2, 7, 64):
        h1, h2 = rng.standard_normal(16), rng.standard_normal(16)
        ids, wt, _ = O.select(h1, h2, count)
        assert wt.sum() == pytest.approx(1.0, abs=1e-15 * count)
        sc = np.array([h1[i // 16] + h2[i % 16] for i in ids])
        # monotone: a higher score never gets a lower weight; ratio = exp(diff)
        order = np.argsort(sc)
        assert np.all(np.diff(wt[order]) >= 0)
        if count > 1:
            assert wt[0] / wt[1] == pytest.approx(math.exp(sc[0] - sc[1]), rel=1e-13)
    ids, wt, _ = O.select([0.3], [0.2], 1)
    assert wt.tolist() == [1.0]


# --------------------------------------------------------------------------
# Scan: exact rational arithmetic of the literal update, closed forms, invariants
# --------------------------------------------------------------------------
def _random_walk(rng, T, n, W, R, d_v, dyadic=False):
    N = n * n
    idx_w = np.stack([np.sort(rng.choice(N, W, replace=False)) for _ in range(T)])
    idx_r = np.stack([np.sort(rng.choice(N, R, replace=False)) for _ in range(T)])
    if dyadic:
        q = lambda *s: rng.integers(-64, 65, s) / 32.0
        pos = lambda *s: rng.integers(1, 33, s) / 32.0
        return dict(state0=q(N, d_v), idx_w=idx_w, wt_w=pos(T, W), idx_r=idx_r, wt_r=pos(T, R),
                    v=q(T, d_v), alpha=pos(T), beta=pos(T))
    wt_w = rng.dirichlet(np.ones(W), T)
    wt_r = rng.dirichlet(np.ones(R), T)
    return dict(state0=rng.standard_normal((N, d_v)) * 0.02, idx_w=idx_w, wt_w=wt_w, idx_r=idx_r,
                wt_r=wt_r, v=rng.standard_normal((T, d_v)), alpha=rng.uniform(0.5, 1.0, T),
                beta=rng.uniform(0.0, 1.0, T))


def _scan_rational(w):
    """The pages' literal update and read, evaluated exactly over the rationals."""
    M = [[Fraction(float(a)) for a in row] for row in w["state0"]]
    ys = []
    for t in range(len(w["alpha"])):
        al, be = Fraction(float(w["alpha"][t])), Fraction(float(w["beta"][t]))
        v = [Fraction(float(a)) for a in w["v"][t]]
        for i, k in zip(w["idx_w"][t], w["wt_w"][t]):
            mt = [al * m for m in M[i]]
            M[i] = [a + be * Fraction(float(k)) * (vv - a) for a, vv in zip(mt, v)]
        ys.append([sum(Fraction(float(q)) * M[i][c] for i, q in zip(w["idx_r"][t], w["wt_r"][t]))
                   for c in range(len(v))])
    return ys, M


@pytest.mark.parametrize("seed", [0, 1])
def test_scan_matches_exact_rational_literal_form(seed):
    rng = np.random.default_rng(seed)
    w = _random_walk(rng, T=8, n=3, W=4, R=3, d_v=3)
    y, M = O.scan(**w)
    ys, Ms = _scan_rational(w)
    np.testing.assert_allclose(y, np.array(ys, dtype=float), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(M, np.array(Ms, dtype=float), rtol=1e-13, atol=1e-15)


def test_scan_dyadic_inputs_exact():
    rng = np.random.default_rng(5)
    w = _random_walk(rng, T=5, n=2, W=2, R=2, d_v=2, dyadic=True)
    y, M = O.scan(**w)
    ys, Ms = _scan_rational(w)
    # few enough dyadic operations that fp64 represents every intermediate exactly
    assert y.tolist() == [[float(a) for a in r] for r in ys]
    assert M.tolist() == [[float(a) for a in r] for r in Ms]


def test_unselected_rows_bit_identical():
    rng = np.random.default_rng(2)
    w = _random_walk(rng, T=40, n=8, W=4, R=4, d_v=5)
    _, M = O.scan(**w)
    touched = np.zeros(64, bool)
    touched[np.unique(w["idx_w"])] = True
    assert (~touched).any()
    assert np.array_equal(M[~touched], np.asarray(w["state0"])[~touched])
    assert not np.array_equal(M[touched], np.asarray(w["state0"])[touched])


def test_alpha_one_beta_zero_is_identity():
    rng = np.random.default_rng(3)
    w = _random_walk(rng, T=20, n=4, W=5, R=3, d_v=4)
    w["alpha"] = np.ones(20)
    w["beta"] = np.zeros(20)
    y, M = O.scan(**w)
    assert np.array_equal(M, w["state0"])
    exp = np.einsum("tr,trd->td", w["wt_r"], np.asarray(w["state0"])[w["idx_r"]])
    np.testing.assert_allclose(y, exp, rtol=1e-14, atol=1e-17)


def test_full_input_gate_overwrites_with_value():
    rng = np.random.default_rng(4)
    w = _random_walk(rng, T=6, n=4, W=1, R=1, d_v=6)
    w["beta"] = np.ones(6)
    w["wt_w"] = np.ones((6, 1))
    w["wt_r"] = np.ones((6, 1))
    w["idx_r"] = w["idx_w"].copy()
    y, M = O.scan(**w)
    # c = beta * k = 1: the slot becomes v_t, up to the roundings of v - alpha M and
    # the sum, i.e. a few ulp of max(|v|, |alpha M|) ~ 3
    np.testing.assert_allclose(y, w["v"], rtol=0, atol=2e-15)
    last = {int(w["idx_w"][t, 0]): t for t in range(6)}
    for s, t in last.items():
        np.testing.assert_allclose(M[s], w["v"][t], rtol=0, atol=2e-15)


def test_single_slot_closed_form_constant_gates():
    # N = W = R = 1: M_t = rho M_{t-1} + c v with rho = (1-c) alpha, c = beta * 1
    T, al, be, m0, v = 50, 0.9, 0.3, 0.7, 2.5
    y, M = O.scan([[m0]], np.zeros((T, 1), int), np.ones((T, 1)), np.zeros((T, 1), int),
                  np.ones((T, 1)), np.full((T, 1), v), np.full(T, al), np.full(T, be))
    rho = (1 - be) * al
    t = np.arange(1, T + 1)
    exp = rho ** t * m0 + be * v * (1 - rho ** t) / (1 - rho)
    np.testing.assert_allclose(y[:, 0], exp, rtol=1e-13)
    assert M[0, 0] == pytest.approx(exp[-1], rel=1e-13)


def test_single_slot_closed_form_varying_gates():
    rng = np.random.default_rng(8)
    T = 30
    al, be, v = rng.uniform(0.2, 1, T), rng.uniform(0, 1, T), rng.standard_normal(T)
    m0 = 0.4
    y, _ = O.scan([[m0]], np.zeros((T, 1), int), np.ones((T, 1)), np.zeros((T, 1), int),
                  np.ones((T, 1)), v[:, None], al, be)
    rho = (1 - be) * al
    for t in range(T):   # M_t = prod_{s<=t} rho_s m0 + sum_s c_s v_s prod_{s<u<=t} rho_u
        exp = np.prod(rho[:t + 1]) * m0 + sum(be[s] * v[s] * np.prod(rho[s + 1:t + 1])
                                              for s in range(t + 1))
        assert y[t, 0] == pytest.approx(exp, rel=1e-12, abs=1e-15)


def test_read_of_one_hot_memory_returns_scattered_weights():
    # d_v = N, M0 = identity rows, no writes (beta = 0, alpha = 1): y_t[i] = q^(i)
    rng = np.random.default_rng(9)
    w = _random_walk(rng, T=10, n=3, W=2, R=4, d_v=9)
    w["state0"] = np.eye(9)
    w["alpha"], w["beta"] = np.ones(10), np.zeros(10)
    y, _ = O.scan(**w)
    for t in range(10):
        exp = np.zeros(9)
        exp[w["idx_r"][t]] = w["wt_r"][t]
        assert np.array_equal(y[t], exp)


def test_scan_linear_in_state_and_values():
    rng = np.random.default_rng(10)
    w1 = _random_walk(rng, T=25, n=4, W=3, R=3, d_v=4)
    w2 = dict(w1, state0=rng.standard_normal((16, 4)), v=rng.standard_normal((25, 4)))
    y1, M1 = O.scan(**w1)
    y2, M2 = O.scan(**w2)
    w3 = dict(w1, state0=2.0 * np.asarray(w1["state0"]) - 3.0 * w2["state0"],
              v=2.0 * np.asarray(w1["v"]) - 3.0 * w2["v"])
    y3, M3 = O.scan(**w3)
    np.testing.assert_allclose(y3, 2 * y1 - 3 * y2, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(M3, 2 * M1 - 3 * M2, rtol=1e-11, atol=1e-13)


def test_scan_chunked_equals_whole():
    rng = np.random.default_rng(12)
    w = _random_walk(rng, T=30, n=4, W=4, R=4, d_v=3)
    y, M = O.scan(**w)
    cut = 13
    first = {k: (v[:cut] if k != "state0" else v) for k, v in w.items()}
    y1, Mc = O.scan(**first)
    second = {k: (v[cut:] if k != "state0" else Mc) for k, v in w.items()}
    y2, M2 = O.scan(**second)
    assert np.array_equal(np.concatenate([y1, y2]), y)
    assert np.array_equal(M2, M)


def test_norm_gate_scale_invariance_and_rms():
    rng = np.random.default_rng(13)
    y = rng.standard_normal((5, 16))
    gam, gate = rng.uniform(0.5, 2, 16), rng.uniform(0, 1, (5, 16))
    o1 = O.rms_norm_gate(y, gam, gate, 0.0)
    o2 = O.rms_norm_gate(7.5 * y, gam, gate, 0.0)
    np.testing.assert_allclose(o1, o2, rtol=1e-14)
    o3 = O.rms_norm_gate(y, np.ones(16), np.ones((5, 16)), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(o3 ** 2, axis=-1)), 1.0, rtol=1e-14)


# --------------------------------------------------------------------------
# Whole path: relabelling, batch independence
# --------------------------------------------------------------------------
def _tiny_layer(rng, B=2, T=12, d=8, H=2, n=3, d_v=4, W=3, R=2):
    P = 4 * n + 2 * d_v + 2
    return dict(x=rng.standard_normal((B, T, d)), w_proj=rng.standard_normal((H * P, d)) / 3,
                A=np.ones(H), b_dt=rng.uniform(-4, -1, H), gamma=np.ones((H, d_v)),
                state0=rng.standard_normal((B, H, n * n, d_v)) * 0.02, H=H, n=n, d_v=d_v, W=W, R=R)


def test_relabelling_slots_permutes_ids_and_keeps_outputs():
    rng = np.random.default_rng(14)
    L = _tiny_layer(rng)
    H, n, d_v = L["H"], L["n"], L["d_v"]
    P = 4 * n + 2 * d_v + 2
    sig, tau = rng.permutation(n), rng.permutation(n)   # new column c of half 1 = old sig[c]
    w = L["w_proj"].reshape(H, P, -1).copy()
    for off, perm in ((0, sig), (n, tau), (2 * n, sig), (3 * n, tau)):
        w[:, off:off + n] = w[:, off + perm]
    L2 = dict(L, w_proj=w.reshape(H * P, -1))
    # old slot (sig[i'], tau[j']) is new slot (i', j'): move the memory rows along
    old_of_new = (sig[:, None] * n + tau[None, :]).reshape(-1)
    L2["state0"] = L["state0"][:, :, old_of_new]
    out1, st1, a1 = O.forward(**L)
    out2, st2, a2 = O.forward(**L2)
    np.testing.assert_allclose(out2, out1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(st2, st1[:, :, old_of_new], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(np.sort(old_of_new[a2["idx_w"]], -1), a1["idx_w"])


def test_batch_entries_are_independent():
    rng = np.random.default_rng(15)
    L = _tiny_layer(rng)
    out, st, _ = O.forward(**L)
    L1 = dict(L, x=L["x"][1:], state0=L["state0"][1:])
    out1, st1, _ = O.forward(**L1)
    assert np.array_equal(out[1:], out1) and np.array_equal(st[1:], st1)


def test_gate_ranges():
    a = np.linspace(-30, 30, 101)
    al = O.forget_gate(a, 1.0, -2.0)
    assert np.all((al > 0) & (al <= 1)) and np.all(np.diff(al) < 0)
    assert np.all(O.forget_gate(a, 0.0, -2.0) == 1.0)
    be = O.input_gate(np.linspace(-20, 20, 41))
    assert np.all((be > 0) & (be < 1)) and np.all(np.diff(be) > 0)


# --------------------------------------------------------------------------
# Whole layer from x: a hand-worked fixture in which every column block, every
# head's gates and every head's norm weight carries its own value, so that a
# mix-up of write and read halves, of the a and b pre-gates, of v and the gate
# vector, or of one head's norm weight for another's changes the expected output
# --------------------------------------------------------------------------
def _val(s):
    """Value of a fixture entry: an integer or fraction, or +-ln3."""
    s = s.strip()
    if s.lstrip("-") == "ln3":
        return -math.log(3.0) if s.startswith("-") else math.log(3.0)
    return float(Fraction(s))


def _vals(a):
    return np.vectorize(_val, otypes=[float])(np.array(a, dtype=object))


def _wiring():
    g = _load("layer_wiring.json")
    H, n, d_v = g["H"], g["n"], g["d_v"]
    P = 4 * n + 2 * d_v + 2
    x = _vals(g["x"]).reshape(1, len(g["x"]), H * P)     # [B=1, T, H*P]
    return g, x, np.eye(H * P)


def test_golden_layer_wiring_pass_a():
    g, x, w = _wiring()
    e = g["expected"]
    a = O.pass_a(x, w, _vals(g["A"]), _vals(g["b_dt"]), g["H"], g["n"], g["d_v"], g["W"], g["R"])
    assert a["idx_w"][0].tolist() == e["idx_w"]
    assert a["idx_r"][0].tolist() == e["idx_r"]
    assert np.all(a["wt_w"] == 1.0) and np.all(a["wt_r"] == 1.0)
    for k, key in (("alpha", "alpha"), ("beta", "beta"), ("v", "v"), ("g", "gate")):
        np.testing.assert_allclose(a[k][0], _vals(e[key]), rtol=1e-12, atol=1e-12, err_msg=k)


def test_golden_layer_wiring_forward():
    g, x, w = _wiring()
    e = g["expected"]
    out, st, _ = O.forward(x, w, _vals(g["A"]), _vals(g["b_dt"]), _vals(g["gamma"]),
                           _vals(g["state0"])[None], g["H"], g["n"], g["d_v"], g["W"], g["R"],
                           eps=_val(g["eps"]))
    np.testing.assert_allclose(out[0], _vals(e["out"]), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st[0], _vals(e["state_final"]), rtol=1e-12, atol=1e-12)
