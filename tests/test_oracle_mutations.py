"""Plant plausible mistakes in the oracle (CPU only) and check the pins catch each.

Every mutant replaces one oracle function for the duration of the test; the pin
suite of tests/test_oracle_pins.py must then fail at least once.
"""
import numpy as np
import pytest

from oracle import sdm_oracle as O
from tests import test_oracle_pins as pins

F64 = np.float64


def _scan_variant(decay_all=False, read_first=False, no_forget=False, sign=1.0):
    def scan(state0, idx_w, wt_w, idx_r, wt_r, v, alpha, beta, store=None, record=False):
        assert store is None and not record, "mutant covers the exact-state forward only"
        M = np.array(state0, dtype=F64, copy=True)
        idx_w, idx_r = np.asarray(idx_w), np.asarray(idx_r)
        wt_w, wt_r = np.asarray(wt_w, F64), np.asarray(wt_r, F64)
        v, alpha, beta = np.asarray(v, F64), np.asarray(alpha, F64), np.asarray(beta, F64)
        y = np.zeros((idx_w.shape[0], M.shape[1]))
        for t in range(idx_w.shape[0]):
            if read_first:
                y[t] = wt_r[t] @ M[idx_r[t]]
            if decay_all:
                M *= alpha[t]
                mt = M[idx_w[t]]
            else:
                mt = M[idx_w[t]] * (1.0 if no_forget else alpha[t])
            M[idx_w[t]] = mt + sign * (beta[t] * wt_w[t])[:, None] * (v[t][None, :] - mt)
            if not read_first:
                y[t] = wt_r[t] @ M[idx_r[t]]
        return y, M
    return scan


def _top_slots_variant(transpose_id=False, high_id_ties=False):
    def top_slots(half1, half2, count):
        h1, h2 = np.asarray(half1, F64), np.asarray(half2, F64)
        n = h1.size
        if not 1 <= count <= n * n:
            raise ValueError("count")
        S = (h1[:, None] + h2[None, :])
        if transpose_id:
            S = S.T
        S = S.reshape(-1)
        ids = np.arange(S.size)
        order = np.lexsort((-ids if high_id_ties else ids, -S))[:count]
        srt = np.sort(S)[::-1]
        gap = float(srt[count - 1] - srt[count]) if count < S.size else float("inf")
        sel = np.sort(order)
        return sel, S[sel], gap
    return top_slots


def _linear_weights(s):
    s = np.asarray(s, F64)
    return s / s.sum()


def _project_no_transpose(x, w):
    return np.asarray(x, F64) @ np.asarray(w, F64)


def _split_swapped(Y, H, n, d_v):
    p = O.__dict__["_orig_split"](Y, H, n, d_v)
    p["kw1"], p["kw2"] = p["kw2"], p["kw1"]
    return p


def _forget_no_bias(a, A, b_dt):
    return np.exp(-np.asarray(A, F64) * O.softplus(a))


def _norm_sum(y, gamma, gate, eps):
    y = np.asarray(y, F64)
    return y / np.sqrt(np.sum(y * y, -1, keepdims=True) + eps) * gamma * gate


def _beta_tanh(b):
    return np.tanh(np.asarray(b, F64))


def _select_roles_swapped(scores, n, W, R):
    """Write slots taken from the read halves and read slots from the write halves."""
    s = np.asarray(scores, F64)
    swapped = np.concatenate([s[..., 2 * n:4 * n], s[..., 0:2 * n]], axis=-1)
    return O.__dict__["_orig_select_from_scores"](swapped, n, W, R)


def _pass_a_variant(swap_ab=False, swap_vg=False):
    def pass_a(x, w_proj, A, b_dt, H, n, d_v, W, R, gate_act=O.GATE_SIGMOID):
        p = O.split_heads(O.project(x, w_proj), H, n, d_v)
        a, b = (p["b"], p["a"]) if swap_ab else (p["a"], p["b"])
        v, g = (p["g"], p["v"]) if swap_vg else (p["v"], p["g"])
        out = dict(v=v, g=O.gate_activation(g, gate_act),
                   alpha=O.forget_gate(a, np.asarray(A, F64), np.asarray(b_dt, F64)),
                   beta=O.input_gate(b),
                   scores=np.concatenate([p["kw1"], p["kw2"], p["kr1"], p["kr2"]], axis=-1))
        out.update(O.select_from_scores(out["scores"], n, W, R))
        return out
    return pass_a


def _forward_head0_gamma(x, w_proj, A, b_dt, gamma, state0, H, n, d_v, W, R, eps=1e-6,
                         gate_act=O.GATE_SIGMOID):
    """Every head normalised with head 0's weight."""
    x = np.asarray(x, F64)
    B, T = x.shape[:2]
    a = O.pass_a(x, w_proj, A, b_dt, H, n, d_v, W, R, gate_act)
    out = np.zeros((B, T, H, d_v))
    st = np.zeros(np.shape(state0))
    for b in range(B):
        for h in range(H):
            walk = {k: a[k][b, :, h] for k in ("idx_w", "wt_w", "idx_r", "wt_r", "v", "g",
                                               "alpha", "beta")}
            o, _, M = O.forward_walk(state0[b][h], walk, np.asarray(gamma, F64)[0], eps)
            out[b, :, h] = o
            st[b, h] = M
    return out, st, a


MUTANTS = {
    "forget gate decays every slot": ("scan", _scan_variant(decay_all=True)),
    "read before write": ("scan", _scan_variant(read_first=True)),
    "forget gate dropped": ("scan", _scan_variant(no_forget=True)),
    "delta sign flipped": ("scan", _scan_variant(sign=-1.0)),
    "slot id transposed": ("top_slots", _top_slots_variant(transpose_id=True)),
    "ties to highest id": ("top_slots", _top_slots_variant(high_id_ties=True)),
    "linear weights instead of softmax": ("softmax", _linear_weights),
    "projection not transposed": ("project", _project_no_transpose),
    "write halves swapped": ("split_heads", _split_swapped),
    "b_dt dropped": ("forget_gate", _forget_no_bias),
    "rms uses sum not mean": ("rms_norm_gate", _norm_sum),
    "input gate tanh": ("input_gate", _beta_tanh),
    "write and read halves swapped": ("select_from_scores", _select_roles_swapped),
    "a and b pre-gates swapped": ("pass_a", _pass_a_variant(swap_ab=True)),
    "v and gate swapped": ("pass_a", _pass_a_variant(swap_vg=True)),
    "every head normalised with head 0's weight": ("forward", _forward_head0_gamma),
}

PIN_CALLS = [
    (pins.test_golden_selection_ids_scores_gap, {}),
    (pins.test_golden_selection_weights, {}),
    (pins.test_golden_projection_layout, {}),
    (pins.test_golden_gates, {}),
    (pins.test_golden_scan_worked_example, {}),
    (pins.test_golden_norm_gate, {}),
    (pins.test_selection_equals_python_brute_force, {"n": 5, "count": 8}),
    (pins.test_softmax_weights_invariants, {}),
    (pins.test_scan_matches_exact_rational_literal_form, {"seed": 0}),
    (pins.test_unselected_rows_bit_identical, {}),
    (pins.test_single_slot_closed_form_constant_gates, {}),
    (pins.test_norm_gate_scale_invariance_and_rms, {}),
    (pins.test_golden_layer_wiring_pass_a, {}),
    (pins.test_golden_layer_wiring_forward, {}),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setitem(O.__dict__, "_orig_split", O.split_heads)
    monkeypatch.setitem(O.__dict__, "_orig_select_from_scores", O.select_from_scores)
    monkeypatch.setattr(O, attr, fn)
    failures = 0
    for call, kw in PIN_CALLS:
        try:
            call(**kw)
        except (AssertionError, ValueError, IndexError):
            failures += 1
    assert failures >= 1, f"no pin caught mutant: {name}"


def test_unmutated_oracle_passes_every_pin_call():
    for call, kw in PIN_CALLS:
        call(**kw)
