"""Pins of the oracle's Gated-DeltaNet-form variant (scan_gdn).

The pages state that with every slot selected (W = R = N = d_qk) and a dense
key the layer becomes Gated DeltaNet's update ("与 GDN 的关系" section of the
ai-paper-analysis.pages.dev summary; section 二 of the m.163.com article).  The
first pin runs an independent dense, matrix-form gated delta recurrence
S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  y_t = S_t q_t
and compares it with scan_gdn given all N slots, the dense key as write weights
and the dense query as read weights.  The others fix special cases.
"""
import numpy as np

from oracle import sdm_oracle as O


def _dense_gdn(S0, K, Q, V, alpha, beta):
    """Matrix-form gated delta rule; S [d_v, d_k]."""
    S = np.array(S0, dtype=np.float64)
    d_k = S.shape[1]
    ys = []
    for k, q, v, a, b in zip(K, Q, V, alpha, beta):
        S = a * S @ (np.eye(d_k) - b * np.outer(k, k)) + b * np.outer(v, k)
        ys.append(S @ q)
    return np.array(ys), S


def _case(rng, T=40, d_k=16, d_v=8):
    K = rng.standard_normal((T, d_k))
    K /= np.linalg.norm(K, axis=1, keepdims=True)  # GDN's L2-normalised keys
    Q = rng.standard_normal((T, d_k))
    V = rng.standard_normal((T, d_v))
    alpha = rng.uniform(0.3, 1.0, T)
    beta = rng.uniform(0.0, 1.0, T)
    S0 = rng.standard_normal((d_v, d_k))
    return K, Q, V, alpha, beta, S0


def test_all_slots_selected_equals_dense_gated_deltanet():
    rng = np.random.default_rng(11)
    K, Q, V, alpha, beta, S0 = _case(rng)
    T, d_k = K.shape
    ids = np.tile(np.arange(d_k), (T, 1))
    y, M = O.scan_gdn(S0.T, ids, K, ids, Q, V, alpha, beta)
    y_ref, S = _dense_gdn(S0, K, Q, V, alpha, beta)
    assert np.allclose(M, S.T, rtol=0, atol=1e-11)
    assert np.allclose(y, y_ref, rtol=0, atol=1e-11)
    # the per-slot rule is a different recurrence here (the pages' printed form)
    y_slot, M_slot = O.scan(S0.T, ids, K, ids, Q, V, alpha, beta)
    assert np.max(np.abs(M_slot - S.T)) > 1e-3


def test_order_of_the_write_set_does_not_matter():
    rng = np.random.default_rng(12)
    K, Q, V, alpha, beta, S0 = _case(rng, T=25)
    T, d_k = K.shape
    ids = np.tile(np.arange(d_k), (T, 1))
    perm = np.array([rng.permutation(d_k) for _ in range(T)])
    Kp = np.take_along_axis(K, perm, axis=1)
    y0, M0 = O.scan_gdn(S0.T, ids, K, ids, Q, V, alpha, beta)
    y1, M1 = O.scan_gdn(S0.T, perm, Kp, ids, Q, V, alpha, beta)
    assert np.allclose(M0, M1, rtol=0, atol=1e-12) and np.allclose(y0, y1, rtol=0, atol=1e-12)


def test_single_slot_of_weight_one_matches_the_per_slot_rule():
    # one slot, weight 1: v - sum_j k_j Mtilde[j] = v - Mtilde[i], the pages' form
    rng = np.random.default_rng(13)
    T, N, d_v = 60, 10, 4
    M0 = rng.standard_normal((N, d_v))
    iw = rng.integers(0, N, (T, 1))
    ir = rng.integers(0, N, (T, 3))
    wr = rng.dirichlet(np.ones(3), T)
    V = rng.standard_normal((T, d_v))
    a, b = rng.uniform(0.2, 1, T), rng.uniform(0, 1, T)
    one = np.ones((T, 1))
    y0, M_slot = O.scan(M0, iw, one, ir, wr, V, a, b)
    y1, M_gdn = O.scan_gdn(M0, iw, one, ir, wr, V, a, b)
    assert np.allclose(M_slot, M_gdn, rtol=0, atol=1e-14)
    assert np.allclose(y0, y1, rtol=0, atol=1e-14)


def test_identity_gates_and_untouched_rows():
    rng = np.random.default_rng(14)
    T, N, d_v, W = 30, 64, 8, 5
    M0 = rng.standard_normal((N, d_v))
    iw = np.array([rng.choice(N // 2, W, replace=False) for _ in range(T)])  # rows < 32 only
    ww = rng.dirichlet(np.ones(W), T)
    ir = np.array([rng.choice(N, 4, replace=False) for _ in range(T)])
    wr = rng.dirichlet(np.ones(4), T)
    V = rng.standard_normal((T, d_v))
    _, M = O.scan_gdn(M0, iw, ww, ir, wr, V, np.ones(T), np.zeros(T))
    assert np.array_equal(M, M0)  # alpha = 1, beta = 0: nothing changes
    _, M = O.scan_gdn(M0, iw, ww, ir, wr, V, rng.uniform(0.2, 1, T), rng.uniform(0, 1, T))
    assert np.array_equal(M[N // 2:], M0[N // 2:])  # never-written rows untouched


# ---- planted mistakes in scan_gdn (CPU): each must fail a pin above ----------
import pytest  # noqa: E402

F64 = np.float64


def _gdn_mutant(kind):
    def scan_gdn(state0, idx_w, wt_w, idx_r, wt_r, v, alpha, beta):
        M = np.array(state0, dtype=F64, copy=True)
        idx_w, idx_r = np.asarray(idx_w), np.asarray(idx_r)
        wt_w, wt_r = np.asarray(wt_w, F64), np.asarray(wt_r, F64)
        v, alpha, beta = np.asarray(v, F64), np.asarray(alpha, F64), np.asarray(beta, F64)
        y = np.zeros((idx_w.shape[0], M.shape[1]))
        for t in range(idx_w.shape[0]):
            rows, k = idx_w[t], wt_w[t]
            mt = alpha[t] * M[rows]
            if kind == "prediction_without_forget":
                pred = k @ M[rows]
            elif kind == "prediction_with_read_weights":
                pred = np.resize(wt_r[t], k.size) @ mt
            elif kind == "sequential_rows":  # rows updated one after another
                for r, kk in zip(rows, k):
                    M[r] = alpha[t] * M[r]
                    M[r] = M[r] + beta[t] * kk * (v[t] - k @ M[rows])
                y[t] = wt_r[t] @ M[idx_r[t]]
                continue
            else:
                pred = k @ mt
            M[rows] = mt + (beta[t] * k)[:, None] * (v[t] - pred)[None, :]
            y[t] = wt_r[t] @ M[idx_r[t]]
        return y, M
    return scan_gdn


@pytest.mark.parametrize("kind", ["prediction_without_forget", "prediction_with_read_weights",
                                  "sequential_rows"])
def test_pins_catch_gdn_mutant(kind, monkeypatch):
    monkeypatch.setattr(O, "scan_gdn", _gdn_mutant(kind))
    failed = 0
    for pin in (test_all_slots_selected_equals_dense_gated_deltanet,
                test_order_of_the_write_set_does_not_matter,
                test_single_slot_of_weight_one_matches_the_per_slot_rule,
                test_identity_gates_and_untouched_rows):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, kind
