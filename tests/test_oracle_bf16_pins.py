"""Pins of the oracle's bf16 state storage (round_bf16 and scan(..., store=round_bf16)).

bf16 keeps the sign, the 8 exponent bits and the top 7 fraction bits of IEEE
binary32: 8 significant bits, normal numbers down to 2^-126, subnormals spaced
2^-133.  The storage variant rounds each written state element to the nearest
such value, ties to the even significand.  The pages keep the live state in full
precision and quantise only training checkpoints (section "训练效率" of the
ai-paper-analysis.pages.dev summary; section 八 of the m.163.com article), so
these pins come from the format's definition, an independent library conversion
(torch's float32 -> bfloat16, round-to-nearest-even) and exact rational
arithmetic, not from the pages.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import sdm_oracle as O


def _torch_bf16(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16).to(
        torch.float64).numpy()


def _exact_round_bf16(fr: Fraction) -> Fraction:
    """Nearest bf16 value of an exact rational (ties to even); finite range only."""
    if fr == 0:
        return Fraction(0)
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()  # 2^e <= a < 2^(e+2)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, -126) - 7)                 # 8 significant bits
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return (fl * quantum) if fr > 0 else -(fl * quantum)


# ---- round_bf16 ----------------------------------------------------------------
def test_round_bf16_equals_torch_on_fp32_values():
    rng = np.random.default_rng(21)
    mag = np.exp2(rng.uniform(-133, 127.9, 200_000))
    x = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    x = np.concatenate([x, rng.standard_normal(100_000).astype(np.float32),
                        np.float32([0.0, -0.0, 1.0, -1.0, 3.3895e38, 3.4e38, 1e-45, -1e-45,
                                    2.0 ** -126, 2.0 ** -127, 65504.0])])
    got = O.round_bf16(x.astype(np.float64))
    exp = _torch_bf16(x)
    assert np.array_equal(got, exp)
    assert np.array_equal(np.signbit(got), np.signbit(exp))


# hand-worked from the definition (8 significant bits, ties to even)
HALFWAY = [
    (1 + 2.0 ** -8, 1.0),                              # tie: 1.0000000|1 -> even 1.0
    (1 + 3 * 2.0 ** -8, 1 + 2.0 ** -6),                # tie: ...01|1 -> ...10
    (-(1 + 2.0 ** -8), -1.0),
    (1 + 2.0 ** -8 + 2.0 ** -40, 1 + 2.0 ** -7),       # just above a tie (below fp32's reach)
    (1 + 2.0 ** -8 - 2.0 ** -40, 1.0),                 # just below a tie
    (255.5, 256.0),                                    # 255 = 1111 1111 (odd) -> 256
    (254.5, 254.0),                                    # 254 even stays
    ((2 - 2.0 ** -8) * 2.0 ** 127, np.inf),            # tie above the largest bf16 -> overflow
    ((2 - 2.0 ** -7) * 2.0 ** 127, (2 - 2.0 ** -7) * 2.0 ** 127),   # largest bf16 itself
    (1.5 * 2.0 ** -133, 2.0 ** -132),                  # subnormal tie -> even multiple
    (2.0 ** -134, 0.0),                                # half the smallest subnormal -> 0
    (0.75 * 2.0 ** -133, 2.0 ** -133),
]


@pytest.mark.parametrize("x,want", HALFWAY)
def test_round_bf16_hand_worked(x, want):
    assert O.round_bf16(np.float64(x)) == want


def test_round_bf16_is_idempotent_and_monotone():
    rng = np.random.default_rng(22)
    x = np.sort(rng.standard_normal(50_000) * 10.0 ** rng.uniform(-5, 5, 50_000))
    r = O.round_bf16(x)
    assert np.array_equal(O.round_bf16(r), r)
    assert np.all(np.diff(r) >= 0)


def test_round_bf16_equals_exact_rational_rounding():
    rng = np.random.default_rng(23)
    x = rng.standard_normal(3000) * 10.0 ** rng.uniform(-3, 3, 3000)
    for xi, ri in zip(x, O.round_bf16(x)):
        assert Fraction(float(ri)) == _exact_round_bf16(Fraction(float(xi)))


# ---- the bf16 scan ----------------------------------------------------------------
def _walk(rng, T, N, d_v, W, R):
    iw = np.array([np.sort(rng.choice(N, W, replace=False)) for _ in range(T)])
    ir = np.array([np.sort(rng.choice(N, R, replace=False)) for _ in range(T)])
    ww = rng.dirichlet(np.ones(W), T).astype(np.float32).astype(np.float64)
    wr = rng.dirichlet(np.ones(R), T).astype(np.float32).astype(np.float64)
    v = rng.standard_normal((T, d_v)).astype(np.float32).astype(np.float64)
    a = rng.uniform(0.3, 1.0, T).astype(np.float32).astype(np.float64)
    b = rng.uniform(0.0, 1.0, T).astype(np.float32).astype(np.float64)
    M0 = O.round_bf16(rng.standard_normal((N, d_v)) * 0.5)
    return M0, iw, ww, ir, wr, v, a, b


def test_bf16_scan_one_token_is_one_rounding_of_the_exact_update():
    rng = np.random.default_rng(24)
    M0, iw, ww, ir, wr, v, a, b = _walk(rng, 1, 40, 8, 6, 5)
    _, M = O.scan(M0, iw, ww, ir, wr, v, a, b, store=O.round_bf16)
    for k, row in enumerate(iw[0]):
        c = Fraction(float(b[0])) * Fraction(float(ww[0, k]))
        for j in range(M0.shape[1]):
            mt = Fraction(float(a[0])) * Fraction(float(M0[row, j]))
            exact = mt + c * (Fraction(float(v[0, j])) - mt)
            assert Fraction(float(M[row, j])) == _exact_round_bf16(exact), (row, j)


def test_bf16_scan_state_is_representable_and_reads_see_it():
    rng = np.random.default_rng(25)
    T, N, d_v = 80, 64, 8
    M0, iw, ww, ir, wr, v, a, b = _walk(rng, T, N, d_v, 12, 10)
    y, M = O.scan(M0, iw, ww, ir, wr, v, a, b, store=O.round_bf16)
    assert np.array_equal(O.round_bf16(M), M)
    # the last token's read sees the stored (rounded) rows
    assert np.allclose(y[-1], wr[-1] @ M[ir[-1]], rtol=0, atol=1e-15)
    # one token: every read row is a stored value
    y1, M1 = O.scan(M0, iw[:1], ww[:1], ir[:1], wr[:1], v[:1], a[:1], b[:1], store=O.round_bf16)
    assert np.array_equal(y1[0], wr[0] @ M1[ir[0]])


def test_bf16_scan_overwrite_stores_rounded_v_and_identity_keeps_state():
    rng = np.random.default_rng(26)
    T, N, d_v = 30, 16, 8
    M0, iw, ww, ir, wr, v, a, b = _walk(rng, T, N, d_v, 1, 1)
    one = np.ones((T, 1))
    _, M = O.scan(M0, iw, one, ir, one, v, a, np.ones(T), store=O.round_bf16)
    last = {int(iw[t, 0]): t for t in range(T)}
    for s, t in last.items():
        assert np.array_equal(M[s], _torch_bf16(v[t].astype(np.float32)))
    _, M = O.scan(M0, iw, one, ir, one, v, np.ones(T), np.zeros(T), store=O.round_bf16)
    assert np.array_equal(M, M0)


def test_bf16_scan_stays_near_the_exact_state():
    rng = np.random.default_rng(27)
    M0, iw, ww, ir, wr, v, a, b = _walk(rng, 200, 64, 16, 16, 16)
    y_b, M_b = O.scan(M0, iw, ww, ir, wr, v, a, b, store=O.round_bf16)
    y_e, M_e = O.scan(M0, iw, ww, ir, wr, v, a, b)
    # each write adds at most half a bf16 spacing (2^-9 relative); alpha, 1 - c <= 1
    # shrink older errors, so the drift stays a few spacings of the values' size
    scale = np.max(np.abs(M_e))
    assert np.max(np.abs(M_b - M_e)) <= 8 * 2.0 ** -9 * scale
    assert np.max(np.abs(M_b - M_e)) > 0  # the rounding really happened


def test_bf16_gdn_scan_rounds_each_write_once():
    rng = np.random.default_rng(28)
    M0, iw, ww, ir, wr, v, a, b = _walk(rng, 1, 30, 4, 5, 3)
    _, M = O.scan_gdn(M0, iw, ww, ir, wr, v, a, b, store=O.round_bf16)
    k = [Fraction(float(x)) for x in ww[0]]
    for j in range(M0.shape[1]):
        mt = [Fraction(float(a[0])) * Fraction(float(M0[r, j])) for r in iw[0]]
        pred = sum(kk * m for kk, m in zip(k, mt))
        for i, row in enumerate(iw[0]):
            exact = mt[i] + Fraction(float(b[0])) * k[i] * (Fraction(float(v[0, j])) - pred)
            assert Fraction(float(M[row, j])) == _exact_round_bf16(exact)


def test_state_must_start_representable():
    M0 = np.full((4, 2), 1 + 2.0 ** -10)
    with pytest.raises(AssertionError):
        O.scan(M0, [[0]], [[1.0]], [[1]], [[1.0]], [[0.0, 0.0]], [1.0], [0.0],
               store=O.round_bf16)


# ---- planted mistakes (CPU): each must fail a pin above ----------------------------
def _truncating(x):
    x = np.asarray(x, np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    return np.ldexp(np.trunc(np.ldexp(x, 8 - e)), e - 8)


def _via_fp32(x):  # double rounding through binary32
    return _torch_bf16(np.asarray(x, np.float64).astype(np.float32))


def _half_away(x):
    x = np.asarray(x, np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    s = np.ldexp(x, 8 - e)
    return np.ldexp(np.sign(s) * np.floor(np.abs(s) + 0.5), e - 8)


def _scan_round_at_end(state0, idx_w, wt_w, idx_r, wt_r, v, alpha, beta, store=None):
    y, M = _orig_scan(state0, idx_w, wt_w, idx_r, wt_r, v, alpha, beta)
    return y, (store(M) if store is not None else M)


def _scan_round_twice(state0, idx_w, wt_w, idx_r, wt_r, v, alpha, beta, store=None):
    if store is None:
        return _orig_scan(state0, idx_w, wt_w, idx_r, wt_r, v, alpha, beta)
    M = np.array(state0, np.float64)
    y = np.zeros((len(idx_w), M.shape[1]))
    for t in range(len(idx_w)):
        rows = np.asarray(idx_w[t])
        mt = store(alpha[t] * M[rows])            # extra rounding of the forget-gated row
        M[rows] = store(mt + (beta[t] * np.asarray(wt_w[t]))[:, None] * (v[t] - mt))
        y[t] = np.asarray(wt_r[t]) @ M[np.asarray(idx_r[t])]
    return y, M


_orig_scan = O.scan
ROUND_PINS = (test_round_bf16_equals_torch_on_fp32_values, test_round_bf16_is_idempotent_and_monotone,
              test_round_bf16_equals_exact_rational_rounding,
              *[lambda x=x, w=w: test_round_bf16_hand_worked(x, w) for x, w in HALFWAY])
SCAN_PINS = (test_bf16_scan_one_token_is_one_rounding_of_the_exact_update,
             test_bf16_scan_state_is_representable_and_reads_see_it,
             test_bf16_scan_overwrite_stores_rounded_v_and_identity_keeps_state,
             test_bf16_scan_stays_near_the_exact_state)


@pytest.mark.parametrize("name,attr,fn,pins", [
    ("truncation", "round_bf16", _truncating, ROUND_PINS),
    ("double rounding via fp32", "round_bf16", _via_fp32, ROUND_PINS),
    ("ties away from zero", "round_bf16", _half_away, ROUND_PINS),
    ("rounded only at the end", "scan", _scan_round_at_end, SCAN_PINS),
    ("forget-gated row rounded too", "scan", _scan_round_twice, SCAN_PINS),
])
def test_pins_catch_bf16_mutant(name, attr, fn, pins, monkeypatch):
    monkeypatch.setattr(O, attr, fn)
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin caught mutant: {name}"
