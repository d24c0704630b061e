"""Pins of the oracle's fp8 state storage (fp8_block_exponent, round_e4m3,
round_fp8_blocks, fp8_state_encode / fp8_state_decode, scan(..., store=...)).

The format: 32-column blocks of a row, each with one power-of-two scale 2^e, the
least e >= -127 with absmax <= 448 2^e, and OCP E4M3 elements (3 fraction bits,
exponents -6..8, subnormals spaced 2^-9, largest 448), each the nearest E4M3 value
of x 2^-e, ties to the even significand.  The pages keep the live state in full
precision and quantise only training checkpoints (section "训练效率" of the
ai-paper-analysis.pages.dev summary; section 八 of the m.163.com article), so the
pins come from the format's definition, an independent library conversion
(torch's float32 -> float8_e4m3fn, round-to-nearest-even), a hand-worked block and
closed forms.  Planted mistakes in the format must fail them.
"""
import inspect

import numpy as np
import pytest
import torch

from oracle import sdm_oracle as O


def _torch_e4m3(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def _e4m3_values():
    """Every finite non-negative E4M3 value, from the bit layout."""
    v = [f * 2.0 ** -9 for f in range(8)]
    v += [(8 + f) * 2.0 ** (E - 10) for E in range(1, 16) for f in range(8)]
    return np.array([x for x in v if x <= 448.0])


def _fp32_cases(rng):
    vals = _e4m3_values()
    mids = (vals[:-1] + vals[1:]) / 2                    # ties: nearest even wins
    x = np.concatenate([vals, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                        np.nextafter(mids.astype(np.float32), np.float32(1e9)),
                        rng.uniform(0, 448, 4000), np.exp(rng.uniform(-16, 6, 4000))])
    x = x[np.abs(x) <= 448].astype(np.float32)
    return np.concatenate([x, -x]).astype(np.float64)   # fp32-representable


def check_round_e4m3(fn=None):
    fn = fn or O.round_e4m3
    x = _fp32_cases(np.random.default_rng(0))
    assert np.array_equal(fn(x), _torch_e4m3(x)), "E4M3 rounding differs from torch's"


def check_block_exponent(fn=None):
    fn = fn or O.fp8_block_exponent
    j = np.arange(-120, 120)
    assert np.array_equal(fn(448.0 * 2.0 ** j), j)                    # on the boundary
    assert np.array_equal(fn(np.nextafter(448.0 * 2.0 ** j, np.inf)), j + 1)
    assert np.array_equal(fn(2.0 ** j), np.maximum(j - 8, -127))     # 2^j <= 1.75 2^j
    assert fn(0.0) == -127 and fn(2.0 ** -140) == -127                # clamped
    a = np.exp(np.random.default_rng(1).uniform(-80, 80, 5000))
    e = fn(a)                                                         # the least such e
    assert np.all(a <= 448.0 * 2.0 ** e)
    assert np.all((e == -127) | (a > 448.0 * 2.0 ** (e - 1)))


# a hand-worked row of 64 columns: two blocks
#  block 0: absmax 3.0 -> e = -7 (448 2^-7 = 3.5 >= 3 > 1.75), s = 120;
#           3.0 2^7 = 384 = 1.5 2^8        -> code 0x7C (field 15, fraction 4)
#           0.1 2^7 = 12.8 -> 13 = 1.625 2^3 -> code 0x55, value 13/128
#           -0.01 2^7 = -1.28 -> -1.25 (step 1/8 in [1, 2)) -> code 0xBA, value -1.25/128
#           5e-4 2^7 = 0.064 -> 0.0625 = 2^-4 (step 1/64 in [2^-4, 2^-3)) -> code 0x18
#           1e-5 2^7 = 0.00128: subnormal, 0.00128 512 = 0.655 -> 1 step of 2^-9 -> code
#           0x01, value 2^-16 (a block of its own would keep it normal: 9.54e-6)
#           the rest 0
#  block 1: absmax 448 exactly -> e = 0, s = 127: 448 -> 0x7E; -2.5 -> 0xC2 (1.25 2^1);
#           0.0015 -> subnormal 0.0015 512 = 0.768 -> 1 -> code 0x01 (2^-9)
def _hand_row():
    x = np.zeros(64)
    x[0], x[1], x[2], x[3], x[20] = 3.0, 0.1, -0.01, 5e-4, 1e-5
    x[32], x[33], x[34] = 448.0, -2.5, 0.0015
    codes = np.zeros(64, np.uint8)
    codes[0], codes[1], codes[2], codes[3], codes[20] = 0x7C, 0x55, 0xBA, 0x18, 0x01
    codes[32], codes[33], codes[34] = 0x7E, 0xC2, 0x01
    vals = np.zeros(64)
    vals[0], vals[1], vals[2], vals[3] = 3.0, 13 / 128, -1.25 / 128, 2.0 ** -4 / 128
    vals[20] = 2.0 ** -16
    vals[32], vals[33], vals[34] = 448.0, -2.5, 2.0 ** -9
    return x, codes, np.array([120, 127], np.uint8), vals


def check_hand_row(rnd=None, enc=None):
    rnd = rnd or O.round_fp8_blocks
    enc = enc or O.fp8_state_encode
    x, codes, exps, vals = _hand_row()
    assert np.array_equal(rnd(x), vals)
    c, e = enc(x)
    assert np.array_equal(c, codes) and np.array_equal(e, exps)
    assert np.array_equal(O.fp8_state_decode(codes, exps), vals)


def check_block_properties(rnd=None):
    rnd = rnd or O.round_fp8_blocks
    rng = np.random.default_rng(2)
    x = rng.standard_normal((40, 128)) * np.exp(rng.uniform(-30, 30, (40, 1)))
    q = rnd(x)
    assert np.array_equal(rnd(q), q)                                  # stored values stay
    assert np.array_equal(rnd(-x), -q)
    assert np.array_equal(rnd(x * 2.0 ** 17), q * 2.0 ** 17)          # scale-free
    blk = x.reshape(40, 4, 32)
    e = O.fp8_block_exponent(np.abs(blk).max(-1))[..., None]
    a = np.abs(blk) * 2.0 ** -e
    half = np.where(a >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 4),
                    2.0 ** -10)
    assert np.all(np.abs(q.reshape(40, 4, 32) - blk) * 2.0 ** -e <= half)   # half a step
    y = x.copy()
    y[:, 40:50] *= 1e6                                                # blocks independent
    qy = rnd(y)
    assert np.array_equal(qy[:, :32], q[:, :32]) and np.array_equal(qy[:, 64:], q[:, 64:])


def check_round_trip(rnd=None, enc=None):
    rnd = rnd or O.round_fp8_blocks
    enc = enc or O.fp8_state_encode
    x = np.random.default_rng(3).standard_normal((16, 96)) * 0.05
    c, e = enc(x)
    assert c.shape == (16, 96) and e.shape == (16, 3)
    assert np.array_equal(O.fp8_state_decode(c, e), rnd(x))


def test_round_e4m3_equals_torch_float8():
    check_round_e4m3()


def test_block_exponent_is_the_least_sufficient_power():
    check_block_exponent()


def test_hand_worked_row():
    check_hand_row()


def test_block_rounding_properties():
    check_block_properties()


def test_encode_decode_round_trip():
    check_round_trip()


def test_scan_with_fp8_store_special_cases():
    rng = np.random.default_rng(4)
    N, d_v, T = 8, 64, 6
    m0 = O.round_fp8_blocks(rng.standard_normal((N, d_v)))
    iw = np.array([[t % N] for t in range(T)])
    ones = np.ones((T, 1))
    v = rng.standard_normal((T, d_v)) * 5
    # beta = 1, one slot of weight 1: the written row holds v as stored
    _, M = O.scan(m0, iw, ones, iw, ones, v, np.full(T, 0.7), np.ones(T), store=O.round_fp8_blocks)
    assert np.array_equal(M[:T], O.round_fp8_blocks(v))
    # alpha = 1, beta = 0: every write leaves the stored row as it was
    _, M = O.scan(m0, iw, ones, iw, ones, v, np.ones(T), np.zeros(T), store=O.round_fp8_blocks)
    assert np.array_equal(M, m0)
    with pytest.raises(AssertionError):   # a state the format cannot hold is refused
        O.scan(rng.standard_normal((N, d_v)), iw, ones, iw, ones, v, np.ones(T), np.zeros(T),
               store=O.round_fp8_blocks)


# ---- planted mistakes (CPU): each must fail a pin -------------------------------------
def _mutant(fn, old, new):
    src = inspect.getsource(fn)
    assert src.count(old) == 1, old
    ns = dict(O.__dict__)
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns[fn.__name__], ns


MUTANTS = {
    "exponent one too small (saturates)": (O.fp8_block_exponent, "(2.0 * m > 1.75)", "0"),
    "exponent from 2^8, not 448": (O.fp8_block_exponent, "(2.0 * m > 1.75)", "(2.0 * m > 1.0)"),
    "rounding toward zero": (O.round_e4m3, "np.rint(a / step)", "np.floor(a / step)"),
    "no subnormal floor": (O.round_e4m3, "np.maximum(k - 1, -6)", "(k - 1)"),
    "four fraction bits": (O.round_e4m3, "- 3)", "- 4)"),
    "blocks of 16": (O.round_fp8_blocks, "x.shape[-1] // FP8_BLOCK, FP8_BLOCK", "x.shape[-1] // 16, 16"),
    "block scale from the mean": (O.round_fp8_blocks, "np.max(np.abs(blk), axis=-1)",
                                  "np.mean(np.abs(blk), axis=-1) * 4"),
}


def _run_pins(name):
    fn, old, new = MUTANTS[name]
    mut, ns = _mutant(fn, old, new)
    if fn is O.fp8_block_exponent:
        check_block_exponent(mut)
        return
    if fn is O.round_e4m3:
        check_round_e4m3(mut)
        return
    check_hand_row(rnd=mut)
    check_block_properties(mut)


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_mutant(name):
    with pytest.raises(AssertionError):
        _run_pins(name)
