"""Pins of the oracle's write-log quantisation (e4m3_encode / e4m3_decode,
quantize_rows / dequantize_rows).

The pages store the training checkpoints in fp8 or int4 for long fine-tuning
(section 八 of the m.163.com article; section "训练效率" of the
ai-paper-analysis.pages.dev summary) and name no format details; the reading taken
is OCP E4M3 and symmetric int4 with one absmax scale per logged row.  Pins: torch's
float32 -> float8_e4m3fn conversion on in-range values (an independent library
routine), hand-worked codes from the format's definition, the round trip of every
code, the int4 packing by hand, and the quantisation error bounds.
"""
import numpy as np
import pytest
import torch

from oracle import sdm_oracle as O


def test_e4m3_equals_torch_on_in_range_values():
    rng = np.random.default_rng(71)
    v = (rng.uniform(-448, 448, 300_000) * np.exp2(-rng.uniform(0, 22, 300_000))).astype(np.float32)
    v = np.concatenate([v, np.float32([0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -6, 1.0])])
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(v), want)


# hand-worked from the definition: code = sign | field << 3 | fraction, value
# 2^(field - 7) (1 + fraction / 8) for field > 0, fraction 2^-9 for field 0
E4M3 = [
    (1.0, 0x38), (-1.0, 0xB8), (448.0, 0x7E), (2.0 ** -6, 0x08), (2.0 ** -9, 0x01),
    (1.0 + 1 / 16, 0x38),        # tie between 1 and 1.125: even fraction 0
    (1.0 + 3 / 16, 0x3A),        # tie between 1.125 and 1.25: even fraction 2
    (1.5 * 2.0 ** -9, 0x02),     # subnormal tie: 2 steps
    (0.5 * 2.0 ** -9, 0x00),     # half the smallest step: 0
    (7 * 2.0 ** -9 + 2.0 ** -11, 0x07),
    (15.5 * 2.0 ** -10, 0x08),   # 2^-6 - 2^-11 rounds up to the smallest normal
    (449.0, 0x7E),               # saturates
]


@pytest.mark.parametrize("x,code", E4M3)
def test_e4m3_hand_worked(x, code):
    assert int(O.e4m3_encode(np.float32(x))) == code
    if x in (1.0, -1.0, 448.0, 2.0 ** -6, 2.0 ** -9):  # exactly representable
        assert O.e4m3_decode(np.uint8(code)) == x


def test_every_code_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)  # NaN excluded
    vals = O.e4m3_decode(codes)
    back = O.e4m3_encode(vals.astype(np.float32))
    zero = vals == 0
    assert np.array_equal(back[~zero], codes[~zero])
    assert np.all((back[zero] & 0x7F) == 0)
    assert np.all(np.diff(vals[:127]) > 0)  # positive codes are increasing


def test_int4_packing_by_hand():
    codes, amax = O.quantize_rows(np.float32([[1, -1, 7, -7]]), "int4")
    assert amax[0] == 7.0
    assert codes.tolist() == [[0xF1, 0x97]]  # nibbles 1, -1 (0xF), 7, -7 (0x9), low first
    assert np.array_equal(O.dequantize_rows(codes, amax, "int4"), np.float32([[1, -1, 7, -7]]))


def test_zero_rows_and_error_bounds():
    rng = np.random.default_rng(72)
    x = (rng.standard_normal((500, 64)) * rng.uniform(0.01, 10, (500, 1))).astype(np.float32)
    x[0] = 0.0
    for fmt, rel in (("fp8", 2.0 ** -4), ("int4", 1.0 / 14 + 1e-6)):
        c, a = O.quantize_rows(x, fmt)
        back = O.dequantize_rows(c, a, fmt)
        assert a[0] == 0 and np.all(back[0] == 0)
        err = np.abs(back - x)
        # int4: half a step of absmax / 7; fp8: a sixteenth of the element itself or
        # half the subnormal step of the row's scale
        if fmt == "int4":
            assert np.all(err <= rel * a[:, None] * (1 + 1e-6))
        else:
            assert np.all(err <= rel * np.abs(x) + a[:, None] / 448 * 2.0 ** -10 * (1 + 1e-6))
        assert np.allclose(np.max(np.abs(back), axis=1), a, rtol=1e-6)


_enc = O.e4m3_encode


def _truncating(v):
    v = np.asarray(v, np.float32)
    return _enc((np.sign(v) * (np.abs(v) * (1 - 2.0 ** -5))).astype(np.float32))


def _ties_away(v):
    v = np.asarray(v, np.float32)
    return _enc((v * np.float32(1 + 2.0 ** -12)).astype(np.float32))


@pytest.mark.parametrize("fn", [_truncating, _ties_away])
def test_pins_catch_e4m3_mutant(fn, monkeypatch):
    monkeypatch.setattr(O, "e4m3_encode", fn)
    failed = 0
    for pin in (test_e4m3_equals_torch_on_in_range_values, test_every_code_round_trips,
                *[lambda x=x, c=c: test_e4m3_hand_worked(x, c) for x, c in E4M3]):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1


def test_pins_catch_high_nibble_first(monkeypatch):
    orig = O.quantize_rows

    def swapped(rows, fmt):
        c, a = orig(rows, fmt)
        return (((c & 15) << 4) | (c >> 4)).astype(np.uint8) if fmt == "int4" else c, a

    monkeypatch.setattr(O, "quantize_rows", swapped)
    with pytest.raises(AssertionError):
        test_int4_packing_by_hand()
