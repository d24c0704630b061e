"""fp8 state storage (SDM_FLAG_STATE_FP8) against the oracle's fp8 walk.

The state is E4M3 codes with one power-of-two exponent per 32-column block of a row
(oracle round_fp8_blocks / fp8_state_encode, pinned in
tests/test_oracle_fp8_state_pins.py).  The kernels requantise each written row from
its fp32 update; the oracle rounds the exact update once.  So the stored states are
equal except where an exact value lies within fp32 error of an E4M3 rounding
boundary (or of a block exponent's boundary): such elements sit one code step
apart, and later writes carry the difference scaled by alpha (1 - c) <= 1.  The
tests therefore require the state equal but for a small fraction of elements, each
within two E4M3 spacings of the walk's scale; y within the fp32 bound, or that plus
two spacings for the tokens that read such an element; out through the norm's
Jacobian from those reads.  Writes of v with beta = 1 and weight 1 are exact, as
is a forget gate of 1 with beta = 0, and every schedule stores the same bytes.
"""
import numpy as np
import pytest
import torch

from oracle import sdm_oracle as O
from sparse_memory_linear_sdm_amd import _lib, dims_for, ops, synth
from tests.gpu_util import (assert_close, check_bf16_reads, check_bf16_state, fp8_spacing, host,
                            layer_inputs, oracle_walks, random_products, say, to_dev)
from tests.test_gpu_chunk import random_products_fast

pytestmark = pytest.mark.gpu

FP8 = _lib.SDM_FLAG_STATE_FP8
SCHEDULES = {"direct": _lib.SDM_FLAG_SCAN_DIRECT, "two_phase": _lib.SDM_FLAG_SCAN_TWO_PHASE}


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"\n[gpu] {request.node.nodeid}")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    yield
    torch.cuda.synchronize()


def _dims(**kw):
    base = dict(B=1, T=64, d_model=64, H=1, n=16, W=8, R=8, d_v=32, in_dtype=_lib.SDM_DTYPE_F32,
                gate_act=_lib.SDM_GATE_SIGMOID, eps=1e-6)
    base.update(kw)
    return _lib.dims(**base)


def _prod_dev(p):
    return {k: to_dev(v) for k, v in p.items()}


def _fp8_buffer(m):
    """Device state buffer (codes plane, then exponent plane) holding m exactly."""
    codes, exps = O.fp8_state_encode(m)
    return torch.from_numpy(np.concatenate([codes.ravel(), exps.ravel()])).cuda()


def _fp8_state(rng, shape, scale=0.3):
    m = O.round_fp8_blocks(rng.standard_normal(shape) * scale)
    return m, _fp8_buffer(m)


def _decode(d, buf, b=None, h=None):
    codes, exps = ops.fp8_state_planes(d, buf)
    if b is not None:
        codes, exps = codes[b, h], exps[b, h]
    return O.fp8_state_decode(host(codes), host(exps))


@pytest.mark.parametrize("schedule", ["direct", "two_phase"])
@pytest.mark.parametrize("B,T,H,n,W,R,d_v,mode", [
    (1, 64, 1, 32, 8, 8, 32, "random"),
    (1, 700, 2, 32, 16, 16, 32, "repeat"),     # several rounds of the two-phase schedule
    (2, 50, 2, 8, 32, 32, 64, "repeat"),       # heavy slot reuse
    (3, 33, 2, 20, 64, 64, 128, "repeat"),
    (1, 30, 1, 16, 128, 128, 256, "random"),
    (2, 300, 2, 16, 32, 128, 64, "random"),    # W = 32 / R = 128
    (8, 40, 4, 16, 16, 16, 128, "random"),     # 32 walks: 64-column slices
])
def test_fp8_state_matches_oracle(B, T, H, n, W, R, d_v, mode, schedule):
    rng = np.random.default_rng(B * 100 + T + W + 9)
    N = n * n
    prod = random_products(rng, B, T, H, n, W, R, d_v, mode)
    m0, state = _fp8_state(rng, (B, H, N, d_v))
    before = state.clone()
    gamma = rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32)
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=SCHEDULES[schedule] | FP8)
    out, y = ops.scan(d, _prod_dev(prod), to_dev(gamma), state, with_y_raw=True)
    torch.cuda.synchronize()
    st = _decode(d, state)
    oh, yh = host(out), host(y)
    walks = [(b, h) for b in range(B) for h in range(H)]
    ref = oracle_walks(prod, m0, gamma, 1e-6, walks, state="fp8")
    flips = late = 0
    c0, e0 = ops.fp8_state_planes(d, before)
    c1, e1 = ops.fp8_state_planes(d, state)
    for (b, h), (o_out, o_y, o_M) in ref.items():
        scale = max(np.abs(o_M).max(), np.abs(m0[b, h]).max())
        flips += check_bf16_state(st[b, h], o_M, scale, f"state walk {(b, h)}", fp8_spacing)
        late += check_bf16_reads(yh[b, :, h], o_y, oh[b, :, h], gamma[h], prod["gate"][b, :, h],
                                 1e-6, scale, R, f"walk {(b, h)}", fp8_spacing)
        untouched = torch.from_numpy(
            np.setdiff1d(np.arange(N), prod["idx_w"][b, :, h].ravel())).cuda()
        assert torch.equal(c1[b, h][untouched], c0[b, h][untouched]), "unwritten codes changed"
        assert torch.equal(e1[b, h][untouched], e0[b, h][untouched]), "unwritten exponents changed"
    say(f"  state elements one code step apart: {flips}; tokens with such reads: {late}")


@pytest.mark.parametrize("schedule", ["direct", "two_phase"])
def test_fp8_writes_of_v_are_exact(schedule):
    """beta = 1, weight 1: every written row holds v as the format stores it, codes
    and exponents bit for bit as the oracle encodes it (values with E4M3 ties and
    near-ties, wide magnitudes); alpha = 1, beta = 0 leaves the buffer unchanged."""
    rng = np.random.default_rng(8)
    B, T, H, n, d_v = 2, 40, 2, 8, 64
    prod = random_products(rng, B, T, H, n, 1, 1, d_v)
    frac = rng.integers(0, 8, (B, T, H, d_v))
    ties = (8 + frac + 0.5) / 8 * rng.choice([-1.0, 1.0], (B, T, H, d_v)) * \
        2.0 ** rng.integers(-20, 8, (B, T, H, d_v))
    v = np.where(rng.random((B, T, H, d_v)) < 0.5, ties, prod["v"] * 100).astype(np.float32)
    m0, st0 = _fp8_state(rng, (B, H, n * n, d_v))
    d = _dims(B=B, T=T, H=H, n=n, W=1, R=1, d_v=d_v, flags=SCHEDULES[schedule] | FP8)
    p1 = dict(prod, alpha=np.ones((B, T, H), np.float32), beta=np.zeros((B, T, H), np.float32))
    st = st0.clone()
    ops.scan(d, _prod_dev(p1), None, st)
    torch.cuda.synchronize()
    assert torch.equal(st, st0)
    p2 = dict(prod, v=v, beta=np.ones((B, T, H), np.float32),
              wt_w=np.ones((B, T, H, 1), np.float32), wt_r=np.ones((B, T, H, 1), np.float32),
              idx_r=prod["idx_w"].copy())
    st = st0.clone()
    _, y = ops.scan(d, _prod_dev(p2), None, st, with_y_raw=True)
    torch.cuda.synchronize()
    vq = O.round_fp8_blocks(v.astype(np.float64))
    assert np.array_equal(host(y).astype(np.float64), vq), "reads of v"
    # the exponent comes from the block's absmax before rounding (a rounded absmax can
    # fall onto 1.75 2^k, whose encoding would take the next exponent down)
    codes, exps = O.fp8_state_encode(v.astype(np.float64))
    c1, e1 = ops.fp8_state_planes(d, st)
    c1, e1 = host(c1), host(e1)
    for b in range(B):
        for h in range(H):
            last = {int(p2["idx_w"][b, t, h, 0]): t for t in range(T)}
            for s_, t in last.items():
                assert np.array_equal(c1[b, h, s_], codes[b, t, h]), (b, h, s_, t)
                assert np.array_equal(e1[b, h, s_], exps[b, t, h]), (b, h, s_, t)


def test_fp8_forward_matches_scan():
    """sdm_forward with an fp8 state: the scan of its products equals sdm_scan with
    the same flags bit for bit."""
    wl = synth.small("layer1p4b", B=2, T=160, d_model=256, n=40, W=16, R=16, d_v=32)
    h, dd = layer_inputs(wl, seed=3)
    d8 = dims_for(wl)
    d8.flags = FP8
    m0 = O.round_fp8_blocks(host(dd["m0"]).astype(np.float64))
    m0b = np.broadcast_to(m0, (wl.B,) + m0.shape)
    st_f = _fp8_buffer(m0b)
    out_f, p_f = ops.forward(d8, dd["x"], dd["w_proj"], dd["A"], dd["b_dt"], dd["gamma"], st_f,
                             debug=True)
    st_s = _fp8_buffer(m0b)
    out_s = ops.scan(d8, p_f, dd["gamma"], st_s)
    torch.cuda.synchronize()
    assert torch.equal(st_f, st_s)
    assert_close(host(out_f), host(out_s), "forward vs scan", rtol=1e-5, atol=1e-6)


def test_fp8_full_size():
    """The 1.4B-like shape (B=8, T=4096, H=4, N=131,044, W=R=64, d_v=128) from a zero
    state: two-phase and direct schedules store the same bytes; two walks against
    the oracle."""
    wl = synth.WORKLOADS["layer1p4b"]
    rng = np.random.default_rng(5)
    B, T, H, n, W, R, d_v = wl.B, wl.T, wl.H, wl.n, wl.W, wl.R, wl.d_v
    prod = random_products_fast(rng, B, T, H, n, W, R, d_v)
    gamma = rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32)
    pd = _prod_dev(prod)
    g = to_dev(gamma)
    dt = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=FP8)
    dd = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=FP8 | _lib.SDM_FLAG_SCAN_DIRECT)
    nbytes = ops.state_shape(dt)[0]
    st_t = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    st_d = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out_t, y_t = ops.scan(dt, pd, g, st_t, with_y_raw=True)
    ops.scan(dd, pd, g, st_d)
    torch.cuda.synchronize()
    assert torch.equal(st_t, st_d), "schedules stored different bytes"
    del st_d
    walks = [(0, 0), (B - 1, H - 1)]
    m0 = np.zeros((H, n * n, d_v))
    ref = oracle_walks(prod, m0, gamma, 1e-6, walks, state="fp8")
    yh, oh = host(y_t), host(out_t)
    for (b, h), (o_out, o_y, o_M) in ref.items():
        st = _decode(dt, st_t, b, h)
        scale = np.abs(o_M).max()
        f = check_bf16_state(st, o_M, scale, f"state walk {(b, h)}", fp8_spacing)
        late = check_bf16_reads(yh[b, :, h], o_y, oh[b, :, h], gamma[h], prod["gate"][b, :, h],
                                1e-6, scale, R, f"walk {(b, h)}", fp8_spacing)
        say(f"  walk {(b, h)}: {f} elements one code step apart, {late} tokens read them")
