"""Shared initial state with copy on first touch (sdm_scan_shared_m0 and
sdm_forward_shared_m0) against the oracle's forward_walk_shared.

* The store starts as NaN and the bitmaps as zero: the effective state, the read
  vectors and the outputs match the oracle (fp32 tolerance), the bitmaps equal
  the oracle's touched sets bit for bit, and rows never touched still hold NaN
  (never written, and never read: a read would have put NaN into the outputs).
* The effective state equals the plain entry's state from a broadcast copy of M0
  bit for bit (the same kernels run on the same values), for every schedule, both
  write rules and the bf16 state.
* Two calls equal one; the decode workload's one-token steps from fresh bitmaps
  equal the plain decode steps from the broadcast copy.
"""
import numpy as np
import pytest
import torch

from sparse_memory_linear_sdm_amd import _lib, dims_for, ops, synth
from tests.gpu_util import (assert_close, broadcast_state, host, layer_inputs, oracle_walks,
                            random_products, say, to_dev)
from oracle import sdm_oracle as O

pytestmark = pytest.mark.gpu

SCHEDULES = {"direct": _lib.SDM_FLAG_SCAN_DIRECT, "stream": _lib.SDM_FLAG_SCAN_STREAM,
             "two_phase": _lib.SDM_FLAG_SCAN_TWO_PHASE, "chunk": _lib.SDM_FLAG_SCAN_CHUNK}


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"\n[gpu] {request.node.nodeid}")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    yield
    torch.cuda.synchronize()


def _dims(**kw):
    base = dict(B=1, T=64, d_model=64, H=1, n=16, W=8, R=8, d_v=16, in_dtype=_lib.SDM_DTYPE_F32,
                gate_act=_lib.SDM_GATE_SIGMOID, eps=1e-6)
    base.update(kw)
    return _lib.dims(**base)


def _bits(touched, N):
    """[B, H, words] int32 bitmaps -> [B, H, N] bool (bit i of word i/32)."""
    u8 = np.ascontiguousarray(host(touched)).view(np.uint8)
    return np.unpackbits(u8, axis=-1, bitorder="little")[..., :N].astype(bool)


def _effective(state, touched, m0):
    st = host(state.float()) if state.dtype == torch.bfloat16 else host(state)
    t = _bits(touched, m0.shape[1])
    return np.where(t[..., None], st, host(m0.float())[None]), t


@pytest.mark.parametrize("schedule", ["direct", "stream", "two_phase"])
@pytest.mark.parametrize("B,T,H,n,W,R,d_v,mode", [
    (2, 64, 2, 32, 8, 8, 32, "random"),        # most slots stay untouched
    (1, 300, 2, 16, 16, 32, 64, "repeat"),
    (2, 40, 1, 8, 32, 32, 128, "random"),      # every slot touched
])
def test_fresh_sequences_match_the_oracle(B, T, H, n, W, R, d_v, mode, schedule):
    rng = np.random.default_rng(B * 10 + T + W)
    N = n * n
    prod = random_products(rng, B, T, H, n, W, R, d_v, mode)
    m0 = (rng.standard_normal((H, N, d_v)) * 0.02).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32)
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=SCHEDULES[schedule])
    m0d = to_dev(m0)
    state = torch.full((B, H, N, d_v), float("nan"), device="cuda:0")
    touched = ops.alloc_touched(d, m0d.device)
    out, y = ops.scan_shared_m0(d, {k: to_dev(v) for k, v in prod.items()}, to_dev(gamma), m0d,
                                state, touched, with_y_raw=True)
    torch.cuda.synchronize()
    eff, tb = _effective(state, touched, m0d)
    st = host(state)
    for b in range(B):
        for h in range(H):
            sel = {k: prod[k][b, :, h] for k in ("idx_w", "wt_w", "idx_r", "wt_r", "v", "gate",
                                                  "alpha", "beta")}
            sel["g"] = sel.pop("gate")
            o_out, o_y, o_M, o_t = O.forward_walk_shared(m0[h], np.zeros((N, d_v)),
                                                         np.zeros(N, bool), sel, gamma[h], 1e-6)
            assert np.array_equal(tb[b, h], o_t), "touched bitmap"
            assert_close(eff[b, h], o_M, f"effective state {(b, h)}")
            assert_close(host(y)[b, :, h], o_y, f"y {(b, h)}")
            assert_close(host(out)[b, :, h], o_out, f"out {(b, h)}")
            assert np.all(np.isnan(st[b, h][~o_t])), "untouched rows were written"
            assert not np.isnan(st[b, h][o_t]).any()
    say(f"  touched {tb.mean():.3f} of the slots")


@pytest.mark.parametrize("schedule,flags", [
    ("direct", 0), ("stream", 0), ("two_phase", 0), ("direct", _lib.SDM_FLAG_DELTA_GDN),
    ("two_phase", _lib.SDM_FLAG_STATE_BF16), ("direct", _lib.SDM_FLAG_STATE_BF16 |
                                              _lib.SDM_FLAG_DELTA_GDN),
    ("chunk", 0), ("chunk", _lib.SDM_FLAG_DELTA_GDN)])
def test_equals_the_plain_entry_on_a_broadcast_copy(schedule, flags):
    rng = np.random.default_rng(5)
    B, T, H, n, W, R, d_v = 2, 200, 2, 20, 16, 16, 64
    N = n * n
    prod = {k: to_dev(v) for k, v in random_products(rng, B, T, H, n, W, R, d_v, "repeat").items()}
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=SCHEDULES[schedule] | flags)
    bf = bool(flags & _lib.SDM_FLAG_STATE_BF16)
    m0 = torch.from_numpy((rng.standard_normal((H, N, d_v)) * 0.02).astype(np.float32)).cuda()
    if bf:
        m0 = m0.to(torch.bfloat16)
    gamma = to_dev(rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32))
    plain = broadcast_state(m0, B)
    out_p, y_p = ops.scan(d, prod, gamma, plain, with_y_raw=True)
    store = torch.zeros_like(plain)
    touched = ops.alloc_touched(d, m0.device)
    out_s, y_s = ops.scan_shared_m0(d, prod, gamma, m0, store, touched, with_y_raw=True)
    torch.cuda.synchronize()
    t = torch.from_numpy(_bits(touched, N)).cuda()
    eff = torch.where(t[..., None], store, m0.unsqueeze(0))
    assert torch.equal(eff, plain)
    if schedule in ("direct", "chunk"):   # fixed summation order: identical reads
        assert torch.equal(y_s, y_p) and torch.equal(out_s, out_p)
    assert_close(host(y_s), host(y_p), "y", rtol=1e-5, atol=1e-6)
    assert_close(host(out_s), host(out_p), "out", rtol=1e-5, atol=1e-6)


def test_two_calls_equal_one():
    rng = np.random.default_rng(6)
    B, T, H, n, W, R, d_v = 2, 120, 2, 16, 8, 8, 32
    N = n * n
    p = random_products(rng, B, T, H, n, W, R, d_v, "random")
    m0 = to_dev((rng.standard_normal((H, N, d_v)) * 0.02).astype(np.float32))
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v)
    st1, t1 = torch.zeros((B, H, N, d_v), device="cuda:0"), ops.alloc_touched(d, m0.device)
    out1 = ops.scan_shared_m0(d, {k: to_dev(v) for k, v in p.items()}, None, m0, st1, t1)
    st2, t2 = torch.zeros_like(st1), ops.alloc_touched(d, m0.device)
    outs = []
    for a, b in ((0, 50), (50, T)):
        dd = _dims(B=B, T=b - a, H=H, n=n, W=W, R=R, d_v=d_v)
        outs.append(ops.scan_shared_m0(dd, {k: to_dev(np.ascontiguousarray(v[:, a:b]))
                                            for k, v in p.items()}, None, m0, st2, t2))
    torch.cuda.synchronize()
    assert torch.equal(t1, t2)
    e1, _ = _effective(st1, t1, m0)
    e2, _ = _effective(st2, t2, m0)
    assert np.array_equal(e1, e2)
    assert_close(host(torch.cat(outs, 1)), host(out1), "out", rtol=1e-5, atol=1e-6)


def test_decode_steps_from_fresh_bitmaps_equal_the_broadcast_copy():
    wl = synth.WORKLOADS["decode256"]
    h, d = layer_inputs(wl, seed=4)
    d1 = dims_for(wl, T=1)
    plain = broadcast_state(d["m0"], wl.B)
    store = torch.zeros_like(plain)
    touched = ops.alloc_touched(d1, plain.device)
    for t in range(6):
        xt = d["x"][:, t:t + 1].contiguous()
        o_p = ops.forward(d1, xt, d["w_proj"], d["A"], d["b_dt"], d["gamma"], plain)
        o_s = ops.forward_shared_m0(d1, xt, d["w_proj"], d["A"], d["b_dt"], d["gamma"], d["m0"],
                                    store, touched)
        torch.cuda.synchronize()
        assert torch.equal(o_p, o_s), f"step {t}"
    tb = torch.from_numpy(_bits(touched, wl.N)).cuda()
    for b0 in range(0, wl.B, 16):   # the states are 32 GiB each: compare in slabs
        sl = slice(b0, b0 + 16)
        eff = torch.where(tb[sl, ..., None], store[sl], d["m0"].unsqueeze(0))
        assert torch.equal(eff, plain[sl]), f"batch entries {b0}.."
    say(f"  touched {tb.float().mean().item():.4f} of the slots after 6 steps")
