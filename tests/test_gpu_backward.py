"""Training path (sdm_scan_train + sdm_scan_backward) against the oracle.

The backward runs on either schedule: the direct reverse walk (one workgroup per
memory) and the slot-owner stream schedule (the default from 256 tokens); every
parity case runs on both.

* The training forward equals sdm_scan with the direct schedule bit for bit (state,
  y, out), and its write log holds the rows each write replaced (oracle log within
  the fp32 tolerance).
* The backward, given the GPU's forward results, the log and random incoming
  gradients (of out and of the final state), matches the oracle's scan_backward
  run on the same values: every gradient within 1e-4 of its tensor's scale (fp32
  sums over up to T tokens against fp64), the initial state restored bit for bit,
  and the gradients bit-reproducible across runs (fixed summation order; on the
  stream schedule d_v is summed with LDS float atomics and is reproducible up to
  summation order only).
"""
import numpy as np
import pytest
import torch

from oracle import sdm_oracle as O
from sparse_memory_linear_sdm_amd import _lib, dims_for, ops, synth
from tests.gpu_util import (assert_close, host, layer_inputs, random_products, say,
                            strided_products, to_dev)

pytestmark = pytest.mark.gpu


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


def _close_to_scale(got, exp, what, rel=1e-4):
    got = np.asarray(got, np.float64)
    exp = np.asarray(exp, np.float64)
    scale = max(np.abs(exp).max(), 1e-30)
    err = np.abs(got - exp)
    bad = err > rel * (np.abs(exp) + scale)
    assert not bad.any(), (f"{what}: {bad.sum()} elements beyond {rel} of the scale {scale:.3e}; "
                           f"max err {err.max():.3e}")


SCHED = {"direct": _lib.SDM_FLAG_SCAN_DIRECT, "stream": _lib.SDM_FLAG_SCAN_STREAM,
         "two_phase": _lib.SDM_FLAG_SCAN_TWO_PHASE}


def _back_dims(d, sched):
    db = _lib.dims(**{k: getattr(d, k) for k in ("B", "T", "d_model", "H", "n", "W", "R", "d_v",
                                                  "in_dtype", "gate_act", "eps", "flags")})
    if sched is not None:
        db.flags |= SCHED[sched]
    return db


def _run(d, prod, gamma, m0, rng, walks, sched=None):
    """GPU forward + backward; oracle backward of the listed walks from the GPU's values."""
    B, T, H, N, dv = d.B, d.T, d.H, d.n * d.n, d.d_v
    db = _back_dims(d, sched)
    pd = {k: to_dev(v) for k, v in prod.items()}
    gam = to_dev(gamma) if gamma is not None else None
    state = to_dev(m0)
    out, y, log = ops.scan_train(d, pd, gam, state)
    torch.cuda.synchronize()
    st_T, y_h = host(state), host(y)
    fmt = ops.log_format(d)
    log_h = (host(log["rows"]) if fmt == "fp32" else
             O.dequantize_rows(host(log["rows"]), host(log["scale"]), fmt))
    d_out = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    d_st = (rng.standard_normal((B, H, N, dv)) * 0.1).astype(np.float32)
    dS = to_dev(d_st)
    g = ops.scan_backward(db, pd, gam, state, dS, y, log, to_dev(d_out))
    torch.cuda.synchronize()
    if fmt == "fp32":
        assert np.array_equal(host(state), m0), "initial state not restored bit for bit"
    gh = {k: host(v) for k, v in g.items() if v is not None}
    gamma_h = gamma if gamma is not None else np.ones((H, dv), np.float32)
    d_gamma = np.zeros((H, dv))
    for b in range(B):
        for h in range(H):
            sel = {k: prod[k][b, :, h] for k in ("idx_w", "wt_w", "idx_r", "wt_r", "v", "gate",
                                                  "alpha", "beta")}
            og, oM0, odM = O.scan_backward(st_T[b, h], log_h[b, :, h], sel["idx_w"], sel["wt_w"],
                                           sel["idx_r"], sel["wt_r"], sel["v"], sel["alpha"],
                                           sel["beta"], y_h[b, :, h], sel["gate"], gamma_h[h],
                                           d.eps, d_out[b, :, h], d_st[b, h])
            d_gamma[h] += og["d_gamma"]
            if (b, h) not in walks:
                continue
            # with a quantised log both sides restore the same decoded rows
            assert np.array_equal(oM0, host(state)[b, h]) if fmt != "fp32" else \
                np.array_equal(oM0, m0[b, h])
            for k in ("d_v", "d_gate", "d_alpha", "d_beta", "d_wt_w", "d_wt_r"):
                _close_to_scale(gh[k][b, :, h], og[k], f"{k} walk {(b, h)}")
            _close_to_scale(host(dS)[b, h], odM, f"d_state walk {(b, h)}")
    _close_to_scale(gh["d_norm_w"], d_gamma, "d_norm_w")
    return out, y, log, state, g, pd, gam, dS


CASES = [
    (1, 64, 1, 16, 8, 8, 16, "random"),
    (1, 300, 2, 12, 64, 128, 64, "repeat"),   # more than 64 ids per token
    (2, 120, 2, 8, 16, 16, 32, "repeat"),     # N = 64: slots rewritten and re-read constantly
    (2, 50, 3, 8, 32, 32, 64, "random"),
    (1, 40, 2, 12, 16, 8, 128, "same"),       # every token the same selection
    (1, 30, 1, 16, 64, 128, 256, "random"),
    (2, 17, 1, 4, 16, 16, 16, "random"),      # every slot written and read by every token
    # several stream rounds (256 tokens) with a ragged last one
    (1, 700, 2, 8, 16, 16, 32, "repeat"),
    (2, 300, 1, 16, 64, 64, 128, "random"),
    (1, 520, 1, 6, 16, 32, 16, "same"),
    (1, 260, 1, 12, 32, 16, 256, "repeat"),
    (1, 300, 1, 1024, 16, 16, 16, "random"),  # N = 1024^2: the largest slot bitmaps
]


@pytest.mark.parametrize("sched", ["direct", "stream"])
@pytest.mark.parametrize("B,T,H,n,W,R,d_v,mode", CASES)
def test_backward_matches_oracle(B, T, H, n, W, R, d_v, mode, sched):
    rng = np.random.default_rng(B * 1000 + T + W + R + d_v)
    prod = random_products(rng, B, T, H, n, W, R, d_v, mode)
    m0 = (rng.standard_normal((B, H, n * n, d_v)) * 0.3).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32)
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v)
    _run(d, prod, gamma, m0, rng, [(b, h) for b in range(B) for h in range(H)], sched)


@pytest.mark.parametrize("sched", ["direct", "stream", "two_phase"])
@pytest.mark.parametrize("T,d_v,W,R,n", [(80, 64, 16, 16, 0), (600, 32, 16, 16, 0),
                                         (300, 16, 16, 16, 0), (270, 256, 16, 16, 0),
                                         (300, 64, 64, 128, 0), (260, 32, 128, 32, 0),
                                         (280, 16, 16, 16, 1024)])  # n = 0: the default
def test_training_forward_equals_scan_and_log_is_the_replaced_rows(sched, T, d_v, W, R, n):
    """State and log equal the direct scan's bit for bit on every schedule (one owner
    applies each slot's writes in token order, the same arithmetic); y and out equal
    sdm_scan's on the direct schedule bit for bit, on the slot-owner ones up to fp32
    summation order; the log holds the oracle's replaced rows."""
    rng = np.random.default_rng(61 + T)
    B, H = 2, 2
    n = n or (10 if max(W, R) <= 64 else 12)
    prod = random_products(rng, B, T, H, n, W, R, d_v, "repeat")
    m0 = (rng.standard_normal((B, H, n * n, d_v)) * 0.3).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32)
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=SCHED[sched])
    pd = {k: to_dev(v) for k, v in prod.items()}
    st_a, st_b, st_c = to_dev(m0), to_dev(m0), to_dev(m0)
    out_a, y_a, log = ops.scan_train(d, pd, to_dev(gamma), st_a)
    dd = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=_lib.SDM_FLAG_SCAN_DIRECT)
    out_b, y_b = ops.scan(dd, pd, to_dev(gamma), st_b, with_y_raw=True)
    _, _, log_d = ops.scan_train(dd, pd, to_dev(gamma), st_c)
    torch.cuda.synchronize()
    assert torch.equal(st_a, st_b) and torch.equal(log["rows"], log_d["rows"])
    if sched == "direct":
        assert torch.equal(y_a, y_b) and torch.equal(out_a, out_b)
    else:
        assert_close(host(y_a), host(y_b), "y_raw")
        assert_close(host(out_a), host(out_b), "out")
    lh = host(log["rows"])
    for b in range(B):
        for h in range(H):
            _, _, olog = O.scan(m0[b, h], prod["idx_w"][b, :, h], prod["wt_w"][b, :, h],
                                prod["idx_r"][b, :, h], prod["wt_r"][b, :, h], prod["v"][b, :, h],
                                prod["alpha"][b, :, h], prod["beta"][b, :, h], record=True)
            assert_close(lh[b, :, h], olog, f"log walk {(b, h)}")


@pytest.mark.parametrize("fmt", ["fp32", "fp8", "int4"])
def test_training_forward_with_wide_slices(fmt):
    """32 walks of d_v = 128: the two-phase training forward runs 256-byte column
    slices (4 parts).  State and log equal the direct schedule's bit for bit (a
    quantised log: the same codes and scales); y and out up to fp32 summation order."""
    rng = np.random.default_rng(67)
    B, T, H, n, W, R, d_v = 8, 300, 4, 12, 32, 32, 128
    prod = random_products(rng, B, T, H, n, W, R, d_v, "repeat")
    m0 = (rng.standard_normal((B, H, n * n, d_v)) * 0.3).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32)
    lf = 0 if fmt == "fp32" else LOG_FLAGS[fmt]
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=SCHED["two_phase"] | lf)
    dd = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=_lib.SDM_FLAG_SCAN_DIRECT | lf)
    pd = {k: to_dev(v) for k, v in prod.items()}
    st_a, st_b = to_dev(m0), to_dev(m0)
    out_a, y_a, log_a = ops.scan_train(d, pd, to_dev(gamma), st_a)
    out_b, y_b, log_b = ops.scan_train(dd, pd, to_dev(gamma), st_b)
    torch.cuda.synchronize()
    assert torch.equal(st_a, st_b)
    assert torch.equal(log_a["rows"], log_b["rows"])
    if fmt != "fp32":
        assert torch.equal(log_a["scale"], log_b["scale"])
    assert_close(host(y_a), host(y_b), "y_raw")
    assert_close(host(out_a), host(out_b), "out")
    if fmt == "fp32":  # the log against the oracle's replaced rows, two walks
        lh = host(log_a["rows"])
        for b, h in ((0, 0), (B - 1, H - 1)):
            _, _, olog = O.scan(m0[b, h], prod["idx_w"][b, :, h], prod["wt_w"][b, :, h],
                                prod["idx_r"][b, :, h], prod["wt_r"][b, :, h], prod["v"][b, :, h],
                                prod["alpha"][b, :, h], prod["beta"][b, :, h], record=True)
            assert_close(lh[b, :, h], olog, f"log walk {(b, h)}")


@pytest.mark.parametrize("sched", ["direct", "stream"])
def test_backward_is_bit_reproducible_and_without_norm_weight(sched):
    rng = np.random.default_rng(62)
    B, T, H, n, W, R, d_v = 2, 300, 2, 8, 16, 16, 32
    prod = random_products(rng, B, T, H, n, W, R, d_v, "repeat")
    m0 = (rng.standard_normal((B, H, n * n, d_v)) * 0.3).astype(np.float32)
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v)
    out, y, log, state, g, pd, gam, dS = _run(d, prod, None, m0, rng, [(0, 0), (1, 1)], sched)
    db = _back_dims(d, sched)
    # the backward left M_0 in `state`: redo the forward to get M_T back, then run the
    # backward twice with the same incoming gradients
    state2 = state.clone()
    ops.scan_train(d, pd, None, state2)
    torch.cuda.synchronize()
    runs = []
    for _ in range(2):
        s_ = state2.clone()
        ds = torch.ones_like(s_) * 0.25
        dout = torch.full_like(y, 0.5)
        runs.append((ops.scan_backward(db, pd, None, s_, ds, y, log, dout), s_, ds))
    torch.cuda.synchronize()
    for k in runs[0][0]:
        if sched == "stream" and k == "d_v":
            assert_close(host(runs[0][0][k]), host(runs[1][0][k]), k)
        else:
            assert torch.equal(runs[0][0][k], runs[1][0][k]), k
    assert torch.equal(runs[0][1], runs[1][1]) and torch.equal(runs[0][2], runs[1][2])


@pytest.mark.parametrize("sched", ["direct", "stream"])
def test_bench_layer_shape_reduced_tokens(sched):
    """The 1.4B-like layer's N, W, R, d_v and H with 256 tokens per sequence, products
    from the GPU's own selection pass."""
    wl = synth.small("layer1p4b", B=2, T=256)
    h, dd = layer_inputs(wl, seed=5)
    dm = dims_for(wl)
    p = ops.select(dm, dd["x"], dd["w_proj"], dd["A"], dd["b_dt"])
    prod = {k: host(v) for k, v in p.items()}
    m0 = np.broadcast_to(h["m0"], (wl.B,) + h["m0"].shape).copy()
    rng = np.random.default_rng(63)
    _run(dm, prod, h["gamma"], m0, rng, [(0, 0), (wl.B - 1, wl.H - 1)], sched)


# ---- quantised write log (fp8 / int4) ----------------------------------------------
LOG_FLAGS = {"fp8": _lib.SDM_FLAG_LOG_FP8, "int4": _lib.SDM_FLAG_LOG_INT4}


@pytest.mark.parametrize("fmt", ["fp8", "int4"])
@pytest.mark.parametrize("T,d_v", [(70, 64), (300, 64), (520, 256), (260, 16)])
def test_quantised_log_codes_equal_the_oracle(fmt, T, d_v):
    """The same forward with an fp32 and a quantised log: identical state, y and out;
    the codes and scales equal the oracle's quantisation of the fp32 rows bit for bit
    (both decide the codes in fp32).  From 256 tokens both run the stream schedule,
    the quantised one staging fp32 rows in the workspace and encoding them after the
    walk."""
    rng = np.random.default_rng(64 + T)
    B, H, n, W, R = 2, 2, 10, 16, 16
    prod = random_products(rng, B, T, H, n, W, R, d_v, "repeat")
    m0 = (rng.standard_normal((B, H, n * n, d_v)) * 0.3).astype(np.float32)
    m0[0, 0, :5] = 0.0  # rows that log as all zeros
    pd = {k: to_dev(v) for k, v in prod.items()}
    d32 = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v)
    dq = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=LOG_FLAGS[fmt])
    st_a, st_b = to_dev(m0), to_dev(m0)
    out_a, y_a, log_a = ops.scan_train(d32, pd, None, st_a)
    out_b, y_b, log_b = ops.scan_train(dq, pd, None, st_b)
    torch.cuda.synchronize()
    assert torch.equal(st_a, st_b)
    if T < 256:
        assert torch.equal(y_a, y_b) and torch.equal(out_a, out_b)
    else:  # reads summed with LDS atomics: equal up to fp32 summation order
        assert_close(host(y_a), host(y_b), "y_raw")
        assert_close(host(out_a), host(out_b), "out")
    codes, amax = O.quantize_rows(host(log_a["rows"]), fmt)
    assert np.array_equal(host(log_b["scale"]), amax)
    assert np.array_equal(host(log_b["rows"]), codes)


@pytest.mark.parametrize("sched", ["direct", "stream"])
@pytest.mark.parametrize("fmt", ["fp8", "int4"])
@pytest.mark.parametrize("B,T,H,n,W,R,d_v,mode", [
    (2, 120, 2, 8, 16, 16, 32, "repeat"),
    (1, 30, 1, 16, 64, 128, 256, "random"),
    (1, 300, 2, 8, 16, 16, 64, "repeat"),
])
def test_backward_with_quantised_log(B, T, H, n, W, R, d_v, mode, fmt, sched):
    """Against the oracle's backward on the decoded rows; both restore the same
    decoded rows.  The distance to the fp32-log gradients is reported."""
    rng = np.random.default_rng(B * 100 + T + d_v)
    prod = random_products(rng, B, T, H, n, W, R, d_v, mode)
    m0 = (rng.standard_normal((B, H, n * n, d_v)) * 0.3).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32)
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=LOG_FLAGS[fmt])
    _, _, _, state, g, _, _, _ = _run(d, prod, gamma, m0, np.random.default_rng(7),
                                      [(b, h) for b in range(B) for h in range(H)], sched)
    d32 = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v)
    _, _, _, _, g32, _, _, _ = _run(d32, prod, gamma, m0, np.random.default_rng(7), [(0, 0)],
                                    sched)
    rel = {k: float((g[k] - g32[k]).abs().max() / g32[k].abs().max()) for k in ("d_v", "d_alpha")}
    drift = float(np.abs(host(state) - m0).max() / np.abs(m0).max())
    say(f"  {fmt} log: gradient distance to the fp32 log {rel}; restored state off by {drift:.2e}")


@pytest.mark.parametrize("fmt", ["fp32", "fp8", "int4"])
@pytest.mark.parametrize("B,T,H,n,W,R,d_v,mode", [
    (8, 260, 4, 8, 16, 16, 128, "repeat"),     # 32 walks: two 256-byte slices, 4 parts
    (16, 130, 4, 10, 16, 16, 64, "random"),    # 64 walks: one slice, 4 parts
])
def test_stream_backward_with_wide_slices(B, T, H, n, W, R, d_v, mode, fmt):
    """Walk counts at which the reverse walk takes 256-byte column slices (16-lane
    owner groups): every walk against the oracle, the state restored."""
    rng = np.random.default_rng(B * 10 + T + d_v)
    prod = random_products(rng, B, T, H, n, W, R, d_v, mode)
    m0 = (rng.standard_normal((B, H, n * n, d_v)) * 0.3).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32)
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=LOG_FLAGS.get(fmt, 0))
    _run(d, prod, gamma, m0, rng, [(b, h) for b in range(B) for h in range(H)], "stream")


def test_stream_backward_over_several_token_chunks():
    """A run long enough that the stream schedule splits it into token chunks (its
    per-token buffers are bounded near 2 GiB): sampled walks against the oracle,
    the initial state restored bit for bit, d_norm_w against the direct schedule."""
    B, T, H, n, W, R, d_v = 8, 66000, 4, 8, 16, 16, 16
    rng = np.random.default_rng(65)
    prod = strided_products(rng, B, T, H, n, W, R, d_v)
    m0 = (rng.standard_normal((B, H, n * n, d_v)) * 0.3).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32)
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v)
    pd = {k: to_dev(v) for k, v in prod.items()}
    gam = to_dev(gamma)
    state = to_dev(m0)
    _, y, log = ops.scan_train(d, pd, gam, state)
    d_out = to_dev(rng.standard_normal((B, T, H, d_v)).astype(np.float32))
    d_st = to_dev((rng.standard_normal((B, H, n * n, d_v)) * 0.1).astype(np.float32))
    st_T = state.clone()
    runs = {}
    for sched in ("stream", "direct"):
        s_, ds = st_T.clone(), d_st.clone()
        g = ops.scan_backward(_back_dims(d, sched), pd, gam, s_, ds, y, log, d_out)
        torch.cuda.synchronize()
        assert np.array_equal(host(s_), m0), f"{sched}: initial state not restored"
        runs[sched] = (g, ds)
    say(f"  stream workspace {_lib.workspace_bytes(_back_dims(d, 'stream'), _lib.SDM_ENTRY_SCAN_BACKWARD) / 2**30:.2f} GiB")
    g, ds = runs["stream"]
    for b, h in [(0, 0), (B - 1, H - 1)]:
        sel = {k: prod[k][b, :, h] for k in prod}
        og, _, odM = O.scan_backward(host(st_T[b, h]), host(log["rows"][b, :, h]), sel["idx_w"],
                                     sel["wt_w"], sel["idx_r"], sel["wt_r"], sel["v"],
                                     sel["alpha"], sel["beta"], host(y[b, :, h]), sel["gate"],
                                     gamma[h], d.eps, host(d_out[b, :, h]), host(d_st[b, h]))
        for k in ("d_v", "d_gate", "d_alpha", "d_beta", "d_wt_w", "d_wt_r"):
            _close_to_scale(host(g[k][b, :, h]), og[k], f"{k} walk {(b, h)}")
        _close_to_scale(host(ds[b, h]), odM, f"d_state walk {(b, h)}")
    _close_to_scale(host(g["d_norm_w"]), host(runs["direct"][0]["d_norm_w"]), "d_norm_w")


def test_quantised_log_over_several_token_chunks():
    """A quantised log on the stream schedule long enough to be staged in several token
    chunks (the staging area counts against the per-chunk bound): state equal to the
    fp32-log run, codes and scales of sampled walks equal to the oracle's quantisation
    of that run's fp32 rows."""
    B, T, H, n, W, R, d_v = 8, 80000, 4, 8, 16, 16, 16
    rng = np.random.default_rng(66)
    prod = strided_products(rng, B, T, H, n, W, R, d_v)
    m0 = (rng.standard_normal((B, H, n * n, d_v)) * 0.3).astype(np.float32)
    pd = {k: to_dev(v) for k, v in prod.items()}
    d32 = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v)
    dq = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=_lib.SDM_FLAG_LOG_FP8)
    nq = _lib.workspace_bytes(dq, _lib.SDM_ENTRY_SCAN_TRAIN)
    staged = B * T * H * W * d_v * 4
    # one chunk would hold at least the staged rows, the entries and one read partial
    # per token and walk
    assert nq < B * T * H * (W * d_v * 4 + (W + R) * 8 + d_v * 4), "expected token chunks"
    st_a, st_b = to_dev(m0), to_dev(m0)
    _, _, log_a = ops.scan_train(d32, pd, None, st_a)
    _, _, log_b = ops.scan_train(dq, pd, None, st_b)
    torch.cuda.synchronize()
    say(f"  workspace {nq / 2**30:.2f} GiB for {staged / 2**30:.2f} GiB of fp32 rows")
    assert torch.equal(st_a, st_b)
    for b, h in [(0, 0), (3, 2), (B - 1, H - 1)]:
        codes, amax = O.quantize_rows(host(log_a["rows"][b, :, h]), "fp8")
        assert np.array_equal(host(log_b["scale"][b, :, h]), amax), (b, h)
        assert np.array_equal(host(log_b["rows"][b, :, h]), codes), (b, h)


def test_training_at_the_full_bench_size():
    """The 1.4B-like layer at full size (8 x 4096 tokens, 4 heads, N = 131,044), products
    from the GPU's own selection, the default schedules (two-phase training forward,
    slot-owner backward): two complete walks against the oracle's reverse walk from
    the GPU's final state, log and y; M0 restored bit for bit for every walk."""
    wl = synth.WORKLOADS["layer1p4b"]
    h, dd = layer_inputs(wl, seed=11)
    dm = dims_for(wl)
    p = ops.select(dm, dd["x"], dd["w_proj"], dd["A"], dd["b_dt"])
    del dd["x"]
    gam = dd["gamma"]
    st = dd["m0"].unsqueeze(0).repeat(wl.B, 1, 1, 1)
    _, y, log = ops.scan_train(dm, p, gam, st)
    gen = torch.Generator(device=st.device).manual_seed(12)
    d_out = torch.randn(y.shape, device=st.device, generator=gen)
    d_st = torch.randn(st.shape, device=st.device, generator=gen) * 0.1
    walks = [(0, 0), (wl.B - 1, wl.H - 1)]
    keep = {(b, hh): (host(st[b, hh]), host(log["rows"][b, :, hh]), host(y[b, :, hh]),
                      host(d_out[b, :, hh]), host(d_st[b, hh])) for b, hh in walks}
    dS = d_st.clone()
    g = ops.scan_backward(dm, p, gam, st, dS, y, log, d_out)
    torch.cuda.synchronize()
    m0_h = host(dd["m0"])
    for b in range(wl.B):
        for hh in range(wl.H):
            assert torch.equal(st[b, hh], dd["m0"][hh]), f"M0 not restored for walk {(b, hh)}"
    for (b, hh), (mT, lg, yy, do, ds) in keep.items():
        sel = {k: host(p[k][b, :, hh]) for k in ("idx_w", "wt_w", "idx_r", "wt_r", "v", "gate",
                                                 "alpha", "beta")}
        og, oM0, odM = O.scan_backward(mT, lg, sel["idx_w"], sel["wt_w"], sel["idx_r"],
                                       sel["wt_r"], sel["v"], sel["alpha"], sel["beta"], yy,
                                       sel["gate"], h["gamma"][hh], wl.eps, do, ds)
        assert np.array_equal(oM0, m0_h[hh])
        for k in ("d_v", "d_gate", "d_alpha", "d_beta", "d_wt_w", "d_wt_r"):
            _close_to_scale(host(g[k][b, :, hh]), og[k], f"{k} walk {(b, hh)}")
        _close_to_scale(host(dS[b, hh]), odM, f"d_state walk {(b, hh)}")
