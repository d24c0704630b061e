"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Stage A  projection + gates          vs oracle pass_a (fp32-accumulation bound)
Stage B  selection from half-scores  ids bit-identical, weights within tolerance
Stage C  scan from given selections  state / y / out within 1e-4 rel, 1e-5 abs;
                                     never-written rows bit-identical
Stage D  whole layer from x          ids equal except near-ties / GEMM-rounding flips
                                     (reported, not failed); outputs within tolerance
bf16 state storage (SDM_FLAG_STATE_BF16) against the oracle's bf16 scan: stored
values equal except rare one-spacing rounding-boundary cases (bound derived in
tests/gpu_util.py); the hardware rounding checked bit-exactly against torch's
float32 -> bfloat16 conversion through exact overwrites.
"""
import numpy as np
import pytest
import torch

from oracle import sdm_oracle as O
from sparse_memory_linear_sdm_amd import _lib, dims_for, ops, synth
from tests.gpu_util import (ATOL, NEAR_TIE, RTOL, assert_close, broadcast_state, check_bf16_reads,
                            check_bf16_state, gemm_bound, host, layer_inputs, oracle_walks,
                            random_products, say, strided_products, to_dev)

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


def _prod_dev(p):
    return {k: to_dev(v) for k, v in p.items()}


# ---------------------------------------------------------------------------
# Stage A
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("wl", [
    synth.WORKLOADS["tiny"],
    synth.small("layer1p4b", B=2, T=160, d_model=256, n=40, W=16, R=16, d_v=32),
    synth.small("layer1p4b", B=1, T=200, d_model=2048, H=2, n=362, W=64, R=64, d_v=128),
])
def test_stage_a_projection_and_gates(wl):
    h, d = layer_inputs(wl, seed=1, with_state=False)
    dm = dims_for(wl)
    p = ops.select(dm, d["x"], d["w_proj"], d["A"], d["b_dt"], with_scores=True)
    torch.cuda.synchronize()
    a = O.pass_a(h["x"], h["w_proj"], h["A"], h["b_dt"], wl.H, wl.n, wl.d_v, wl.W, wl.R)
    x2 = h["x"].reshape(-1, wl.d_model)
    bound = gemm_bound(x2, h["w_proj"], wl.d_model).reshape(wl.B, wl.T, wl.H, wl.P)
    sc = host(p["scores"]).astype(np.float64)
    err = np.abs(sc - a["scores"])
    assert np.all(err <= bound[..., :4 * wl.n]), f"scores max err {err.max()}"
    o4 = 4 * wl.n
    errv = np.abs(host(p["v"]) - a["v"])
    assert np.all(errv <= bound[..., o4:o4 + wl.d_v]), f"v max err {errv.max()}"
    assert_close(host(p["gate"]), a["g"], "gate")
    assert_close(host(p["alpha"]), a["alpha"], "alpha")
    assert_close(host(p["beta"]), a["beta"], "beta")
    say(f"  scores max |err| {err.max():.3e}  (bound min {bound[..., :o4].min():.3e})")


# ---------------------------------------------------------------------------
# Stage B
# ---------------------------------------------------------------------------
def _scores_case(rng, B, T, H, n, kind):
    shp = (B, T, H, 4 * n)
    if kind == "normal":
        return rng.standard_normal(shp).astype(np.float32)
    if kind == "ties":        # few levels: many exact ties across the cut
        return (rng.integers(-3, 4, shp) * 0.25).astype(np.float32)
    if kind == "zeros":       # signed zeros and equal scores everywhere
        s = np.zeros(shp, np.float32)
        s[rng.random(shp) < 0.5] = -0.0
        return s
    if kind == "wide":        # magnitudes across many binades
        return (rng.standard_normal(shp) * np.exp2(rng.integers(-30, 30, shp))).astype(np.float32)
    if kind == "flat_half":   # each role's first half constant, its second half not
        s = rng.standard_normal(shp).astype(np.float32)
        s[..., 0:n] = 1.25
        s[..., 2 * n:3 * n] = -0.5
        return s
    raise ValueError(kind)


@pytest.mark.parametrize("n,W,R,kind", [
    (32, 8, 8, "normal"), (362, 64, 64, "normal"), (362, 64, 64, "ties"),
    (40, 128, 100, "normal"), (40, 128, 128, "ties"), (8, 64, 20, "normal"),
    (4, 16, 16, "normal"), (16, 1, 1, "ties"), (16, 8, 8, "zeros"), (64, 64, 64, "wide"),
    (1024, 64, 64, "normal"), (1000, 33, 65, "ties"), (1, 1, 1, "normal"),
    (362, 64, 64, "zeros"), (362, 64, 64, "flat_half"), (40, 128, 100, "flat_half"),
    (1024, 64, 64, "zeros"),
])
def test_stage_b_selection_bit_exact(n, W, R, kind):
    rng = np.random.default_rng(n * 1000 + W + R)
    B, T, H = 2, 24, 3
    s = _scores_case(rng, B, T, H, n, kind)
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=R)
    g = ops.select_from_scores(d, to_dev(s))
    torch.cuda.synchronize()
    o = O.select_from_scores(s, n, W, R)
    for role, cnt in (("w", W), ("r", R)):
        gi = host(g[f"idx_{role}"])
        assert gi.shape == o[f"idx_{role}"].shape
        mism = np.argwhere(gi != o[f"idx_{role}"])
        assert mism.size == 0, f"ids differ ({role}) at {mism[:3].tolist()}"
        assert_close(host(g[f"wt_{role}"]), o[f"wt_{role}"], f"wt_{role}")


# ---------------------------------------------------------------------------
# Stage C
# ---------------------------------------------------------------------------
SCHEDULES = {"direct": _lib.SDM_FLAG_SCAN_DIRECT, "stream": _lib.SDM_FLAG_SCAN_STREAM,
             "two_phase": _lib.SDM_FLAG_SCAN_TWO_PHASE}


@pytest.mark.parametrize("schedule", ["direct", "stream", "two_phase"])
@pytest.mark.parametrize("B,T,H,n,W,R,d_v,mode", [
    (1, 64, 1, 32, 8, 8, 16, "random"),
    (1, 700, 2, 32, 16, 16, 32, "repeat"),     # several rounds of the stream schedule
    (2, 50, 3, 8, 32, 32, 32, "random"),       # N = 64, W = R = 32: heavy slot reuse
    (2, 50, 2, 8, 32, 32, 64, "repeat"),
    (1, 40, 2, 8, 16, 8, 128, "same"),
    (3, 33, 2, 20, 64, 64, 128, "repeat"),
    (1, 30, 1, 16, 128, 128, 256, "random"),
    (2, 17, 1, 4, 16, 16, 16, "random"),       # every slot written by every token
    (2, 300, 2, 16, 32, 128, 64, "random"),    # the pages' W = 32 / R = 128 ablation shape
])
def test_stage_c_scan(B, T, H, n, W, R, d_v, mode, schedule):
    rng = np.random.default_rng(B * 100 + T + W)
    N = n * n
    prod = random_products(rng, B, T, H, n, W, R, d_v, mode)
    m0 = (rng.standard_normal((B, H, N, d_v)) * 0.02).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32)
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=SCHEDULES[schedule])
    state = to_dev(m0)
    out, y = ops.scan(d, _prod_dev(prod), to_dev(gamma), state, with_y_raw=True)
    torch.cuda.synchronize()
    st, oh, yh = host(state), host(out), host(y)
    ref = oracle_walks(prod, m0, gamma, 1e-6, [(b, h) for b in range(B) for h in range(H)])
    for (b, h), (o_out, o_y, o_M) in ref.items():
        assert_close(yh[b, :, h], o_y, f"y_raw walk {(b, h)}")
        assert_close(oh[b, :, h], o_out, f"out walk {(b, h)}")
        assert_close(st[b, h], o_M, f"state walk {(b, h)}")
        untouched = np.setdiff1d(np.arange(N), prod["idx_w"][b, :, h].ravel())
        assert np.array_equal(st[b, h][untouched], m0[b, h][untouched]), "unwritten rows changed"


# Enough walks that the two-phase plan takes 256-byte column slices (64 floats per
# slice, at most 4 parts): 16-lane owner groups, several rounds, ragged tails.
@pytest.mark.parametrize("state_dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("B,T,H,n,W,R,d_v,mode", [
    (16, 300, 4, 16, 16, 16, 64, "random"),    # 64 walks, one slice, 4 parts
    (8, 520, 4, 24, 32, 32, 128, "repeat"),    # 32 walks, two slices, 4 parts
    (4, 100, 4, 12, 16, 48, 256, "random"),    # 16 walks, four slices, 4 parts
    (8, 270, 8, 8, 32, 32, 128, "repeat"),     # 64 walks, two slices, 2 parts; N = 64
    (16, 270, 4, 4, 1, 1, 64, "random"),       # W = R = 1 (most lanes idle), N = 16
    (8, 260, 4, 12, 64, 128, 128, "repeat"),   # R > 64: two id chunks per token when bucketing
])
def test_stage_c_scan_wide_slices(B, T, H, n, W, R, d_v, mode, state_dtype):
    rng = np.random.default_rng(B * 100 + T + W + 3)
    N = n * n
    prod = random_products(rng, B, T, H, n, W, R, d_v, mode)
    gamma = rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32)
    flags = SCHEDULES["two_phase"]
    if state_dtype == "bf16":
        m0, state = _bf16_state(rng, (B, H, N, d_v))
        flags |= _lib.SDM_FLAG_STATE_BF16
    else:
        m0 = (rng.standard_normal((B, H, N, d_v)) * 0.02).astype(np.float32)
        state = to_dev(m0)
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=flags)
    out, y = ops.scan(d, _prod_dev(prod), to_dev(gamma), state, with_y_raw=True)
    # the direct schedule on the same inputs: the same state bit for bit
    st_d = to_dev(m0) if state_dtype == "fp32" else to_dev(m0).to(torch.bfloat16)
    dd = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v,
               flags=(flags & ~SCHEDULES["two_phase"]) | _lib.SDM_FLAG_SCAN_DIRECT)
    out_d, _ = ops.scan(dd, _prod_dev(prod), to_dev(gamma), st_d, with_y_raw=True)
    torch.cuda.synchronize()
    assert torch.equal(state, st_d), "two-phase state differs from the direct schedule's"
    walks = [(b, h) for b in range(B) for h in range(H)]
    oh, yh = host(out), host(y)
    if state_dtype == "bf16":
        st = state.to(torch.float64).cpu().numpy()
        ref = oracle_walks(prod, m0, gamma, 1e-6, walks, state="bf16")
        for (b, h), (o_out, o_y, o_M) in ref.items():
            scale = max(np.abs(o_M).max(), np.abs(m0[b, h]).max())
            check_bf16_state(st[b, h], o_M, scale, f"state walk {(b, h)}")
            check_bf16_reads(yh[b, :, h], o_y, oh[b, :, h], gamma[h], prod["gate"][b, :, h],
                             1e-6, scale, R, f"walk {(b, h)}")
        return
    st = host(state)
    ref = oracle_walks(prod, m0, gamma, 1e-6, walks)
    for (b, h), (o_out, o_y, o_M) in ref.items():
        assert_close(yh[b, :, h], o_y, f"y_raw walk {(b, h)}")
        assert_close(oh[b, :, h], o_out, f"out walk {(b, h)}")
        assert_close(st[b, h], o_M, f"state walk {(b, h)}")
    assert_close(oh, host(out_d), "out against the direct schedule")


@pytest.mark.parametrize("B,T,H,n,W,R,d_v,mode", [
    (2, 64, 2, 8, 64, 64, 32, "random"),       # every slot selected (the GDN-reduction shape)
    (1, 300, 2, 16, 32, 128, 64, "random"),    # W = 32 / R = 128
    (2, 50, 1, 12, 16, 16, 256, "repeat"),
    (1, 40, 1, 32, 8, 8, 16, "same"),
])
def test_stage_c_gdn_variant(B, T, H, n, W, R, d_v, mode):
    """SDM_FLAG_DELTA_GDN: key-weighted error term, against the oracle's scan_gdn."""
    rng = np.random.default_rng(B * 1000 + T + W + R)
    N = n * n
    prod = random_products(rng, B, T, H, n, W, R, d_v, mode)
    m0 = (rng.standard_normal((B, H, N, d_v)) * 0.02).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32)
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=_lib.SDM_FLAG_DELTA_GDN)
    state = to_dev(m0)
    out, y = ops.scan(d, _prod_dev(prod), to_dev(gamma), state, with_y_raw=True)
    torch.cuda.synchronize()
    st, oh, yh = host(state), host(out), host(y)
    walks = [(b, h) for b in range(B) for h in range(H)]
    ref = oracle_walks(prod, m0, gamma, 1e-6, walks, rule="gdn")
    slot = oracle_walks(prod, m0, gamma, 1e-6, walks[:1], rule="slot")
    for (b, h), (o_out, o_y, o_M) in ref.items():
        assert_close(yh[b, :, h], o_y, f"y_raw walk {(b, h)}")
        assert_close(oh[b, :, h], o_out, f"out walk {(b, h)}")
        assert_close(st[b, h], o_M, f"state walk {(b, h)}")
        untouched = np.setdiff1d(np.arange(N), prod["idx_w"][b, :, h].ravel())
        assert np.array_equal(st[b, h][untouched], m0[b, h][untouched]), "unwritten rows changed"
    if W > 1:  # the two rules really differ on these inputs
        b, h = walks[0]
        assert np.max(np.abs(slot[(b, h)][2] - ref[(b, h)][2])) > 1e-6


@pytest.mark.parametrize("flags", [0, _lib.SDM_FLAG_DELTA_GDN, _lib.SDM_FLAG_STATE_BF16,
                                   _lib.SDM_FLAG_DELTA_GDN | _lib.SDM_FLAG_STATE_BF16])
def test_direct_schedule_is_deterministic(flags):
    """The direct schedule sums in a fixed order (no atomics): repeated runs agree bit
    for bit in state, y and out -- which also shows the LDS partial sums of one
    token are never overwritten by the next token's before they are read."""
    rng = np.random.default_rng(9)
    B, T, H, n, W, R, d_v = 2, 200, 2, 20, 16, 16, 64
    prod = _prod_dev(random_products(rng, B, T, H, n, W, R, d_v, "repeat"))
    m0 = torch.from_numpy((rng.standard_normal((B, H, n * n, d_v)) * 0.02).astype(np.float32))
    m0 = m0.to(torch.bfloat16 if flags & _lib.SDM_FLAG_STATE_BF16 else torch.float32).cuda()
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=_lib.SDM_FLAG_SCAN_DIRECT | flags)
    runs = []
    for _ in range(3):
        st = m0.clone()
        out, y = ops.scan(d, prod, None, st, with_y_raw=True)
        runs.append((st, out, y))
    torch.cuda.synchronize()
    for st, out, y in runs[1:]:
        assert torch.equal(st, runs[0][0]) and torch.equal(y, runs[0][2])
        assert torch.equal(out, runs[0][1])


@pytest.mark.parametrize("schedule", ["direct", "stream", "two_phase"])
def test_stage_c_identity_and_overwrite_exact(schedule):
    rng = np.random.default_rng(7)
    B, T, H, n, d_v = 2, 20, 2, 8, 32
    prod = random_products(rng, B, T, H, n, 1, 1, d_v)
    m0 = (rng.standard_normal((B, H, n * n, d_v)) * 0.02).astype(np.float32)
    d = _dims(B=B, T=T, H=H, n=n, W=1, R=1, d_v=d_v, flags=SCHEDULES[schedule])
    # alpha = 1, beta = 0: the state must come back bit-identical
    p1 = dict(prod, alpha=np.ones((B, T, H), np.float32), beta=np.zeros((B, T, H), np.float32))
    st = to_dev(m0)
    ops.scan(d, _prod_dev(p1), None, st)
    assert np.array_equal(host(st), m0)
    # beta = 1 with weight 1: each written slot holds exactly v_t; reading it returns v_t
    p2 = dict(prod, beta=np.ones((B, T, H), np.float32), wt_w=np.ones((B, T, H, 1), np.float32),
              wt_r=np.ones((B, T, H, 1), np.float32), idx_r=prod["idx_w"].copy())
    st = to_dev(m0)
    _, y = ops.scan(d, _prod_dev(p2), None, st, with_y_raw=True)
    assert np.array_equal(host(y), p2["v"])
    sth = host(st)
    for b in range(B):
        for h in range(H):
            last = {int(p2["idx_w"][b, t, h, 0]): t for t in range(T)}
            for s, t in last.items():
                assert np.array_equal(sth[b, h, s], p2["v"][b, t, h])


# ---------------------------------------------------------------------------
# bf16 state storage
# ---------------------------------------------------------------------------
def _bf16_state(rng, shape):
    """Random bf16 state: host fp64 copy of the exact values, device bf16 tensor."""
    m = torch.from_numpy((rng.standard_normal(shape) * 0.02).astype(np.float32)).to(torch.bfloat16)
    return m.to(torch.float64).numpy(), m.to(torch.device("cuda:0"))


@pytest.mark.parametrize("schedule,rule", [("direct", "slot"), ("stream", "slot"),
                                           ("two_phase", "slot"), ("direct", "gdn")])
@pytest.mark.parametrize("B,T,H,n,W,R,d_v,mode", [
    (1, 64, 1, 32, 8, 8, 16, "random"),
    (1, 700, 2, 32, 16, 16, 32, "repeat"),     # several rounds of the stream schedules
    (2, 50, 2, 8, 32, 32, 64, "repeat"),       # heavy slot reuse
    (3, 33, 2, 20, 64, 64, 128, "repeat"),
    (1, 30, 1, 16, 128, 128, 256, "random"),
    (2, 300, 2, 16, 32, 128, 64, "random"),    # W = 32 / R = 128
])
def test_stage_c_bf16_state(B, T, H, n, W, R, d_v, mode, schedule, rule):
    rng = np.random.default_rng(B * 100 + T + W + 7)
    N = n * n
    prod = random_products(rng, B, T, H, n, W, R, d_v, mode)
    m0, state = _bf16_state(rng, (B, H, N, d_v))
    gamma = rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32)
    flags = SCHEDULES[schedule] | _lib.SDM_FLAG_STATE_BF16
    if rule == "gdn":
        flags |= _lib.SDM_FLAG_DELTA_GDN
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=flags)
    out, y = ops.scan(d, _prod_dev(prod), to_dev(gamma), state, with_y_raw=True)
    torch.cuda.synchronize()
    st = state.to(torch.float64).cpu().numpy()
    oh, yh = host(out), host(y)
    walks = [(b, h) for b in range(B) for h in range(H)]
    ref = oracle_walks(prod, m0, gamma, 1e-6, walks, rule=rule, state="bf16")
    flips = late = 0
    for (b, h), (o_out, o_y, o_M) in ref.items():
        scale = max(np.abs(o_M).max(), np.abs(m0[b, h]).max())
        flips += check_bf16_state(st[b, h], o_M, scale, f"state walk {(b, h)}")
        late += check_bf16_reads(yh[b, :, h], o_y, oh[b, :, h], gamma[h],
                                 prod["gate"][b, :, h], 1e-6, scale, R, f"walk {(b, h)}")
        untouched = np.setdiff1d(np.arange(N), prod["idx_w"][b, :, h].ravel())
        assert np.array_equal(st[b, h][untouched], m0[b, h][untouched]), "unwritten rows changed"
    say(f"  state elements one rounding step apart: {flips}; tokens with such reads: {late}")


@pytest.mark.parametrize("schedule", ["direct", "stream", "two_phase"])
def test_stage_c_bf16_rounding_is_hardware_nearest_even(schedule):
    """beta = 1, weight 1: every written row holds v rounded to bf16, bit for bit as
    torch converts it; alpha = 1, beta = 0 leaves the state bit-identical."""
    rng = np.random.default_rng(8)
    B, T, H, n, d_v = 2, 40, 2, 8, 64
    prod = random_products(rng, B, T, H, n, 1, 1, d_v)
    # values with ties and near-ties of bf16 rounding in every row
    ties = (1.0 + (2 * rng.integers(0, 128, (B, T, H, d_v)) + 1) * 2.0 ** -8) * \
        rng.choice([-1.0, 1.0], (B, T, H, d_v)) * 2.0 ** rng.integers(-20, 20, (B, T, H, d_v))
    v = np.where(rng.random((B, T, H, d_v)) < 0.5, ties, prod["v"]).astype(np.float32)
    m0, st0 = _bf16_state(rng, (B, H, n * n, d_v))
    d = _dims(B=B, T=T, H=H, n=n, W=1, R=1, d_v=d_v,
              flags=SCHEDULES[schedule] | _lib.SDM_FLAG_STATE_BF16)
    p1 = dict(prod, alpha=np.ones((B, T, H), np.float32), beta=np.zeros((B, T, H), np.float32))
    st = st0.clone()
    ops.scan(d, _prod_dev(p1), None, st)
    assert torch.equal(st, st0)
    p2 = dict(prod, v=v, beta=np.ones((B, T, H), np.float32),
              wt_w=np.ones((B, T, H, 1), np.float32), wt_r=np.ones((B, T, H, 1), np.float32),
              idx_r=prod["idx_w"].copy())
    st = st0.clone()
    _, y = ops.scan(d, _prod_dev(p2), None, st, with_y_raw=True)
    torch.cuda.synchronize()
    vb = torch.from_numpy(v).to(torch.bfloat16)
    assert torch.equal(torch.from_numpy(host(y)), vb.to(torch.float32)), "reads of v"
    stc = st.cpu()
    for b in range(B):
        for h in range(H):
            last = {int(p2["idx_w"][b, t, h, 0]): t for t in range(T)}
            for s_, t in last.items():
                assert torch.equal(stc[b, h, s_], vb[b, t, h]), (b, h, s_, t)


def test_bf16_state_forward_matches_scan_and_halves_nothing_else():
    """sdm_forward with a bf16 state: same products as with fp32, the scan of them
    equals sdm_scan with the same flags bit for bit."""
    wl = synth.small("layer1p4b", B=2, T=160, d_model=256, n=40, W=16, R=16, d_v=32)
    h, dd = layer_inputs(wl, seed=3)
    d32, dbf = dims_for(wl), dims_for(wl)
    dbf.flags = _lib.SDM_FLAG_STATE_BF16
    m0b = dd["m0"].to(torch.bfloat16)
    st_f = broadcast_state(m0b, wl.B)
    out_f, p_f = ops.forward(dbf, dd["x"], dd["w_proj"], dd["A"], dd["b_dt"], dd["gamma"], st_f,
                             debug=True)
    st_32 = broadcast_state(dd["m0"], wl.B)
    _, p_32 = ops.forward(d32, dd["x"], dd["w_proj"], dd["A"], dd["b_dt"], dd["gamma"], st_32,
                          debug=True)
    st_s = broadcast_state(m0b, wl.B)
    out_s = ops.scan(dbf, p_f, dd["gamma"], st_s)
    torch.cuda.synchronize()
    for k in ("idx_w", "idx_r", "wt_w", "v", "alpha"):
        assert torch.equal(p_f[k], p_32[k]), k
    assert torch.equal(st_f, st_s)
    assert_close(host(out_f), host(out_s), "forward vs scan", rtol=1e-5, atol=1e-6)


# ---------------------------------------------------------------------------
# Stage D
# ---------------------------------------------------------------------------
def _compare_ids_from_x(gpu_p, orc, bound_rows):
    """Count id mismatches; each must be a near-tie or a GEMM-rounding flip."""
    flips = ties = 0
    for role in ("w", "r"):
        gi, oi = host(gpu_p[f"idx_{role}"]), orc[f"idx_{role}"]
        bad = np.argwhere(np.any(gi != oi, axis=-1))
        for idx in map(tuple, bad):
            gap = orc[f"gap_{role}"][idx]
            if gap < NEAR_TIE:
                ties += 1
            elif gap <= 2 * bound_rows[idx]:
                flips += 1
            else:
                raise AssertionError(f"ids differ at {idx} ({role}) with oracle gap {gap}")
    return ties, flips


@pytest.mark.parametrize("wl", [
    synth.WORKLOADS["tiny"],
    synth.small("layer1p4b", B=2, T=96, d_model=512, H=2, n=64, W=32, R=48, d_v=64),
])
def test_stage_d_forward_from_x(wl):
    h, d = layer_inputs(wl, seed=2)
    dm = dims_for(wl)
    state = broadcast_state(d["m0"], wl.B)
    out, p = ops.forward(dm, d["x"], d["w_proj"], d["A"], d["b_dt"], d["gamma"], state,
                         debug=True, with_scores=True)
    torch.cuda.synchronize()
    m0b = np.broadcast_to(h["m0"], (wl.B,) + h["m0"].shape)
    o_out, o_st, o_a = O.forward(h["x"], h["w_proj"], h["A"], h["b_dt"], h["gamma"], m0b, wl.H,
                                 wl.n, wl.d_v, wl.W, wl.R, wl.eps)
    x2 = h["x"].reshape(-1, wl.d_model)
    bnd = gemm_bound(x2, h["w_proj"], wl.d_model).reshape(wl.B, wl.T, wl.H, wl.P)
    bound_rows = bnd[..., :4 * wl.n].max(-1)
    ties, flips = _compare_ids_from_x(p, o_a, bound_rows)
    say(f"  near-ties {ties}, rounding flips {flips}")
    # ids from the GPU's own scores are bit-exact
    s = O.select_from_scores(host(p["scores"]), wl.n, wl.W, wl.R)
    assert np.array_equal(host(p["idx_w"]), s["idx_w"])
    assert np.array_equal(host(p["idx_r"]), s["idx_r"])
    if ties == 0 and flips == 0:
        assert_close(host(out), o_out, "out")
        assert_close(host(state), o_st, "state")
    else:  # walks with a flip are checked from the GPU's own selection
        ph = {k: host(v) for k, v in p.items()}
        ref = oracle_walks(ph, h["m0"], h["gamma"], wl.eps,
                           [(b, hh) for b in range(wl.B) for hh in range(wl.H)])
        for (b, hh), (oo, _, oM) in ref.items():
            assert_close(host(out)[b, :, hh], oo, f"out {(b, hh)}")
            assert_close(host(state)[b, hh], oM, f"state {(b, hh)}")


def test_forward_scan_over_several_token_chunks():
    """A run long enough that both slot-owner schedules split it into token chunks
    (their per-token buffers are bounded near 2 GiB): 32 walks of d_v = 128, which the
    two-phase schedule runs in 256-byte slices (3 chunks) and the stream schedule in
    128-byte ones (2 chunks).  The state equals the direct schedule's bit for bit, y
    and out agree within tolerance, and one walk's final state and reads match the
    oracle."""
    B, T, H, n, W, R, d_v = 8, 56000, 4, 8, 16, 16, 128
    rng = np.random.default_rng(66)
    prod = strided_products(rng, B, T, H, n, W, R, d_v)
    m0 = (rng.standard_normal((B, H, n * n, d_v)) * 0.3).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32)
    pd = _prod_dev(prod)
    gam = to_dev(gamma)
    res = {}
    for sched in ("direct", "stream", "two_phase"):
        d = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=SCHEDULES[sched])
        st = to_dev(m0)
        out, y = ops.scan(d, pd, gam, st, with_y_raw=True)
        torch.cuda.synchronize()
        res[sched] = (st, out, y)
        say(f"  {sched}: workspace {_lib.workspace_bytes(d, _lib.SDM_ENTRY_SCAN) / 2**30:.2f} GiB")
    st_d, out_d, y_d = res["direct"]
    for sched in ("stream", "two_phase"):
        st, out, y = res[sched]
        assert torch.equal(st, st_d), f"{sched}: state differs from the direct schedule's"
        for what, a, b in (("y_raw", y, y_d), ("out", out, out_d)):
            bad = int(((a - b).abs() > ATOL + RTOL * b.abs()).sum())
            assert bad == 0, f"{sched} {what}: {bad} elements outside tolerance"
    b, h = B - 1, H - 1
    o_y, o_M = O.scan(m0[b, h], *(prod[k][b, :, h] for k in ("idx_w", "wt_w", "idx_r", "wt_r",
                                                               "v", "alpha", "beta")))
    assert_close(host(st_d[b, h]), o_M, f"final state walk {(b, h)}")
    assert_close(host(res["two_phase"][2][b, :, h]), o_y, f"y_raw walk {(b, h)}")


def test_chunked_calls_equal_one_call():
    wl = synth.small("layer1p4b", B=2, T=80, d_model=256, H=2, n=24, W=16, R=16, d_v=32)
    _, d = layer_inputs(wl, seed=3)
    s1 = broadcast_state(d["m0"], wl.B)
    o1 = ops.forward(dims_for(wl), d["x"], d["w_proj"], d["A"], d["b_dt"], d["gamma"], s1)
    s2 = broadcast_state(d["m0"], wl.B)
    outs = []
    for t0, t1 in ((0, 30), (30, 31), (31, 80)):
        xs = d["x"][:, t0:t1].contiguous()
        outs.append(ops.forward(dims_for(wl, T=t1 - t0), xs, d["w_proj"], d["A"], d["b_dt"],
                                d["gamma"], s2))
    torch.cuda.synchronize()
    # the state is updated slot by slot in token order: bit-identical however the
    # tokens are split; read sums are accumulated in a run-dependent order
    assert torch.equal(s1, s2)
    assert_close(host(torch.cat(outs, dim=1)), host(o1), "out", rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("T", [40, 300])
def test_schedules_agree(T):
    wl = synth.small("layer1p4b", B=2, T=T, d_model=128, H=3, n=12, W=24, R=16, d_v=64)
    _, d = layer_inputs(wl, seed=5)
    res = {}
    for name, flag in SCHEDULES.items():
        st = broadcast_state(d["m0"], wl.B)
        dm = dims_for(wl)
        dm.flags = flag
        o = ops.forward(dm, d["x"], d["w_proj"], d["A"], d["b_dt"], d["gamma"], st)
        res[name] = (host(o), host(st))
    for name in ("stream", "two_phase"):
        assert np.array_equal(res["direct"][1], res[name][1]), name
        assert_close(res[name][0], res["direct"][0], f"out {name}", rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("T", [8, 600])
def test_timing_flag_records_every_launch_and_changes_nothing(T):
    wl = synth.small("layer1p4b", B=2, T=T, d_model=128, H=2, n=12, W=16, R=16, d_v=64)
    _, d = layer_inputs(wl, seed=6)
    _lib.timing_read()  # drop anything recorded earlier
    res = []
    for flags in (0, _lib.SDM_FLAG_TIMING):
        st = broadcast_state(d["m0"], wl.B)
        dm = dims_for(wl)
        dm.flags = flags
        o = ops.forward(dm, d["x"], d["w_proj"], d["A"], d["b_dt"], d["gamma"], st)
        res.append((host(o), host(st)))
    # the state is bitwise reproducible; the read sums of reads served inside a round's
    # write phase are added with LDS atomics, so `out` may differ in the last bits
    assert np.array_equal(res[0][1], res[1][1])
    assert_close(res[1][0], res[0][0], "out with timing", rtol=1e-5, atol=1e-6)
    rec = _lib.timing_read()
    names = [n for n, _ in rec]
    scan = ["scan_direct"] if T < 16 else ["bucket_count", "bucket_offsets", "bucket_scatter_rev",
                                           "two_phase_scan", "norm_gate"]
    assert names == ["proj_gemm_bf16", "select"] + scan, names
    assert all(ms > 0.0 for _, ms in rec), rec
    assert _lib.timing_read() == []


@pytest.mark.parametrize("wl", [
    synth.WORKLOADS["tiny"],
    synth.small("layer1p4b", B=2, T=300, d_model=256, H=2, n=24, W=16, R=24, d_v=32),
])
def test_slot_relabelling_permutes_ids_and_keeps_outputs(wl):
    """Permuting the columns of each half-key block (the same permutation for the write
    and the read half) and the rows of M0 to match relabels every slot: each output
    column of the projection is the same dot product, so the half-scores move
    bitwise and the ids map through the relabelling exactly.  The softmax weights are
    summed in id order, so they, and with them the state and out, agree up to
    rounding."""
    h, d = layer_inputs(wl, seed=8)
    n, P = wl.n, wl.P
    rng = np.random.default_rng(9)
    p1, p2 = rng.permutation(n), rng.permutation(n)
    relabel = (p1[:, None] * n + p2[None, :]).reshape(-1)  # old id -> new id
    w = d["w_proj"].clone()
    for hh in range(wl.H):
        for blk, perm in ((0, p1), (1, p2), (2, p1), (3, p2)):
            base = hh * P + blk * n
            w[base + torch.as_tensor(perm, device=w.device)] = d["w_proj"][base:base + n]
    m0 = d["m0"].clone()
    m0[:, torch.as_tensor(relabel, device=m0.device)] = d["m0"]
    res = []
    for wp, mm in ((d["w_proj"], d["m0"]), (w, m0)):
        st = broadcast_state(mm, wl.B)
        out, pr = ops.forward(dims_for(wl), d["x"], wp, d["A"], d["b_dt"], d["gamma"], st,
                              debug=True, with_scores=True)
        res.append((host(out), host(st), {k: host(v) for k, v in pr.items()}))
    (o_a, s_a, p_a), (o_b, s_b, p_b) = res
    sc_a = p_a["scores"].reshape(wl.B, wl.T, wl.H, 4, n)
    sc_b = p_b["scores"].reshape(wl.B, wl.T, wl.H, 4, n)
    for blk, perm in ((0, p1), (1, p2), (2, p1), (3, p2)):
        assert np.array_equal(sc_b[..., blk, perm], sc_a[..., blk, :]), f"half-score block {blk}"
    for role in ("w", "r"):
        ids_a, wt_a = p_a[f"idx_{role}"], p_a[f"wt_{role}"]
        mapped = relabel[ids_a]
        order = np.argsort(mapped, axis=-1, kind="stable")
        assert np.array_equal(np.take_along_axis(mapped, order, -1), p_b[f"idx_{role}"]), role
        assert_close(p_b[f"wt_{role}"], np.take_along_axis(wt_a, order, -1), f"wt_{role}")
    assert_close(s_b[:, :, relabel], s_a, "state", rtol=1e-5, atol=1e-6)
    assert_close(o_b, o_a, "out", rtol=1e-5, atol=1e-6)


def test_batch_entries_are_independent():
    """A batch of sequences equals each sequence run alone: the state bit for bit, out
    up to the order of the read sums (the slot-owner plan depends on the batch)."""
    wl = synth.small("layer1p4b", B=3, T=300, d_model=128, H=2, n=16, W=16, R=16, d_v=32)
    _, d = layer_inputs(wl, seed=10)
    st = broadcast_state(d["m0"], wl.B)
    out = host(ops.forward(dims_for(wl), d["x"], d["w_proj"], d["A"], d["b_dt"], d["gamma"], st))
    for b in range(wl.B):
        s1 = broadcast_state(d["m0"], 1)
        o1 = ops.forward(dims_for(wl, B=1), d["x"][b:b + 1].contiguous(), d["w_proj"], d["A"],
                         d["b_dt"], d["gamma"], s1)
        assert torch.equal(s1[0], st[b]), b
        assert_close(host(o1)[0], out[b], f"out {b}", rtol=1e-5, atol=1e-6)


def test_empty_call_changes_nothing():
    wl = synth.small("tiny", T=0)
    _, d = layer_inputs(synth.WORKLOADS["tiny"], seed=4)
    st = broadcast_state(d["m0"], 1)
    before = st.clone()
    dm = dims_for(wl)
    x = torch.empty((1, 0, wl.d_model), device="cuda")
    out = ops.forward(dm, x, d["w_proj"], d["A"], d["b_dt"], d["gamma"], st)
    torch.cuda.synchronize()
    assert out.shape == (1, 0, 1, 16) and torch.equal(st, before)


def test_hip_path_is_the_loaded_library():
    lib = _lib.load()
    assert lib._name.endswith("libsdm.so")
    with open("/proc/self/maps") as f:
        assert any("libsdm.so" in line for line in f)
