"""The key-weighted rule's reverse walk on the chunk schedule (chunk_back_kernel,
SDM_FLAG_DELTA_GDN with SDM_FLAG_SCAN_CHUNK, or by default from 256 tokens with an
fp32 log and W, R <= 64) against the oracle's reverse walk (scan_backward,
rule="gdn", pinned by central differences; its chunkwise form scan_backward_chunkwise
is pinned to it).

Shapes cover slot spaces so small that every slot is written and read by every
token (chains of 32 writers, reads of rows that earlier writers of the chunk left,
reads of the chunk-start row before a slot's first writer), slots that tokens only
read (several reads in one chunk), ragged last chunks, W = R = 1, W = R = 64, d_v from
16 to 256 and several walks.  Each case runs the training forward on the chunk
schedule and on the direct schedule; the backward of each must match the oracle's
backward of the same log within 1e-4 of each gradient's scale, restore M0 bit for
bit, agree with the sliced direct reverse walk on the same log, and give the same
bits on a second run.
"""
import numpy as np
import pytest
import torch

from oracle import sdm_oracle as O
from sparse_memory_linear_sdm_amd import _lib, ops
from tests.gpu_util import host, random_products, say, to_dev

pytestmark = pytest.mark.gpu

GDN = _lib.SDM_FLAG_DELTA_GDN
CHUNK = _lib.SDM_FLAG_SCAN_CHUNK
DIRECT = _lib.SDM_FLAG_SCAN_DIRECT


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


def _close_to_scale(got, exp, what, rel=1e-4, extra=0.0):
    got = np.asarray(got, np.float64)
    exp = np.asarray(exp, np.float64)
    scale = max(np.abs(exp).max(), 1e-30)
    err = np.abs(got - exp)
    bad = err > rel * (np.abs(exp) + scale) + extra
    assert not bad.any(), (f"{what}: {bad.sum()} elements beyond {rel} of the scale {scale:.3e}; "
                           f"max err {err.max():.3e}")


CASES = [
    (1, 64, 1, 16, 8, 8, 16, "random"),
    (2, 75, 2, 6, 16, 12, 32, "random"),      # N = 36: chains and shared reads in every chunk
    (2, 33, 1, 8, 64, 64, 64, "random"),      # N = 64 = W = R: every slot, every token
    (1, 50, 1, 4, 16, 16, 16, "random"),      # N = 16 = W = R
    (1, 300, 2, 40, 64, 64, 128, "repeat"),   # runs of identical selections
    (1, 260, 1, 362, 64, 64, 128, "random"),  # the bench's slot space: few collisions
    (3, 40, 2, 12, 1, 1, 16, "random"),       # W = R = 1
    (1, 40, 1, 12, 16, 16, 256, "random"),    # d_v = 256: 16 slices
    (8, 45, 4, 10, 8, 24, 64, "random"),      # 32 walks, R > W
]


@pytest.mark.parametrize("fwd", ["chunk", "direct"])
@pytest.mark.parametrize("B,T,H,n,W,R,d_v,mode", CASES)
def test_chunk_backward_matches_oracle(B, T, H, n, W, R, d_v, mode, fwd):
    rng = np.random.default_rng(B * 1000 + T + W + d_v + (fwd == "chunk"))
    N = n * n
    prod = random_products(rng, B, T, H, n, W, R, d_v, mode)
    m0 = (rng.standard_normal((B, H, N, d_v)) * 0.02).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32)
    kw = dict(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v)
    pd = {k: to_dev(v) for k, v in prod.items()}
    gam = to_dev(gamma)
    state = to_dev(m0)
    fl = CHUNK if fwd == "chunk" else DIRECT
    out, y, log = ops.scan_train(_dims(**kw, flags=GDN | fl), pd, gam, state)
    torch.cuda.synchronize()
    st_T, y_h, log_h = host(state), host(y), host(log["rows"])
    d_out = rng.standard_normal((B, T, H, d_v)).astype(np.float32)
    d_st = (rng.standard_normal((B, H, N, d_v)) * 0.1).astype(np.float32)
    db = _dims(**kw, flags=GDN | CHUNK)
    runs = []
    for rep in range(2):
        st, dS = to_dev(st_T), to_dev(d_st)
        g = ops.scan_backward(db, pd, gam, st, dS, y, log, to_dev(d_out))
        torch.cuda.synchronize()
        runs.append((st, dS, g))
    st, dS, g = runs[0]
    for k in ("d_v", "d_gate", "d_alpha", "d_beta", "d_wt_w", "d_wt_r", "d_norm_w"):
        assert torch.equal(g[k], runs[1][2][k]), f"{k} not reproducible"
    assert torch.equal(dS, runs[1][1]) and torch.equal(st, runs[1][0])
    assert np.array_equal(host(st), m0), "initial state not restored bit for bit"
    # the sliced direct reverse walk on the same log
    st_s, dS_s = to_dev(st_T), to_dev(d_st)
    g_s = ops.scan_backward(_dims(**kw, flags=GDN | DIRECT), pd, gam, st_s, dS_s, y, log,
                            to_dev(d_out))
    torch.cuda.synchronize()
    assert torch.equal(st_s, st)
    gh = {k: host(v) for k, v in g.items() if v is not None}
    dSh = host(dS)
    for k in ("d_v", "d_alpha", "d_beta", "d_wt_w", "d_wt_r"):  # the same dy: no cancellation
        _close_to_scale(gh[k], host(g_s[k]), f"{k} vs the sliced walk")
    _close_to_scale(dSh, host(dS_s), "d_state vs the sliced walk")
    d_gamma = np.zeros((H, d_v))
    for b in range(B):
        for h in range(H):
            sel = {k: prod[k][b, :, h] for k in ("idx_w", "wt_w", "idx_r", "wt_r", "v", "gate",
                                                  "alpha", "beta")}
            og, oM0, odM = O.scan_backward(st_T[b, h], log_h[b, :, h], sel["idx_w"], sel["wt_w"],
                                           sel["idx_r"], sel["wt_r"], sel["v"], sel["alpha"],
                                           sel["beta"], y_h[b, :, h], sel["gate"], gamma[h],
                                           1e-6, d_out[b, :, h], d_st[b, h], rule="gdn")
            d_gamma[h] += og["d_gamma"]
            assert np.array_equal(oM0, host(st)[b, h])
            for k in ("d_v", "d_gate", "d_alpha", "d_beta", "d_wt_w"):
                _close_to_scale(gh[k][b, :, h], og[k], f"{k} walk {(b, h)}")
            # d_wt_r = <dy, M[r]>: the RMSNorm is scale-free, so along y the two terms of
            # dy = s (u - yhat mean(u yhat)) cancel (with R = 1 the result is
            # s^3 eps <u, y> / q).  fp32 leaves an error of a few ulps of the terms:
            # 16 2^-24 s |u| times the walk's largest row norm.
            yt = y_h[b, :, h].astype(np.float64)
            st_ = 1.0 / np.sqrt(np.mean(yt * yt, axis=1) + 1e-6)
            ut = d_out[b, :, h] * gamma[h] * sel["gate"]
            rmax = max(np.linalg.norm(log_h[b, :, h], axis=-1).max(),
                       np.linalg.norm(st_T[b, h], axis=-1).max())
            extra = (16 * 2.0 ** -24 * st_ * np.linalg.norm(ut, axis=1) * rmax)[:, None]
            _close_to_scale(gh["d_wt_r"][b, :, h], og["d_wt_r"], f"d_wt_r walk {(b, h)}",
                            extra=extra)
            _close_to_scale(dSh[b, h], odM, f"d_state walk {(b, h)}")
    _close_to_scale(gh["d_norm_w"], d_gamma, "d_norm_w")



def test_gdn_training_at_the_full_bench_size():
    """The 1.4B-like layer at full size (8 x 4096 tokens, 4 heads, N = 131,044) with the
    key-weighted rule, products from the GPU's own selection and the default schedules
    (chunk training forward with its log, chunkwise reverse walk): two complete walks
    against the oracle's reverse walk from the GPU's final state, log and y; M0
    restored bit for bit for every walk; every walk's gradients against the sliced
    direct reverse walk on the same log."""
    from sparse_memory_linear_sdm_amd import dims_for, synth
    from tests.gpu_util import layer_inputs
    wl = synth.WORKLOADS["layer1p4b"]
    h, dd = layer_inputs(wl, seed=13)
    dm = dims_for(wl)
    dm.flags |= GDN
    p = ops.select(dm, dd["x"], dd["w_proj"], dd["A"], dd["b_dt"])
    del dd["x"]
    gam = dd["gamma"]
    st = dd["m0"].unsqueeze(0).repeat(wl.B, 1, 1, 1)
    _, y, log = ops.scan_train(dm, p, gam, st)
    gen = torch.Generator(device=st.device).manual_seed(14)
    d_out = torch.randn(y.shape, device=st.device, generator=gen)
    d_st = torch.randn(st.shape, device=st.device, generator=gen) * 0.1
    walks = [(0, 0), (wl.B - 1, wl.H - 1)]
    keep = {(b, hh): (host(st[b, hh]), host(log["rows"][b, :, hh]), host(y[b, :, hh]),
                      host(d_out[b, :, hh]), host(d_st[b, hh])) for b, hh in walks}
    st_s = st.clone()
    dS, dS_s = d_st.clone(), d_st.clone()
    g = ops.scan_backward(dm, p, gam, st, dS, y, log, d_out)
    torch.cuda.synchronize()
    say("  chunkwise reverse walk done")
    for b in range(wl.B):
        for hh in range(wl.H):
            assert torch.equal(st[b, hh], dd["m0"][hh]), f"M0 not restored for walk {(b, hh)}"
    ds = type(dm).from_buffer_copy(dm)
    ds.flags = dm.flags | DIRECT
    g_s = ops.scan_backward(ds, p, gam, st_s, dS_s, y, log, d_out)
    torch.cuda.synchronize()
    assert torch.equal(st_s, st)
    for k in ("d_v", "d_alpha", "d_beta", "d_wt_w", "d_wt_r"):
        _close_to_scale(host(g[k]), host(g_s[k]), f"{k} vs the sliced walk")
    _close_to_scale(host(dS), host(dS_s), "d_state vs the sliced walk")
    del g_s, dS_s, st_s
    m0_h = host(dd["m0"])
    for (b, hh), (mT, lg, yy, do, dst) in keep.items():
        sel = {k: host(p[k][b, :, hh]) for k in ("idx_w", "wt_w", "idx_r", "wt_r", "v", "gate",
                                                 "alpha", "beta")}
        og, oM0, odM = O.scan_backward(mT, lg, sel["idx_w"], sel["wt_w"], sel["idx_r"],
                                       sel["wt_r"], sel["v"], sel["alpha"], sel["beta"], yy,
                                       sel["gate"], h["gamma"][hh], wl.eps, do, dst, rule="gdn")
        assert np.array_equal(oM0, m0_h[hh])
        for k in ("d_v", "d_gate", "d_alpha", "d_beta", "d_wt_w", "d_wt_r"):
            _close_to_scale(host(g[k][b, :, hh]), og[k], f"{k} walk {(b, hh)}")
        _close_to_scale(host(dS[b, hh]), odM, f"d_state walk {(b, hh)}")
        say(f"  walk {(b, hh)} matches the oracle")


def test_gdn_chunk_training_at_the_8b_slot_space():
    """The 8B-like slot space (N = 1024^2, W = R = 64, d_v = 128; the largest row offsets
    of the chunk kernels) with the key-weighted rule on the chunk schedule, 2 x 2 walks
    of 1200 tokens (38 chunks, the last ragged): inference state and out against the
    oracle's walk, then the training forward and the chunkwise reverse walk against the
    oracle's reverse walk on one walk, M0 restored bit for bit for every walk."""
    from tests.test_gpu_chunk import random_products_fast
    rng = np.random.default_rng(17)
    B, T, H, n, W, R, d_v = 2, 1200, 2, 1024, 64, 64, 128
    N = n * n
    prod = random_products_fast(rng, B, T, H, n, W, R, d_v)
    m0 = (rng.standard_normal((B, H, N, d_v)) * 0.02).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32)
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=GDN | CHUNK)
    pd = {k: to_dev(v) for k, v in prod.items()}
    gam = to_dev(gamma)
    state = to_dev(m0)
    out, y, log = ops.scan_train(d, pd, gam, state)
    torch.cuda.synchronize()
    b, hh = B - 1, H - 1
    sel = {k: prod[k][b, :, hh] for k in ("idx_w", "wt_w", "idx_r", "wt_r", "v", "gate", "alpha",
                                          "beta")}
    y_o, M_o, log_o = O.scan_gdn(m0[b, hh], sel["idx_w"], sel["wt_w"], sel["idx_r"], sel["wt_r"],
                                 sel["v"], sel["alpha"], sel["beta"], record=True)
    st_T = host(state)
    _close_to_scale(st_T[b, hh], M_o, "state", rel=1e-5)
    _close_to_scale(host(y)[b, :, hh], y_o, "y", rel=1e-5)
    log_h = host(log["rows"])
    _close_to_scale(log_h[b, :, hh], log_o, "log", rel=1e-5)
    del M_o, log_o
    d_out = rng.standard_normal((B, T, H, d_v)).astype(np.float32)
    d_st = (rng.standard_normal((B, H, N, d_v)) * 0.1).astype(np.float32)
    dS = to_dev(d_st)
    g = ops.scan_backward(d, pd, gam, state, dS, y, log, to_dev(d_out))
    torch.cuda.synchronize()
    assert torch.equal(state, to_dev(m0)), "initial state not restored bit for bit"
    og, oM0, odM = O.scan_backward(st_T[b, hh], log_h[b, :, hh], sel["idx_w"], sel["wt_w"],
                                   sel["idx_r"], sel["wt_r"], sel["v"], sel["alpha"], sel["beta"],
                                   host(y)[b, :, hh], sel["gate"], gamma[hh], 1e-6,
                                   d_out[b, :, hh], d_st[b, hh], rule="gdn")
    assert np.array_equal(oM0, m0[b, hh])
    for k in ("d_v", "d_gate", "d_alpha", "d_beta", "d_wt_w", "d_wt_r"):
        _close_to_scale(host(g[k][b, :, hh]), og[k], f"{k}")
    _close_to_scale(host(dS)[b, hh], odM, "d_state")
