"""Training of the key-weighted (GDN-form) write rule: sdm_scan_train and
sdm_scan_backward with SDM_FLAG_DELTA_GDN against the oracle.  With an fp32 log the
training forward takes the chunk schedule from 64 tokens and the reverse walk from 256
(with W, R <= 64; tests/test_gpu_chunk_backward.py covers it on its own), while the
walks are few enough; else the direct schedule split over column slices of the state.  The cases cover both slice widths (16 and 32
columns), one slice per walk (norm and gate inside the walk) and several.

* The training forward gives state, y and out bit-identical to the inference scan of
  the same rule on the same schedule, and its write log equals the oracle's
  scan_gdn(record=True) log within the fp32 tolerance.
* The backward, given the GPU's forward results, the log and seeded incoming
  gradients, matches the oracle's scan_backward(rule="gdn") run on the same values:
  every gradient within 1e-4 of its tensor's scale, the initial state restored bit for
  bit, and the gradients bit-reproducible across runs.
"""
import numpy as np
import pytest
import torch

from oracle import sdm_oracle as O
from sparse_memory_linear_sdm_amd import _lib, ops
from tests.gpu_util import assert_close, host, random_products, say, to_dev

pytestmark = pytest.mark.gpu

GDN = _lib.SDM_FLAG_DELTA_GDN


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


CASES = [
    (1, 64, 1, 16, 8, 8, 16, "random", 0),
    (2, 50, 2, 8, 32, 32, 64, "repeat", 0),    # N = 64, W = R = 32: heavy slot reuse
    (1, 40, 1, 12, 128, 100, 64, "random", 0),  # the largest W
    (1, 300, 2, 40, 64, 64, 128, "random", 0),  # 300 tokens: the chunk schedule logs the rows
    (2, 17, 1, 4, 16, 16, 16, "random", 0),    # every slot in every write set
    (1, 30, 1, 16, 16, 16, 256, "same", 0),
    (1, 64, 2, 16, 16, 16, 32, "random", _lib.SDM_FLAG_LOG_FP8),
    (1, 64, 1, 16, 16, 16, 64, "repeat", _lib.SDM_FLAG_LOG_INT4),
    (16, 6, 4, 8, 16, 16, 128, "random", 0),   # 64 walks: 4 slices of 32 columns
    (32, 5, 4, 8, 16, 24, 128, "random", 0),   # 128 walks: 32-column slices (the cap)
    (64, 3, 4, 8, 16, 16, 128, "random", 0),   # 256 walks: 32-column slices (the cap)
    (64, 3, 4, 8, 16, 16, 64, "repeat", _lib.SDM_FLAG_LOG_FP8),
    (64, 3, 4, 8, 16, 16, 32, "random", 0),    # one 32-column slice: norm in the walk
]


@pytest.mark.parametrize("B,T,H,n,W,R,d_v,mode,logfl", CASES)
def test_gdn_training_matches_oracle(B, T, H, n, W, R, d_v, mode, logfl):
    rng = np.random.default_rng(B * 1000 + T + W + logfl)
    N = n * n
    prod = random_products(rng, B, T, H, n, W, R, d_v, mode)
    m0 = (rng.standard_normal((B, H, N, d_v)) * 0.02).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32)
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=GDN | logfl)
    pd = {k: to_dev(v) for k, v in prod.items()}
    gam = to_dev(gamma)
    state = to_dev(m0)
    out, y, log = ops.scan_train(d, pd, gam, state)
    # the inference scan of the same rule on the same schedule (the chunk one from 64
    # tokens with an fp32 log while B H d_v / 16 <= 1024, else the direct one): identical
    # results
    chunked = T >= 64 and not logfl and B * H * (d_v // 16) <= 1024
    sched = _lib.SDM_FLAG_SCAN_CHUNK if chunked else _lib.SDM_FLAG_SCAN_DIRECT
    st_i = to_dev(m0)
    out_i, y_i = ops.scan(_dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=GDN | sched), pd,
                          gam, st_i, with_y_raw=True)
    torch.cuda.synchronize()
    assert torch.equal(state, st_i) and torch.equal(y, y_i) and torch.equal(out, out_i)
    fmt = ops.log_format(d)
    log_h = (host(log["rows"]) if fmt == "fp32" else
             O.dequantize_rows(host(log["rows"]), host(log["scale"]), fmt))
    st_T, y_h = host(state), host(y)
    d_out = rng.standard_normal((B, T, H, d_v)).astype(np.float32)
    d_st = (rng.standard_normal((B, H, N, d_v)) * 0.1).astype(np.float32)
    runs = []
    for rep in range(2):
        st = to_dev(st_T)
        dS = to_dev(d_st)
        g = ops.scan_backward(d, pd, gam, st, dS, y, log, to_dev(d_out))
        torch.cuda.synchronize()
        runs.append((st, dS, g))
    st, dS, g = runs[0]
    for k in ("d_v", "d_gate", "d_alpha", "d_beta", "d_wt_w", "d_wt_r", "d_norm_w"):
        assert torch.equal(g[k], runs[1][2][k]), f"{k} not reproducible"
    assert torch.equal(dS, runs[1][1])
    if fmt == "fp32":
        assert np.array_equal(host(st), m0), "initial state not restored bit for bit"
    gh = {k: host(v) for k, v in g.items() if v is not None}
    d_gamma = np.zeros((H, d_v))
    for b in range(B):
        for h in range(H):
            sel = {k: prod[k][b, :, h] for k in ("idx_w", "wt_w", "idx_r", "wt_r", "v", "gate",
                                                  "alpha", "beta")}
            if fmt == "fp32":
                _, _, o_log = O.scan_gdn(m0[b, h], sel["idx_w"], sel["wt_w"], sel["idx_r"],
                                         sel["wt_r"], sel["v"], sel["alpha"], sel["beta"],
                                         record=True)
                assert_close(log_h[b, :, h], o_log, f"log walk {(b, h)}")
            og, oM0, odM = O.scan_backward(st_T[b, h], log_h[b, :, h], sel["idx_w"], sel["wt_w"],
                                           sel["idx_r"], sel["wt_r"], sel["v"], sel["alpha"],
                                           sel["beta"], y_h[b, :, h], sel["gate"], gamma[h],
                                           d.eps, d_out[b, :, h], d_st[b, h], rule="gdn")
            d_gamma[h] += og["d_gamma"]
            # with a quantised log both sides restore the same decoded rows
            assert np.array_equal(oM0, host(st)[b, h])
            for k in ("d_v", "d_gate", "d_alpha", "d_beta", "d_wt_w", "d_wt_r"):
                _close_to_scale(gh[k][b, :, h], og[k], f"{k} walk {(b, h)}")
            _close_to_scale(host(dS)[b, h], odM, f"d_state walk {(b, h)}")
    _close_to_scale(gh["d_norm_w"], d_gamma, "d_norm_w")


def test_gdn_training_refuses_slot_owner_schedules_and_chunk_quantised_logs():
    rng = np.random.default_rng(0)
    pd = {k: to_dev(v) for k, v in random_products(rng, 1, 64, 1, 16, 8, 8, 16).items()}
    st = torch.zeros((1, 1, 256, 16), device="cuda")
    for fl in (_lib.SDM_FLAG_SCAN_TWO_PHASE, _lib.SDM_FLAG_SCAN_STREAM,
               _lib.SDM_FLAG_SCAN_CHUNK | _lib.SDM_FLAG_LOG_FP8):
        with pytest.raises(_lib.SdmError) as e:
            ops.scan_train(_dims(T=64, flags=GDN | fl), pd, None, st)
        assert e.value.code == _lib.SDM_ERR_UNSUPPORTED


@pytest.mark.parametrize("fmt", ["fp8", "int4"])
def test_gdn_quantised_log_over_staged_token_chunks(fmt):
    """A quantised log is staged in fp32 per token chunk of at most 256 MiB and
    encoded after each chunk's walk: 4 x 300 tokens x 4 heads x W = 128 x d_v = 128
    takes two chunks.  The codes equal the oracle's encoding of the fp32 log of the
    same walk, and state, y and out equal the fp32-log run bit for bit."""
    rng = np.random.default_rng(11)
    B, T, H, n, W, R, d_v = 4, 300, 4, 16, 128, 64, 128
    prod = random_products(rng, B, T, H, n, W, R, d_v, "random")
    m0 = (rng.standard_normal((B, H, n * n, d_v)) * 0.3).astype(np.float32)
    flag = _lib.SDM_FLAG_LOG_FP8 if fmt == "fp8" else _lib.SDM_FLAG_LOG_INT4
    pd = {k: to_dev(v) for k, v in prod.items()}
    st_a, st_b = to_dev(m0), to_dev(m0)
    # quantised logs take the direct schedule: the fp32 run names it
    out_a, y_a, log_a = ops.scan_train(
        _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=GDN | _lib.SDM_FLAG_SCAN_DIRECT),
        pd, None, st_a)
    out_b, y_b, log_b = ops.scan_train(
        _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=GDN | flag), pd, None, st_b)
    torch.cuda.synchronize()
    assert torch.equal(st_a, st_b) and torch.equal(y_a, y_b) and torch.equal(out_a, out_b)
    rows = host(log_a["rows"])
    del log_a
    codes, amax = O.quantize_rows(rows, fmt)
    assert np.array_equal(host(log_b["scale"]), amax)
    assert np.array_equal(host(log_b["rows"]), codes)
