"""The chunkwise schedule of the scan (SDM_FLAG_SCAN_CHUNK) against the oracle.

Both write rules: the per-slot rule against scan(), the key-weighted (GDN) rule
against scan_gdn() -- the sequential recurrences that define the result; the chunkwise
form is a reordering of the same arithmetic (the oracle's own chunkwise form is
pinned to them).  Shapes cover ragged last chunks, slot spaces so small that most
tokens of a chunk share slots (long chains of writers of one slot), W = R = 1, the
largest W, and every d_v.  At the 1.4B-like full size, two walks are compared with the
oracle and every walk with the other GPU schedules.
"""
import numpy as np
import pytest
import torch

from oracle import sdm_oracle as O
from sparse_memory_linear_sdm_amd import _lib, dims_for, ops, synth
from tests.gpu_util import (ATOL, RTOL, assert_close, host, layer_inputs, oracle_walks,
                            random_products, say, to_dev)

pytestmark = pytest.mark.gpu

CHUNK = _lib.SDM_FLAG_SCAN_CHUNK
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


def _prod_dev(p):
    return {k: to_dev(v) for k, v in p.items()}


def _close_dev(got, exp, what):
    """assert_close's rule, evaluated on the device (for multi-GB tensors)."""
    bad = (got - exp).abs() > ATOL + RTOL * exp.abs()
    nbad = int(bad.sum())
    assert nbad == 0, (f"{what}: {nbad} elements out of tolerance; max |err| "
                       f"{float((got - exp).abs().max()):.3e}")


@pytest.mark.parametrize("rule", ["slot", "gdn"])
@pytest.mark.parametrize("B,T,H,n,W,R,d_v,mode", [
    (1, 64, 1, 16, 8, 8, 16, "random"),
    (2, 75, 2, 6, 16, 12, 32, "random"),       # N = 36: chains of writers, ragged last chunk
    (1, 40, 1, 12, 128, 100, 64, "random"),    # the largest W; 128 of 144 slots per token
    (1, 300, 2, 40, 64, 64, 128, "repeat"),    # runs of identical selections
    (2, 33, 1, 8, 1, 1, 16, "random"),         # W = R = 1, one token in the last chunk
    (1, 96, 1, 16, 16, 16, 256, "random"),
    (1, 50, 2, 8, 16, 8, 64, "same"),          # every token the same slots
    (3, 31, 1, 4, 16, 16, 32, "random"),       # every slot written by every token, T < 32
    (1, 70, 1, 12, 128, 128, 256, "repeat"),   # the largest LDS use of both kernels
    (4, 1, 2, 8, 16, 16, 32, "random"),        # one token per walk
])
def test_chunk_schedule_matches_oracle(rule, B, T, H, n, W, R, d_v, mode):
    rng = np.random.default_rng(B * 1000 + T * 7 + W + (rule == "gdn"))
    N = n * n
    prod = random_products(rng, B, T, H, n, W, R, d_v, mode)
    m0 = (rng.standard_normal((B, H, N, d_v)) * 0.02).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32)
    flags = CHUNK | (GDN if rule == "gdn" else 0)
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=flags)
    state = to_dev(m0)
    out, y = ops.scan(d, _prod_dev(prod), to_dev(gamma), state, with_y_raw=True)
    torch.cuda.synchronize()
    st, oh, yh = host(state), host(out), host(y)
    walks = [(b, h) for b in range(B) for h in range(H)]
    ref = oracle_walks(prod, m0, gamma, 1e-6, walks, rule=rule)
    for (b, h), (o_out, o_y, o_M) in ref.items():
        assert_close(yh[b, :, h], o_y, f"y_raw walk {(b, h)}")
        assert_close(oh[b, :, h], o_out, f"out walk {(b, h)}")
        assert_close(st[b, h], o_M, f"state walk {(b, h)}")
        untouched = np.setdiff1d(np.arange(N), prod["idx_w"][b, :, h].ravel())
        assert np.array_equal(st[b, h][untouched], m0[b, h][untouched]), "unwritten rows changed"


@pytest.mark.parametrize("rule", ["slot", "gdn"])
def test_chunk_schedule_is_deterministic_and_chunked_calls_agree(rule):
    rng = np.random.default_rng(5)
    B, T, H, n, W, R, d_v = 2, 96, 2, 8, 16, 16, 32
    prod = random_products(rng, B, T, H, n, W, R, d_v, "random")
    m0 = (rng.standard_normal((B, H, n * n, d_v)) * 0.02).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32)
    flags = CHUNK | (GDN if rule == "gdn" else 0)
    runs = []
    for _ in range(2):
        state = to_dev(m0)
        out, y = ops.scan(_dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=flags),
                          _prod_dev(prod), to_dev(gamma), state, with_y_raw=True)
        runs.append((out, y, state))
    torch.cuda.synchronize()
    for a, b in zip(runs[0], runs[1]):
        assert torch.equal(a, b), "two calls differ"
    # two calls over consecutive token ranges (not aligned to the chunk length) equal one
    state = to_dev(m0)
    outs = []
    for t0, t1 in ((0, 45), (45, T)):
        part = {k: np.ascontiguousarray(v[:, t0:t1]) for k, v in prod.items()}
        o, _ = ops.scan(_dims(B=B, T=t1 - t0, H=H, n=n, W=W, R=R, d_v=d_v, flags=flags),
                        _prod_dev(part), to_dev(gamma), state, with_y_raw=True)
        outs.append(host(o))
    torch.cuda.synchronize()
    assert_close(np.concatenate(outs, axis=1), host(runs[0][0]), "chunked calls")
    assert_close(host(state), host(runs[0][2]), "state after chunked calls")


def test_chunk_schedule_forward_from_x():
    wl = synth.small("tiny", T=100)
    h, d = layer_inputs(wl, seed=2)
    for extra in (0, GDN):
        dm = dims_for(wl)
        dm.flags = CHUNK | extra
        st = d["m0"].unsqueeze(0).clone()
        out, prod = ops.forward(dm, d["x"], d["w_proj"], d["A"], d["b_dt"], d["gamma"], st,
                                debug=True)
        dd = dims_for(wl)
        dd.flags = _lib.SDM_FLAG_SCAN_DIRECT | extra
        st2 = d["m0"].unsqueeze(0).clone()
        out2 = ops.scan(dd, prod, d["gamma"], st2)
        torch.cuda.synchronize()
        assert_close(host(out), host(out2), f"forward out flags {extra}")
        assert_close(host(st), host(st2), f"forward state flags {extra}")


def test_chunk_schedule_rejects_bf16_state_and_quantised_training_logs():
    d = _dims(T=64, flags=CHUNK | _lib.SDM_FLAG_STATE_BF16)
    assert _lib.workspace_bytes(_dims(T=64, flags=CHUNK), _lib.SDM_ENTRY_SCAN) > 0
    rng = np.random.default_rng(0)
    prod = _prod_dev(random_products(rng, 1, 64, 1, 16, 8, 8, 16))
    with pytest.raises(_lib.SdmError) as e:
        ops.scan(d, prod, None, torch.zeros((1, 1, 256, 16), dtype=torch.bfloat16,
                                             device="cuda"))
    assert e.value.code == _lib.SDM_ERR_UNSUPPORTED
    for lf in (_lib.SDM_FLAG_LOG_FP8, _lib.SDM_FLAG_LOG_INT4):
        with pytest.raises(_lib.SdmError) as e:
            ops.scan_train(_dims(T=64, flags=CHUNK | lf), prod, None,
                           torch.zeros((1, 1, 256, 16), device="cuda"))
        assert e.value.code == _lib.SDM_ERR_UNSUPPORTED


@pytest.mark.parametrize("rule", ["slot", "gdn"])
@pytest.mark.parametrize("B,T,H,n,W,R,d_v,mode", [
    (2, 75, 2, 6, 16, 12, 32, "random"),       # N = 36: chains of writers in every chunk
    (1, 300, 2, 40, 64, 64, 128, "repeat"),    # runs of identical selections
    (1, 40, 1, 12, 128, 100, 64, "random"),    # the largest W
])
def test_chunk_training_forward_and_backward(rule, B, T, H, n, W, R, d_v, mode):
    """The training forward on the chunk schedule: the last writer of each slot also
    logs the row every writer of its chain replaced.  State, y and out equal the chunk
    inference scan bit for bit; the log equals the oracle's log of the walk; the
    reverse walk on these results matches the oracle's backward and restores M0."""
    rng = np.random.default_rng(B * 100 + T + W + (rule == "gdn"))
    N = n * n
    prod = random_products(rng, B, T, H, n, W, R, d_v, mode)
    m0 = (rng.standard_normal((B, H, N, d_v)) * 0.02).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32)
    flags = CHUNK | (GDN if rule == "gdn" else 0)
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=flags)
    pd = _prod_dev(prod)
    g = to_dev(gamma)
    state = to_dev(m0)
    out, y, log = ops.scan_train(d, pd, g, state)
    st_i = to_dev(m0)
    out_i, y_i = ops.scan(d, pd, g, st_i, with_y_raw=True)
    torch.cuda.synchronize()
    assert torch.equal(state, st_i) and torch.equal(y, y_i) and torch.equal(out, out_i)
    log_h, st_T, y_h = host(log["rows"]), host(state), host(y)
    d_out = rng.standard_normal((B, T, H, d_v)).astype(np.float32)
    d_st = (rng.standard_normal((B, H, N, d_v)) * 0.1).astype(np.float32)
    st, dS = to_dev(st_T), to_dev(d_st)
    gr = ops.scan_backward(d, pd, g, st, dS, y, log, to_dev(d_out))
    torch.cuda.synchronize()
    assert np.array_equal(host(st), m0), "initial state not restored bit for bit"
    gh = {k: host(v) for k, v in gr.items() if v is not None}
    walk = O.scan_gdn if rule == "gdn" else O.scan
    for b in range(B):
        for h in range(H):
            sel = {k: prod[k][b, :, h] for k in ("idx_w", "wt_w", "idx_r", "wt_r", "v", "gate",
                                                  "alpha", "beta")}
            _, _, o_log = walk(m0[b, h], sel["idx_w"], sel["wt_w"], sel["idx_r"], sel["wt_r"],
                               sel["v"], sel["alpha"], sel["beta"], record=True)
            assert_close(log_h[b, :, h], o_log, f"log walk {(b, h)}")
            og, _, odM = O.scan_backward(st_T[b, h], log_h[b, :, h], sel["idx_w"], sel["wt_w"],
                                         sel["idx_r"], sel["wt_r"], sel["v"], sel["alpha"],
                                         sel["beta"], y_h[b, :, h], sel["gate"], gamma[h], 1e-6,
                                         d_out[b, :, h], d_st[b, h], rule=rule)
            for k in ("d_v", "d_gate", "d_alpha", "d_beta", "d_wt_w", "d_wt_r"):
                got, exp = gh[k][b, :, h].astype(np.float64), og[k]
                scale = max(np.abs(exp).max(), 1e-30)
                assert np.all(np.abs(got - exp) <= 1e-4 * (np.abs(exp) + scale)), f"{k} {(b, h)}"
            scale = max(np.abs(odM).max(), 1e-30)
            assert np.all(np.abs(host(dS)[b, h] - odM) <= 1e-4 * (np.abs(odM) + scale)), \
                f"d_state {(b, h)}"


@pytest.mark.parametrize("rule", ["slot", "gdn"])
def test_chunk_schedule_full_size(rule):
    """The 1.4B-like shape (B=8, T=4096, H=4, N=131072, W=R=64, d_v=128): two walks
    against the oracle, every walk against the slot-owner (per-slot rule) or the
    direct (GDN rule) schedule."""
    wl = synth.WORKLOADS["layer1p4b"]
    rng = np.random.default_rng(3)
    B, T, H, n, W, R, d_v = wl.B, wl.T, wl.H, wl.n, wl.W, wl.R, wl.d_v
    prod = random_products_fast(rng, B, T, H, n, W, R, d_v)
    N = n * n
    m0 = (rng.standard_normal((B, H, N, d_v)) * 0.02).astype(np.float32)
    gamma = rng.uniform(0.5, 1.5, (H, d_v)).astype(np.float32)
    pd = _prod_dev(prod)
    g = to_dev(gamma)
    extra = GDN if rule == "gdn" else 0
    state = to_dev(m0)
    out, y = ops.scan(_dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=CHUNK | extra), pd, g,
                      state, with_y_raw=True)
    other = _lib.SDM_FLAG_SCAN_DIRECT if rule == "gdn" else _lib.SDM_FLAG_SCAN_TWO_PHASE
    state2 = to_dev(m0)
    out2, y2 = ops.scan(_dims(B=B, T=T, H=H, n=n, W=W, R=R, d_v=d_v, flags=other | extra), pd, g,
                        state2, with_y_raw=True)
    torch.cuda.synchronize()
    _close_dev(y, y2, "y_raw against the other schedule")
    _close_dev(out, out2, "out against the other schedule")
    _close_dev(state, state2, "state against the other schedule")
    del state2, y2, out2
    walks = [(0, 0), (B - 1, H - 1)]
    say(f"  oracle walks {walks}")
    ref = oracle_walks(prod, m0, gamma, 1e-6, walks, rule=rule)
    st, yh = host(state), host(y)
    for (b, h), (o_out, o_y, o_M) in ref.items():
        assert_close(yh[b, :, h], o_y, f"y_raw walk {(b, h)}")
        assert_close(st[b, h], o_M, f"state walk {(b, h)}")


def random_products_fast(rng, B, T, H, n, W, R, d_v):
    """Ascending distinct ids for many tokens at once: W (or R) draws from disjoint
    equal bins of the slot space, one per bin, so ids are distinct and sorted."""
    N = n * n
    shp = (B, T, H)

    def ids(count):
        width = N // count
        off = rng.integers(0, width, shp + (count,))
        return (np.arange(count) * width + off).astype(np.int32)

    return dict(idx_w=ids(W), wt_w=rng.dirichlet(np.ones(W), shp).astype(np.float32),
                idx_r=ids(R), wt_r=rng.dirichlet(np.ones(R), shp).astype(np.float32),
                v=rng.standard_normal(shp + (d_v,)).astype(np.float32),
                gate=rng.uniform(0, 1, shp + (d_v,)).astype(np.float32),
                alpha=rng.uniform(0.3, 1.0, shp).astype(np.float32),
                beta=rng.uniform(0.0, 1.0, shp).astype(np.float32))
