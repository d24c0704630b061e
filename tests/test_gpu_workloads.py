"""Parity at the workloads' real shapes.

* The 1.4B-like layer at full size (B=8, T=4096, d=2048, H=4, N=131044, W=R=64,
  d_v=128), run exactly as bench.py times it: sampled token rows are checked for
  the projection, gates and selection, and two whole (b, h) walks (every token's
  output and the final state) against the oracle run from the GPU's selection.
* The 8B-like layer (N = 2^20 slots, d=4096, H=8), the long single sequence (N =
  2^18, repeated blocks) and the decode workload (256 sequences, 64 one-token
  steps) at their real N, d_model and H with fewer tokens, so that the oracle
  finishes in seconds.
"""
import numpy as np
import pytest
import torch

from oracle import sdm_oracle as O
from sparse_memory_linear_sdm_amd import _lib, dims_for, ops, synth
from tests.gpu_util import (NEAR_TIE, assert_close, broadcast_state, gemm_bound, host,
                            layer_inputs, say, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"\n[gpu] {request.node.nodeid}")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _sampled_rows_check(wl, h, p, rows):
    """Stages A, B and D on the listed flattened token rows (b*T + t)."""
    x2 = h["x"].reshape(-1, wl.d_model)[rows]
    a = O.pass_a(x2, h["w_proj"], h["A"], h["b_dt"], wl.H, wl.n, wl.d_v, wl.W, wl.R)
    ridx = torch.as_tensor(rows, device=p["idx_w"].device)
    flat = lambda k: host(p[k].reshape((wl.B * wl.T, wl.H) + tuple(p[k].shape[3:]))[ridx])
    sc = flat("scores").astype(np.float64)
    bound = gemm_bound(x2, h["w_proj"], wl.d_model).reshape(len(rows), wl.H, wl.P)
    assert np.all(np.abs(sc - a["scores"]) <= bound[..., :4 * wl.n]), "scores beyond fp32 bound"
    assert_close(flat("alpha"), a["alpha"], "alpha")
    assert_close(flat("beta"), a["beta"], "beta")
    assert_close(flat("gate"), a["g"], "gate")
    # selection from the GPU's own scores: bit-exact ids
    s = O.select_from_scores(sc.astype(np.float32), wl.n, wl.W, wl.R)
    for role in ("w", "r"):
        assert np.array_equal(flat(f"idx_{role}"), s[f"idx_{role}"]), f"ids {role}"
        assert_close(flat(f"wt_{role}"), s[f"wt_{role}"], f"wt_{role}")
    # against the oracle from x: mismatches only at near-ties or GEMM-rounding flips
    brow = bound[..., :4 * wl.n].max(-1)
    flips = ties = 0
    for role in ("w", "r"):
        diff = np.any(flat(f"idx_{role}") != a[f"idx_{role}"], axis=-1)
        for idx in map(tuple, np.argwhere(diff)):
            gap = a[f"gap_{role}"][idx]
            assert gap <= 2 * brow[idx] or gap < NEAR_TIE, f"id mismatch at {idx}, gap {gap}"
            ties += gap < NEAR_TIE
            flips += gap >= NEAR_TIE
    say(f"  sampled rows {len(rows)}: near-ties {ties}, rounding flips {flips}")


def _walk_check(wl, h, p, state, out, walks, m0):
    for b, hh in walks:
        sel = {k: host(p[k][b, :, hh]) for k in ("idx_w", "wt_w", "idx_r", "wt_r", "v", "gate",
                                                  "alpha", "beta")}
        sel["g"] = sel.pop("gate")
        o_out, _, o_M = O.forward_walk(m0[hh], sel, h["gamma"][hh], wl.eps)
        assert_close(host(out[b, :, hh]), o_out, f"out walk {(b, hh)}")
        st = host(state[b, hh])
        assert_close(st, o_M, f"state walk {(b, hh)}")
        untouched = np.setdiff1d(np.arange(wl.N), sel["idx_w"].ravel())
        assert np.array_equal(st[untouched], m0[hh][untouched]), "unwritten rows changed"
        say(f"  walk {(b, hh)}: {untouched.size} slots never written")


def test_layer1p4b_full_size_bf16_state():
    """The same layer with the state stored in bf16 (SDM_FLAG_STATE_BF16): two whole
    walks against the oracle's bf16 scan run from the GPU's selection."""
    from tests.gpu_util import check_bf16_reads, check_bf16_state
    wl = synth.WORKLOADS["layer1p4b"]
    h, d = layer_inputs(wl, seed=0)
    dm = dims_for(wl)
    dm.flags = _lib.SDM_FLAG_STATE_BF16
    m0b = d["m0"].to(torch.bfloat16)
    m0h = m0b.to(torch.float64).cpu().numpy()
    state = broadcast_state(m0b, wl.B)
    p = ops.select(dm, d["x"], d["w_proj"], d["A"], d["b_dt"])
    out, y = ops.scan(dm, p, d["gamma"], state, with_y_raw=True)
    torch.cuda.synchronize()
    for b, hh in [(0, 0), (wl.B - 1, wl.H - 1)]:
        sel = {k: host(p[k][b, :, hh]) for k in ("idx_w", "wt_w", "idx_r", "wt_r", "v", "gate",
                                                  "alpha", "beta")}
        sel["g"] = sel.pop("gate")
        o_out, o_y, o_M = O.forward_walk(m0h[hh], sel, h["gamma"][hh], wl.eps, state="bf16")
        st = state[b, hh].to(torch.float64).cpu().numpy()
        scale = max(np.abs(o_M).max(), np.abs(m0h[hh]).max())
        flips = check_bf16_state(st, o_M, scale, f"state walk {(b, hh)}")
        late = check_bf16_reads(host(y[b, :, hh]), o_y, host(out[b, :, hh]), h["gamma"][hh],
                                sel["g"], wl.eps, scale, wl.R, f"walk {(b, hh)}")
        untouched = np.setdiff1d(np.arange(wl.N), sel["idx_w"].ravel())
        assert np.array_equal(st[untouched], m0h[hh][untouched]), "unwritten rows changed"
        say(f"  walk {(b, hh)}: {flips} state elements one rounding step apart, "
            f"{late} tokens with such reads")


def test_layer1p4b_full_size_as_benchmarked():
    wl = synth.WORKLOADS["layer1p4b"]
    h, d = layer_inputs(wl, seed=0)
    dm = dims_for(wl)
    state = broadcast_state(d["m0"], wl.B)
    # the benchmark's step: selection pass, then the scan, with library workspaces
    p = ops.select(dm, d["x"], d["w_proj"], d["A"], d["b_dt"], with_scores=True)
    out = ops.scan(dm, p, d["gamma"], state)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(wl.B * wl.T, 24, replace=False))
    _sampled_rows_check(wl, h, p, rows)
    _walk_check(wl, h, p, state, out, [(0, 0), (wl.B - 1, wl.H - 1)], h["m0"])
    # sdm_forward runs the same kernels: identical products, state and output
    st2 = broadcast_state(d["m0"], wl.B)
    out2, p2 = ops.forward(dm, d["x"], d["w_proj"], d["A"], d["b_dt"], d["gamma"], st2,
                           debug=True)
    torch.cuda.synchronize()
    for k in ("idx_w", "idx_r"):
        assert torch.equal(p2[k], p[k])
    assert torch.equal(st2, state)
    assert_close(host(out2), host(out), "forward vs select+scan", rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("name,T", [("layer8b", 256), ("long1m", 8192)])
def test_large_slot_workloads_reduced_tokens(name, T):
    wl = synth.small(name, T=T)
    h, d = layer_inputs(wl, seed=1)
    dm = dims_for(wl)
    state = broadcast_state(d["m0"], wl.B)
    out, p = ops.forward(dm, d["x"], d["w_proj"], d["A"], d["b_dt"], d["gamma"], state,
                         debug=True, with_scores=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(wl.B * wl.T, 12, replace=False))
    _sampled_rows_check(wl, h, p, rows)
    _walk_check(wl, h, p, state, out, [(0, 0), (wl.B - 1, wl.H - 1)], h["m0"])


def test_decode_steps_equal_one_call_and_oracle():
    wl = synth.WORKLOADS["decode256"]   # 256 sequences x 64 one-token steps
    h, d = layer_inputs(wl, seed=2)
    d1 = dims_for(wl, T=1)
    st_steps = broadcast_state(d["m0"], wl.B)
    outs = []
    for t in range(wl.T):
        xt = d["x"][:, t:t + 1].contiguous()
        outs.append(ops.forward(d1, xt, d["w_proj"], d["A"], d["b_dt"], d["gamma"], st_steps))
    out_steps = torch.cat(outs, dim=1)
    st_one = broadcast_state(d["m0"], wl.B)
    out_one, p = ops.forward(dims_for(wl), d["x"], d["w_proj"], d["A"], d["b_dt"], d["gamma"],
                             st_one, debug=True, with_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(st_steps, st_one), "64 one-token calls differ from one 64-token call"
    assert_close(host(out_steps), host(out_one), "decode out", rtol=1e-5, atol=1e-6)
    rng = np.random.default_rng(2)
    rows = np.sort(rng.choice(wl.B * wl.T, 12, replace=False))
    _sampled_rows_check(wl, h, p, rows)
    _walk_check(wl, h, p, st_one, out_one, [(0, 0), (17, 2), (wl.B - 1, wl.H - 1)], h["m0"])
