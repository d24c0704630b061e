"""Parity on the code paths that only the long and 8B-like workloads take.

* long1m (B=1, H=4, N=2^18, d=2048, repeated 4096-token blocks) at T = 65,536:
  - the half-scores are staged in the workspace in two row chunks (the second
    starts at row 32,768);
  - the scan plan is 4 walks x 4 slices of 32 floats x 16 parts, run in two token
    chunks (54,784 + 10,752 tokens) under the ~2 GiB per-chunk bound;
  - each chunk has more than 65,536 (group, round) counts, so the bucket offsets
    come from the two-kernel wide form (bucket_totals + bucket_offsets).
* layer8b (B=4, T=8192, d=4096, H=8, N=2^20) at its full size: the half-scores
  are staged in four row chunks.

Each run goes through sdm_forward exactly as bench.py calls it (no score dump).
The kernel-timing record confirms which launches ran.  A second selection pass
that dumps the half-scores in one piece must produce the same products bit for
bit.  Sampled token rows are checked against the oracle from x (stages A, B, D),
and two whole (b, h) walks against the oracle run from the GPU's selection.
"""
import collections

import numpy as np
import pytest
import torch

from sparse_memory_linear_sdm_amd import _lib, dims_for, ops, synth
from tests.gpu_util import broadcast_state, host, layer_inputs, say
from tests.test_gpu_workloads import _sampled_rows_check, _walk_check

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    say(f"\n[gpu] {request.node.nodeid}")
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _run(wl, seed):
    h, d = layer_inputs(wl, seed=seed)
    dm = dims_for(wl)
    dm.flags = _lib.SDM_FLAG_TIMING
    state = broadcast_state(d["m0"], wl.B)
    _lib.timing_read()  # drop records of earlier calls
    out, p = ops.forward(dm, d["x"], d["w_proj"], d["A"], d["b_dt"], d["gamma"], state,
                         debug=True)
    torch.cuda.synchronize()
    launches = collections.Counter(name for name, _ in _lib.timing_read(1 << 16))
    say(f"  launches: {dict(launches)}")
    # the selection again, half-scores dumped in one piece: the same products
    q = ops.select(dims_for(wl), d["x"], d["w_proj"], d["A"], d["b_dt"], with_scores=True)
    torch.cuda.synchronize()
    for k in ops.PRODUCT_FIELDS:
        assert torch.equal(p[k], q[k]), f"{k}: staged selection differs from the one-piece run"
    return h, p, q, state, out, launches


def test_long1m_score_chunks_token_chunks_wide_offsets():
    wl = synth.small("long1m", T=65536)
    h, p, q, state, out, launches = _run(wl, seed=3)
    assert launches["proj_gemm_bf16"] == 2 and launches["select"] == 2, "score row chunks"
    assert launches["two_phase_scan"] == 2, "token chunks of the scan"
    assert launches["bucket_totals"] == 2, "wide offsets form"
    rng = np.random.default_rng(3)
    rows = np.sort(np.concatenate([rng.choice(32768, 6, replace=False),
                                   32768 + rng.choice(32768, 6, replace=False)]))
    _sampled_rows_check(wl, h, q, rows)
    _walk_check(wl, h, p, state, out, [(0, 0), (0, wl.H - 1)], h["m0"])


def test_layer8b_full_size_score_chunks():
    wl = synth.WORKLOADS["layer8b"]
    h, p, q, state, out, launches = _run(wl, seed=4)
    assert launches["proj_gemm_bf16"] == 4 and launches["select"] == 4, "score row chunks"
    rng = np.random.default_rng(4)
    rows = np.sort(rng.choice(wl.B * wl.T, 16, replace=False))
    _sampled_rows_check(wl, h, q, rows)
    _walk_check(wl, h, p, state, out, [(0, 0), (wl.B - 1, wl.H - 1)], h["m0"])


def test_long1m_full_size():
    """The long workload at its full length (T = 1,048,576, as bench.py runs it: 32
    score chunks, 20 token chunks of the two-phase scan).  A whole walk of the oracle
    would take minutes, so: 24 sampled token rows against the oracle from x (spread
    over the run, the repeated blocks included); the first 32,768 tokens of walk
    (0, 0) against the oracle's walk; the final state of all four walks bit for bit
    against the direct schedule run on the same products (the schedules agree bit for
    bit on the state, and the direct one is pinned to the oracle); out against it
    within the fp32 tolerance; rows no token wrote equal to M0 in every walk (at this
    length 64 writes per token reach every one of the 262,144 slots, so that last check
    finds none)."""
    from oracle import sdm_oracle as O
    from tests.gpu_util import assert_close

    wl = synth.WORKLOADS["long1m"]
    say("  generating the inputs")
    h, d = layer_inputs(wl, seed=5)
    dm = dims_for(wl)
    dm.flags = _lib.SDM_FLAG_TIMING
    state = broadcast_state(d["m0"], wl.B)
    _lib.timing_read()
    out, p = ops.forward(dm, d["x"], d["w_proj"], d["A"], d["b_dt"], d["gamma"], state,
                         debug=True)
    torch.cuda.synchronize()
    launches = collections.Counter(name for name, _ in _lib.timing_read(1 << 16))
    say(f"  launches: {dict(launches)}")
    assert launches["proj_gemm_bf16"] == 32 and launches["select"] == 32, "score row chunks"
    assert launches["two_phase_scan"] == 20, "token chunks of the scan"
    # sampled rows: the selection of just those rows, half-scores dumped, equals the
    # full run's products at those rows bit for bit, then stages A, B, D
    rng = np.random.default_rng(5)
    rows = np.sort(np.concatenate([rng.choice(wl.T // 2, 12, replace=False),
                                   wl.T // 2 + rng.choice(wl.T // 2, 12, replace=False)]))
    ridx = torch.as_tensor(rows, device=d["x"].device)
    xs = d["x"].reshape(-1, wl.d_model)[ridx].reshape(1, len(rows), wl.d_model).contiguous()
    ws = synth.small("long1m", T=len(rows))
    q = ops.select(dims_for(ws), xs, d["w_proj"], d["A"], d["b_dt"], with_scores=True)
    torch.cuda.synchronize()
    for k in ops.PRODUCT_FIELDS:
        assert torch.equal(q[k][0], p[k][0, ridx]), f"{k}: row selection differs"
    _sampled_rows_check(ws, dict(h, x=h["x"][:, rows]), q, np.arange(len(rows)))
    # the oracle on the first 32,768 tokens of walk (0, 0)
    K = 32768
    say("  oracle walk (0, 0), first 32768 tokens")
    sel = {k: host(p[k][0, :K, 0]) for k in ("idx_w", "wt_w", "idx_r", "wt_r", "v", "gate",
                                             "alpha", "beta")}
    sel["g"] = sel.pop("gate")
    o_out, _, _ = O.forward_walk(h["m0"][0], sel, h["gamma"][0], wl.eps)
    assert_close(host(out[0, :K, 0]), o_out, "out, walk (0, 0), first 32768 tokens")
    # the direct schedule on the same products
    say("  direct schedule over the whole run")
    dd = dims_for(wl)
    dd.flags = _lib.SDM_FLAG_SCAN_DIRECT
    st2 = broadcast_state(d["m0"], wl.B)
    out2 = ops.scan(dd, p, d["gamma"], st2)
    torch.cuda.synchronize()
    assert torch.equal(state, st2), "state differs from the direct schedule's"
    bad = int(((out - out2).abs() > 1e-5 + 1e-4 * out2.abs()).sum())
    assert bad == 0, f"out: {bad} elements beyond the fp32 tolerance of the direct schedule's"
    del st2, out2
    for hh in range(wl.H):
        written = torch.zeros(wl.N, dtype=torch.bool, device=state.device)
        written[p["idx_w"][0, :, hh].reshape(-1).long()] = True
        assert torch.equal(state[0, hh][~written], d["m0"][hh][~written]), "unwritten rows changed"
        say(f"  walk (0, {hh}): {int((~written).sum())} slots never written")
