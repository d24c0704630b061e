"""sdm_forward captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

The ABI promises that calls may be captured: nothing in a call allocates,
synchronises or clears memory with a memset.  Each replay continues from the
state the previous one left, exactly as repeated eager calls do, so every replay
is checked against an eager run advanced in lock-step (state bitwise, outputs
within fp32 tolerance); eager work and host synchronisations sit between the
replays.
"""
import numpy as np
import pytest
import torch

from sparse_memory_linear_sdm_amd import _lib, dims_for, ops, synth
from tests.gpu_util import assert_close, broadcast_state, host, layer_inputs, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,B,T", [("decode256", 16, 1), ("layer1p4b", 2, 300)])
def test_forward_graph_replays_match_eager(name, B, T):
    say(f"\n[gpu] graph capture {name} B={B} T={T}")
    wl = synth.small(name, B=B, T=T, d_model=256, H=2, n=24)
    _, d = layer_inputs(wl, seed=9)
    dm = dims_for(wl)
    dev = d["x"].device
    ws = torch.empty(max(_lib.workspace_bytes(dm, _lib.SDM_ENTRY_FORWARD), 1), dtype=torch.uint8,
                     device=dev)
    st_e = broadcast_state(d["m0"], wl.B)
    st_g = st_e.clone()
    out_e = torch.empty((wl.B, wl.T, wl.H, wl.d_v), device=dev)
    out_g = torch.empty_like(out_e)
    args = (d["x"], d["w_proj"], d["A"], d["b_dt"], d["gamma"])

    # warm-up on a side stream (torch's capture protocol), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        scratch = st_g.clone()
        ops.forward(dm, *args, scratch, out=torch.empty_like(out_g), ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ops.forward(dm, *args, st_g, out=out_g, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(st_g, st_e), "capture must not have run the kernels"

    for k in range(4):
        graph.replay()
        ops.forward(dm, *args, st_e, out=out_e, ws=torch.empty_like(ws))
        junk = torch.randn(1024, device=dev).sum()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(st_g, st_e), f"state after replay {k}"
        assert_close(host(out_g), host(out_e), f"out after replay {k}", rtol=1e-5, atol=1e-6)
        say(f"  replay {k}: state identical, out within tolerance")
