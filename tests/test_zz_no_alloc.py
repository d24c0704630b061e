"""sdm_forward_noalloc (workspace in the library's fixed per-GPU array) against
sdm_forward (caller's workspace) through the C ABI.

Calls in a row on the same GPU, each smaller than the one before, so that every
call after the first runs on the array the previous one left behind: two
slot-owner (two-phase) schedule calls (300 and 40 tokens), then direct-schedule
ones (12 tokens, and a one-token decode step; the library picks the direct
schedule below 16 tokens).  The state must come out bit for bit as sdm_forward
leaves it (every slot has one owner that applies its writes in token order on
both), the output within the fp32 tolerance (the two-phase schedule sums its dirty
reads with LDS float atomics, so only the summation order may differ) and, on the
direct schedule, bit for bit.
"""
import pytest
import torch

from sparse_memory_linear_sdm_amd import _lib, dims_for, ops, synth
from tests.gpu_util import assert_close, broadcast_state, host, layer_inputs, say

pytestmark = pytest.mark.gpu


def _pair(wl, seed):
    _, d = layer_inputs(wl, seed=seed)
    dm = dims_for(wl)
    assert _lib.workspace_bytes(dm, _lib.SDM_ENTRY_FORWARD) <= _lib.SDM_NOALLOC_SCRATCH_BYTES
    st_ref = broadcast_state(d["m0"], wl.B)
    st_na = st_ref.clone()
    out_ref = ops.forward(dm, d["x"], d["w_proj"], d["A"], d["b_dt"], d["gamma"], st_ref)
    out_na = torch.empty_like(out_ref)
    _lib.sdm_forward_noalloc(dm, d["x"], d["w_proj"], d["A"], d["b_dt"], d["gamma"], st_na, out_na)
    torch.cuda.synchronize()
    return st_ref, st_na, out_ref, out_na


def test_noalloc_forward_equals_forward_on_consecutive_calls():
    say("\n[gpu] sdm_forward_noalloc: calls of decreasing size on the same array")
    for k, (B, T) in enumerate([(4, 300), (2, 40), (3, 12), (16, 1)]):
        wl = synth.small("layer1p4b", B=B, T=T, d_model=256, H=2, n=24, W=16, R=16)
        st_ref, st_na, out_ref, out_na = _pair(wl, seed=20 + k)
        assert torch.equal(st_na, st_ref), f"state differs (B={B}, T={T})"
        assert_close(host(out_na), host(out_ref), f"out (B={B}, T={T})", rtol=1e-5, atol=1e-6)
        if T < 16:  # direct schedule: fixed summation order, bit for bit
            assert torch.equal(out_na, out_ref), f"out not bitwise (B={B}, T={T})"
        say(f"  B={B} T={T}: state bitwise, out within tolerance")


def test_noalloc_forward_refuses_sizes_beyond_its_array():
    wl = synth.WORKLOADS["layer1p4b"]
    dm = dims_for(wl)
    assert _lib.workspace_bytes(dm, _lib.SDM_ENTRY_FORWARD) > _lib.SDM_NOALLOC_SCRATCH_BYTES
    x = torch.empty(16, device="cuda")
    with pytest.raises(_lib.SdmError) as e:
        _lib.sdm_forward_noalloc(dm, x, x, x, x, None, x, x)
    assert e.value.code == _lib.SDM_ERR_WORKSPACE
