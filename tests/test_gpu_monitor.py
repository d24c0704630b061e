"""Slot-update histogram (sdm_slot_histogram) against the oracle: integer counts,
bit-exact.  Cases: random write sets, accumulation over two calls, the collapsed
selection, ids outside [0, N) (skipped by the kernel's own bounds check), and the
1.4B-like layer's selection at full size (B=8, T=4096, H=4, N=131044, W=64)."""
import numpy as np
import pytest
import torch

from oracle import sdm_oracle as O
from sparse_memory_linear_sdm_amd import _lib, dims_for, ops, synth
from tests.gpu_util import host, layer_inputs, random_products, say, to_dev

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


@pytest.mark.parametrize("B,T,H,n,W", [(1, 1, 1, 4, 1), (3, 50, 2, 16, 8), (2, 333, 3, 20, 64),
                                       (1, 40, 1, 12, 128)])
def test_histogram_equals_oracle_and_accumulates(B, T, H, n, W):
    rng = np.random.default_rng(B + T + W)
    p = random_products(rng, B, T, H, n, W, 1, 16)
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=1)
    ids = to_dev(p["idx_w"])
    c = ops.slot_histogram(d, ids)
    want = O.slot_update_counts(p["idx_w"], n * n)
    assert np.array_equal(host(c), want)
    ops.slot_histogram(d, ids, counts=c)
    assert np.array_equal(host(c), 2 * want)


def test_collapsed_selection_and_ids_out_of_range():
    B, T, H, n, W = 2, 30, 2, 8, 6
    same = np.array([1, 5, 9, 33, 60, 63], np.int32)
    ids = np.broadcast_to(same, (B, T, H, W)).copy()
    d = _dims(B=B, T=T, H=H, n=n, W=W, R=1)
    c = host(ops.slot_histogram(d, to_dev(ids)))
    assert np.array_equal(c, O.slot_update_counts(ids, n * n))
    assert c[:, same].min() == B * T and c.sum() == B * T * H * W
    bad = ids.copy()
    bad[0, :, 0, 0] = -1          # not counted
    bad[1, :, 1, 5] = n * n       # one past the last slot: not counted
    c = host(ops.slot_histogram(d, to_dev(bad)))
    assert c.sum() == B * T * H * W - 2 * T
    ok = bad.copy()
    ok[ok < 0] = 0
    ok[ok >= n * n] = 0
    want = O.slot_update_counts(ok, n * n)
    want[0, 0] -= T               # the -1 ids of head 0, mapped to slot 0 above
    want[1, 0] -= T               # the N ids of head 1
    assert np.array_equal(c, want)


def test_layer1p4b_selection_full_size():
    wl = synth.WORKLOADS["layer1p4b"]
    _, d = layer_inputs(wl, seed=0, with_state=False)
    dm = dims_for(wl)
    p = ops.select(dm, d["x"], d["w_proj"], d["A"], d["b_dt"])
    c = ops.slot_histogram(dm, p["idx_w"])
    torch.cuda.synchronize()
    want = O.slot_update_counts(host(p["idx_w"]), wl.N)
    assert np.array_equal(host(c), want)
    top = np.sort(want, axis=1)[:, ::-1]
    share = top[:, : wl.N // 100].sum(1) / want.sum(1)
    say(f"  writes on the most-written 1% of slots, per head: {np.round(share, 3)}")
