"""The C ABI on a machine without a GPU: the library loads, exports every entry
point include/sdm.h declares, sizes workspaces, and rejects bad arguments before
anything would be enqueued (so no device is touched by these tests)."""
import ctypes
import os
import re

import pytest

from sparse_memory_linear_sdm_amd import _lib
from sparse_memory_linear_sdm_amd import synth, dims_for

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdm.h")
FAKE = 0x100000  # an address that is never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libsdm.so is not built (run __graft_entry__.build())")
    return _lib.load()


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"SDM_API\s+[\w\s\*]*?\b(sdm_\w+)\s*\(", txt)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_header_constants_match_binding():
    txt = open(HEADER).read()
    consts = dict(re.findall(r"#define (SDM_\w+) \(?(-?\d+)\)?", txt))
    for k, v in consts.items():
        if hasattr(_lib, k):
            assert getattr(_lib, k) == int(v), k


def test_version_and_status_strings(lib):
    assert _lib.abi_version() == 2
    for code in (0, -1, -2, -3, -4, -5, -6, -7, 12345):
        assert isinstance(_lib.status_string(code), str) and _lib.status_string(code)
    assert _lib.status_string(-5) == "workspace missing or too small"


def _d(**kw):
    base = dict(B=2, T=8, d_model=64, H=2, n=8, W=4, R=4, d_v=16, in_dtype=1, gate_act=1,
                eps=1e-6, flags=0)
    base.update(kw)
    return _lib.dims(**base)


def _sel(**over):
    f = {k: FAKE for k in ("idx_w", "wt_w", "idx_r", "wt_r", "v", "gate", "alpha", "beta")}
    f["scores"] = None
    f.update(over)
    return _lib.SdmSel(*[f[k] for k in ("idx_w", "wt_w", "idx_r", "wt_r", "v", "gate", "alpha",
                                        "beta", "scores")])


def _select(lib, d, x=FAKE, w=FAKE, A=FAKE, b=FAKE, sel=None, ws=FAKE, nb=1 << 40):
    sel = sel if sel is not None else _sel()
    return lib.sdm_select(ctypes.byref(d), x, w, A, b, ctypes.byref(sel), ws, nb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(H=0), _lib.SDM_ERR_SHAPE), (dict(n=0), _lib.SDM_ERR_SHAPE),
    (dict(W=0), _lib.SDM_ERR_SHAPE), (dict(R=-1), _lib.SDM_ERR_SHAPE),
    (dict(n=2, W=5), _lib.SDM_ERR_SHAPE), (dict(B=-1), _lib.SDM_ERR_SHAPE),
    (dict(eps=-1.0), _lib.SDM_ERR_SHAPE), (dict(eps=float("nan")), _lib.SDM_ERR_SHAPE),
    (dict(n=16, W=129), _lib.SDM_ERR_UNSUPPORTED), (dict(n=1025), _lib.SDM_ERR_UNSUPPORTED),
    (dict(d_v=48), _lib.SDM_ERR_UNSUPPORTED), (dict(d_model=60), _lib.SDM_ERR_UNSUPPORTED),
    (dict(flags=256), _lib.SDM_ERR_UNSUPPORTED), (dict(flags=3), _lib.SDM_ERR_SHAPE),
    (dict(flags=16 | 2), _lib.SDM_ERR_UNSUPPORTED), (dict(flags=16 | 4), _lib.SDM_ERR_UNSUPPORTED),
    (dict(flags=6), _lib.SDM_ERR_SHAPE), (dict(flags=8 | 5), _lib.SDM_ERR_SHAPE),
    (dict(in_dtype=7), _lib.SDM_ERR_DTYPE), (dict(gate_act=3), _lib.SDM_ERR_DTYPE),
])
def test_bad_dims_rejected_by_every_entry(lib, kw, code):
    d = _d(**kw)
    assert _select(lib, d) == code
    assert lib.sdm_select_from_scores(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None) == code
    s = _sel()
    assert lib.sdm_scan(ctypes.byref(d), ctypes.byref(s), None, FAKE, FAKE, None, FAKE, 1 << 40,
                        None) == code
    assert lib.sdm_forward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, FAKE,
                           1 << 40, None) == code
    assert lib.sdm_workspace_bytes(ctypes.byref(d), 2) == 0


def test_timing_flag_is_accepted_and_read_is_safe_without_records(lib):
    # the instrumentation bit combines with one schedule bit; validation still runs first
    for sched in (0, _lib.SDM_FLAG_SCAN_DIRECT, _lib.SDM_FLAG_SCAN_TWO_PHASE):
        d0, d1 = _d(T=64, flags=sched), _d(T=64, flags=sched | _lib.SDM_FLAG_TIMING)
        for entry in (_lib.SDM_ENTRY_SELECT, _lib.SDM_ENTRY_SCAN, _lib.SDM_ENTRY_FORWARD):
            assert (lib.sdm_workspace_bytes(ctypes.byref(d1), entry) ==
                    lib.sdm_workspace_bytes(ctypes.byref(d0), entry))
        assert _select(lib, d1, x=None) == _lib.SDM_ERR_NULL
    assert _lib.timing_read() == []
    assert lib.sdm_timing_read(None, 0) == 0
    assert lib.sdm_timing_read(None, 4) == _lib.SDM_ERR_NULL


def test_bf16_state_flag_is_accepted_everywhere(lib):
    # storage only: every schedule and both write rules accept it, workspaces are unchanged
    bf = _lib.SDM_FLAG_STATE_BF16
    for extra in (0, _lib.SDM_FLAG_SCAN_DIRECT, _lib.SDM_FLAG_SCAN_STREAM,
                  _lib.SDM_FLAG_SCAN_TWO_PHASE, _lib.SDM_FLAG_DELTA_GDN,
                  _lib.SDM_FLAG_DELTA_GDN | _lib.SDM_FLAG_SCAN_DIRECT):
        d0, d1 = _d(T=64, flags=extra), _d(T=64, flags=extra | bf)
        for entry in (_lib.SDM_ENTRY_SELECT, _lib.SDM_ENTRY_SCAN, _lib.SDM_ENTRY_FORWARD):
            assert (lib.sdm_workspace_bytes(ctypes.byref(d1), entry) ==
                    lib.sdm_workspace_bytes(ctypes.byref(d0), entry))
        assert lib.sdm_workspace_bytes(ctypes.byref(d1), _lib.SDM_ENTRY_FORWARD) > 0
        assert _select(lib, d1, x=None) == _lib.SDM_ERR_NULL
    d = _d(T=64, flags=bf | _lib.SDM_FLAG_DELTA_GDN | _lib.SDM_FLAG_SCAN_TWO_PHASE)
    assert _select(lib, d) == _lib.SDM_ERR_UNSUPPORTED


def test_shared_m0_entries_validate_first(lib):
    d = _d(T=64)
    s = _sel()
    # sdm_scan_shared_m0(dims, in, norm_w, m0, state, touched, out, y_raw, ws, ws_bytes, stream)
    scan = lambda m0=FAKE, st=FAKE, tch=FAKE, dd=d: lib.sdm_scan_shared_m0(
        ctypes.byref(dd), ctypes.byref(s), None, m0, st, tch, FAKE, None, FAKE, 1 << 40, None)
    assert scan(m0=None) == _lib.SDM_ERR_NULL
    assert scan(tch=None) == _lib.SDM_ERR_NULL
    assert scan(tch=FAKE + 4) == _lib.SDM_ERR_ALIGN
    assert scan(m0=FAKE + 8) == _lib.SDM_ERR_ALIGN
    assert scan(m0=None, dd=_d(T=0)) == _lib.SDM_OK          # empty call: nothing to do
    assert scan(dd=_d(H=0)) == _lib.SDM_ERR_SHAPE
    fwd = lambda m0=FAKE, tch=FAKE, dd=d: lib.sdm_forward_shared_m0(
        ctypes.byref(dd), FAKE, FAKE, FAKE, FAKE, None, m0, FAKE, tch, FAKE, FAKE, 1 << 40, None)
    assert fwd(m0=None) == _lib.SDM_ERR_NULL
    assert fwd(tch=FAKE + 2) == _lib.SDM_ERR_ALIGN
    assert fwd(tch=None, dd=_d(B=0)) == _lib.SDM_OK


def test_training_entries_validate_first(lib):
    d = _d(T=64)
    s = _sel()
    train = lambda dd=d, log=FAKE, y=FAKE, sc=None, ws=FAKE, nb=1 << 40: lib.sdm_scan_train(
        ctypes.byref(dd), ctypes.byref(s), None, FAKE, FAKE, y, log, sc, ws, nb, None)
    for bad in (_lib.SDM_FLAG_STATE_BF16, _lib.SDM_FLAG_DELTA_GDN):
        assert train(dd=_d(T=64, flags=bad), sc=FAKE) == _lib.SDM_ERR_UNSUPPORTED
    # the direct schedule needs no workspace; the stream schedule (an fp32 log from 256
    # tokens, or asked for) takes its buckets from the workspace
    assert lib.sdm_workspace_bytes(ctypes.byref(d), _lib.SDM_ENTRY_SCAN_TRAIN) == 0
    for ds in (_d(T=64, flags=_lib.SDM_FLAG_SCAN_STREAM), _d(T=256),
               _d(T=64, flags=_lib.SDM_FLAG_SCAN_TWO_PHASE)):
        nt = lib.sdm_workspace_bytes(ctypes.byref(ds), _lib.SDM_ENTRY_SCAN_TRAIN)
        assert nt > ds.B * ds.T * ds.H * (ds.W + ds.R) * 8
        assert train(dd=ds, nb=nt - 1) == _lib.SDM_ERR_WORKSPACE
        assert train(dd=ds, ws=None) == _lib.SDM_ERR_WORKSPACE
    dd = _d(T=256, flags=_lib.SDM_FLAG_SCAN_DIRECT | _lib.SDM_FLAG_LOG_INT4)
    assert lib.sdm_workspace_bytes(ctypes.byref(dd), _lib.SDM_ENTRY_SCAN_TRAIN) == 0
    # a quantised log on the stream schedule stages the fp32 rows in the workspace
    for fl in (_lib.SDM_FLAG_LOG_INT4, _lib.SDM_FLAG_LOG_FP8):
        dq = _d(T=256, flags=fl)
        nq = lib.sdm_workspace_bytes(ctypes.byref(dq), _lib.SDM_ENTRY_SCAN_TRAIN)
        n32 = lib.sdm_workspace_bytes(ctypes.byref(_d(T=256)), _lib.SDM_ENTRY_SCAN_TRAIN)
        assert nq >= n32 + dq.B * dq.T * dq.H * dq.W * dq.d_v * 4
        assert train(dd=dq, sc=FAKE, nb=nq - 1) == _lib.SDM_ERR_WORKSPACE
    assert train(log=None) == _lib.SDM_ERR_NULL
    assert train(y=None) == _lib.SDM_ERR_NULL        # the backward needs y_raw
    assert train(log=FAKE + 4) == _lib.SDM_ERR_ALIGN
    assert train(dd=_d(T=0), log=None) == _lib.SDM_OK
    fp8, int4 = _lib.SDM_FLAG_LOG_FP8, _lib.SDM_FLAG_LOG_INT4
    assert train(dd=_d(T=64, flags=fp8)) == _lib.SDM_ERR_NULL          # scales needed
    assert train(dd=_d(T=64, flags=int4), sc=FAKE + 4) == _lib.SDM_ERR_ALIGN
    assert train(dd=_d(T=64, flags=fp8 | int4), sc=FAKE) == _lib.SDM_ERR_SHAPE
    g = _lib.SdmScanGrads(*([FAKE] * 6 + [None]))
    back = lambda dd=d, grads=g, ws=FAKE, nb=1 << 40, sc=None: lib.sdm_scan_backward(
        ctypes.byref(dd), ctypes.byref(s), None, FAKE, FAKE, FAKE, FAKE, sc, FAKE,
        ctypes.byref(grads), ws, nb, None)
    assert back(dd=_d(T=64, flags=_lib.SDM_FLAG_DELTA_GDN)) == _lib.SDM_ERR_UNSUPPORTED
    assert back(grads=_lib.SdmScanGrads(*([FAKE] * 5 + [None, None]))) == _lib.SDM_ERR_NULL
    assert back(ws=None) == _lib.SDM_ERR_WORKSPACE
    assert back(dd=_d(T=64, flags=_lib.SDM_FLAG_LOG_INT4)) == _lib.SDM_ERR_NULL
    need = lib.sdm_workspace_bytes(ctypes.byref(d), _lib.SDM_ENTRY_SCAN_BACKWARD)
    assert need == d.B * d.H * d.d_v * 4
    assert back(nb=need - 1) == _lib.SDM_ERR_WORKSPACE
    assert back(grads=_lib.SdmScanGrads(*([FAKE] * 6 + [FAKE + 8]))) == _lib.SDM_ERR_ALIGN
    # the stream schedule (forced, or by default from 256 tokens) takes its buckets,
    # dy, per-slice partial dots and per-part d_v from the workspace
    for ds in (_d(T=64, flags=_lib.SDM_FLAG_SCAN_STREAM), _d(T=256),
               _d(T=64, flags=_lib.SDM_FLAG_SCAN_TWO_PHASE)):
        ns = lib.sdm_workspace_bytes(ctypes.byref(ds), _lib.SDM_ENTRY_SCAN_BACKWARD)
        assert ns > ds.B * ds.T * ds.H * (ds.W + ds.R) * 8
        assert back(dd=ds, nb=ns - 1) == _lib.SDM_ERR_WORKSPACE
    dd = _d(T=256, flags=_lib.SDM_FLAG_SCAN_DIRECT)
    assert lib.sdm_workspace_bytes(ctypes.byref(dd), _lib.SDM_ENTRY_SCAN_BACKWARD) == need


def test_null_dims(lib):
    assert lib.sdm_select(None, FAKE, FAKE, FAKE, FAKE, None, FAKE, 0, None) == _lib.SDM_ERR_NULL
    assert lib.sdm_workspace_bytes(None, 0) == 0


def test_null_and_misaligned_pointers(lib):
    d = _d()
    assert _select(lib, d, x=None) == _lib.SDM_ERR_NULL
    assert _select(lib, d, sel=_sel(wt_r=None)) == _lib.SDM_ERR_NULL
    assert _select(lib, d, x=FAKE + 4) == _lib.SDM_ERR_ALIGN
    assert _select(lib, d, sel=_sel(v=FAKE + 8)) == _lib.SDM_ERR_ALIGN
    assert _select(lib, d, sel=_sel(scores=FAKE + 2)) == _lib.SDM_ERR_ALIGN
    s = _sel()
    assert lib.sdm_scan(ctypes.byref(d), ctypes.byref(s), None, None, FAKE, None, None, 0,
                        None) == _lib.SDM_ERR_NULL
    assert lib.sdm_scan(ctypes.byref(d), ctypes.byref(s), FAKE + 4, FAKE, FAKE, None, None, 0,
                        None) == _lib.SDM_ERR_ALIGN
    assert lib.sdm_forward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, FAKE,
                           1 << 40, None) == _lib.SDM_ERR_NULL


def test_workspace_checks(lib):
    d = _d()
    need = lib.sdm_workspace_bytes(ctypes.byref(d), _lib.SDM_ENTRY_SELECT)
    assert need == 16 * 2 * 4 * 8 * 4 or need >= 16 * 2 * 4 * 8 * 4
    assert _select(lib, d, ws=None) == _lib.SDM_ERR_WORKSPACE
    assert _select(lib, d, nb=need - 1) == _lib.SDM_ERR_WORKSPACE
    fneed = lib.sdm_workspace_bytes(ctypes.byref(d), _lib.SDM_ENTRY_FORWARD)
    assert fneed > need
    assert lib.sdm_forward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, FAKE,
                           fneed - 1, None) == _lib.SDM_ERR_WORKSPACE
    assert lib.sdm_workspace_bytes(ctypes.byref(d), 99) == 0


def test_empty_calls_are_noops(lib):
    for kw in (dict(B=0), dict(T=0)):
        d = _d(**kw)
        assert _select(lib, d, x=None, ws=None, nb=0) == _lib.SDM_OK
        s = _sel()
        assert lib.sdm_scan(ctypes.byref(d), ctypes.byref(s), None, None, None, None, None, 0,
                            None) == _lib.SDM_OK
        assert lib.sdm_forward(ctypes.byref(d), None, None, None, None, None, None, None, None,
                               None, 0, None) == _lib.SDM_OK
        assert lib.sdm_workspace_bytes(ctypes.byref(d), 2) == 0


def test_workspace_sizes_of_the_workloads(lib):
    for name, wl in synth.WORKLOADS.items():
        d = dims_for(wl)
        per_th = 4 * (2 * wl.W + 2 * wl.R + 2 * wl.d_v + 2)
        fwd = lib.sdm_workspace_bytes(ctypes.byref(d), _lib.SDM_ENTRY_FORWARD)
        assert fwd >= wl.tokens * wl.H * per_th, name
        sel = lib.sdm_workspace_bytes(ctypes.byref(d), _lib.SDM_ENTRY_SELECT)
        assert 0 < sel <= (1 << 30) + 256 or sel == wl.tokens * wl.H * 16 * wl.n, name
