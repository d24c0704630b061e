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
    assert _lib.abi_version() == 4
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
    (dict(flags=1024), _lib.SDM_ERR_UNSUPPORTED), (dict(flags=3), _lib.SDM_ERR_SHAPE),
    (dict(flags=512), _lib.SDM_ERR_UNSUPPORTED),                 # fp8 state with d_v = 16
    (dict(flags=512 | 32, d_v=32), _lib.SDM_ERR_SHAPE),          # two storage formats
    (dict(flags=512 | 16, d_v=32), _lib.SDM_ERR_UNSUPPORTED),    # fp8: per-slot rule only
    (dict(flags=512 | 2, d_v=32), _lib.SDM_ERR_UNSUPPORTED),     # fp8: not the stream schedule
    (dict(flags=512 | 256, d_v=32), _lib.SDM_ERR_UNSUPPORTED),   # nor the chunk schedule
    (dict(flags=256 | 1), _lib.SDM_ERR_SHAPE), (dict(flags=256 | 32), _lib.SDM_ERR_UNSUPPORTED),
    (dict(flags=16 | 2), _lib.SDM_ERR_UNSUPPORTED), (dict(flags=16 | 4), _lib.SDM_ERR_UNSUPPORTED),
    (dict(flags=6), _lib.SDM_ERR_SHAPE), (dict(flags=8 | 5), _lib.SDM_ERR_SHAPE),
    (dict(in_dtype=7), _lib.SDM_ERR_DTYPE), (dict(gate_act=3), _lib.SDM_ERR_DTYPE),
])
def test_bad_dims_rejected_by_every_entry(lib, kw, code):
    d = _d(**kw)
    assert _select(lib, d) == code
    assert lib.sdm_select_from_scores(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, 0,
                                      None) == code
    s = _sel()
    assert lib.sdm_scan(ctypes.byref(d), ctypes.byref(s), None, FAKE, FAKE, None, FAKE, 1 << 40,
                        None) == code
    assert lib.sdm_forward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, FAKE,
                           1 << 40, None) == code
    assert lib.sdm_workspace_bytes(ctypes.byref(d), 2) == 0


def test_select_from_scores_needs_no_workspace(lib):
    d = _d()
    assert lib.sdm_workspace_bytes(ctypes.byref(d), _lib.SDM_ENTRY_SELECT_FROM_SCORES) == 0
    # a workspace may still be passed; a misaligned one is rejected before any launch
    assert lib.sdm_select_from_scores(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 4, 64,
                                      None) == _lib.SDM_ERR_ALIGN
    assert lib.sdm_select_from_scores(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, None, 0,
                                      None) == _lib.SDM_ERR_NULL


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
        # 32 tokens: the key-weighted rule takes its sliced walk with either storage
        d0, d1 = _d(T=32, flags=extra), _d(T=32, flags=extra | bf)
        for entry in (_lib.SDM_ENTRY_SELECT, _lib.SDM_ENTRY_SCAN, _lib.SDM_ENTRY_FORWARD):
            assert (lib.sdm_workspace_bytes(ctypes.byref(d1), entry) ==
                    lib.sdm_workspace_bytes(ctypes.byref(d0), entry))
        assert lib.sdm_workspace_bytes(ctypes.byref(d1), _lib.SDM_ENTRY_FORWARD) > 0
        assert _select(lib, d1, x=None) == _lib.SDM_ERR_NULL
    d = _d(T=64, flags=bf | _lib.SDM_FLAG_DELTA_GDN | _lib.SDM_FLAG_SCAN_TWO_PHASE)
    assert _select(lib, d) == _lib.SDM_ERR_UNSUPPORTED
    # from 64 tokens the key-weighted rule's default is the chunk walk, which keeps an
    # fp32 state: a bf16 state stays on the sliced walk
    gdn = _lib.SDM_FLAG_DELTA_GDN
    ws = lambda fl: lib.sdm_workspace_bytes(ctypes.byref(_d(T=64, flags=fl)), _lib.SDM_ENTRY_SCAN)
    assert ws(gdn | bf) == ws(gdn | bf | _lib.SDM_FLAG_SCAN_DIRECT) != ws(gdn)
    assert ws(gdn) == ws(gdn | _lib.SDM_FLAG_SCAN_CHUNK)


def test_fp8_state_flag(lib):
    # storage only: the two-phase and direct schedules accept it with unchanged workspaces
    f8 = _lib.SDM_FLAG_STATE_FP8
    for extra in (0, _lib.SDM_FLAG_SCAN_DIRECT, _lib.SDM_FLAG_SCAN_TWO_PHASE):
        for T in (8, 300):
            d0, d1 = _d(T=T, d_v=32, flags=extra), _d(T=T, d_v=32, flags=extra | f8)
            for entry in (_lib.SDM_ENTRY_SELECT, _lib.SDM_ENTRY_SCAN, _lib.SDM_ENTRY_FORWARD):
                assert (lib.sdm_workspace_bytes(ctypes.byref(d1), entry) ==
                        lib.sdm_workspace_bytes(ctypes.byref(d0), entry))
            assert _select(lib, d1, x=None) == _lib.SDM_ERR_NULL
    d = _d(T=64, d_v=32, flags=f8)
    s = _sel()
    # not in training (the log and its reverse walk keep fp32 state) ...
    assert lib.sdm_scan_train(ctypes.byref(d), ctypes.byref(s), None, FAKE, FAKE, FAKE, FAKE,
                              None, FAKE, 1 << 40, None) == _lib.SDM_ERR_UNSUPPORTED
    g = _lib.SdmScanGrads(*([FAKE] * 6 + [None]))
    assert lib.sdm_scan_backward(ctypes.byref(d), ctypes.byref(s), None, FAKE, FAKE, FAKE, FAKE,
                                 None, FAKE, ctypes.byref(g), FAKE, 1 << 40,
                                 None) == _lib.SDM_ERR_UNSUPPORTED
    # ... nor with a shared initial state (its rows are copied in the fp32/bf16 layouts)
    assert lib.sdm_scan_shared_m0(ctypes.byref(d), ctypes.byref(s), None, FAKE, FAKE, FAKE, FAKE,
                                  None, FAKE, 1 << 40, None) == _lib.SDM_ERR_UNSUPPORTED
    assert lib.sdm_forward_shared_m0(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                                     FAKE, FAKE, FAKE, 1 << 40, None) == _lib.SDM_ERR_UNSUPPORTED


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
    assert train(dd=_d(T=64, flags=_lib.SDM_FLAG_STATE_BF16), sc=FAKE) == _lib.SDM_ERR_UNSUPPORTED
    # the key-weighted rule trains on the direct and chunk schedules: the chunk one by
    # default from 64 tokens with an fp32 log (its workspace), else the direct one
    gdn = _lib.SDM_FLAG_DELTA_GDN
    for fl in (_lib.SDM_FLAG_SCAN_STREAM, _lib.SDM_FLAG_SCAN_TWO_PHASE):
        assert train(dd=_d(T=64, flags=gdn | fl)) == _lib.SDM_ERR_UNSUPPORTED
    assert train(dd=_d(T=512, flags=gdn), log=None) == _lib.SDM_ERR_NULL
    ws_of = lambda dd: lib.sdm_workspace_bytes(ctypes.byref(dd), _lib.SDM_ENTRY_SCAN_TRAIN)
    assert ws_of(_d(T=512, flags=gdn)) == ws_of(_d(T=512, flags=gdn | _lib.SDM_FLAG_SCAN_CHUNK)) > 0
    assert ws_of(_d(T=64, flags=gdn)) == ws_of(_d(T=64, flags=gdn | _lib.SDM_FLAG_SCAN_CHUNK)) > 0
    assert ws_of(_d(T=63, flags=gdn)) == 0
    assert ws_of(_d(T=512, flags=gdn | _lib.SDM_FLAG_LOG_INT4)) == \
        ws_of(_d(T=512, flags=gdn | _lib.SDM_FLAG_LOG_INT4 | _lib.SDM_FLAG_SCAN_DIRECT))
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
    assert back(dd=_d(T=64, flags=_lib.SDM_FLAG_DELTA_GDN), ws=None) == _lib.SDM_ERR_WORKSPACE
    # its reverse walks (chunkwise from 256 tokens, else sliced): dy and every slice's
    # share of the dot products (one slice at d_v = 16) come from the workspace
    dg = _d(T=512, flags=_lib.SDM_FLAG_DELTA_GDN)
    ng = lib.sdm_workspace_bytes(ctypes.byref(dg), _lib.SDM_ENTRY_SCAN_BACKWARD)
    assert ng >= dg.B * dg.T * dg.H * (dg.d_v * 4 + dg.R * 4 + dg.W * 8 + 4)
    assert back(dd=dg, nb=ng - 1) == _lib.SDM_ERR_WORKSPACE
    # which reverse walk: the chunk one from 256 tokens (or with the chunk flag) with an
    # fp32 log and W, R <= 64, each walk with a workspace of its own size
    gdn, chunk, direct = (_lib.SDM_FLAG_DELTA_GDN, _lib.SDM_FLAG_SCAN_CHUNK,
                          _lib.SDM_FLAG_SCAN_DIRECT)
    bw = lambda **kw: lib.sdm_workspace_bytes(ctypes.byref(_d(**kw)), _lib.SDM_ENTRY_SCAN_BACKWARD)
    assert bw(T=512, flags=gdn | chunk) == ng != bw(T=512, flags=gdn | direct)
    assert bw(T=255, flags=gdn) == bw(T=255, flags=gdn | direct) != bw(T=255, flags=gdn | chunk)
    for fmt in (_lib.SDM_FLAG_LOG_FP8, _lib.SDM_FLAG_LOG_INT4):
        assert bw(T=512, flags=gdn | fmt) == bw(T=512, flags=gdn | direct | fmt)
    assert bw(T=512, W=65, flags=gdn) == bw(T=512, W=65, flags=gdn | direct)
    assert bw(T=512, R=65, flags=gdn | chunk) == bw(T=512, R=65, flags=gdn | direct)
    # by default the chunk walks run while their (walk, 16-column slice) workgroups are
    # few enough: at most 256 for the reverse walk, 1024 for the forward walks
    big = dict(T=512, d_v=128, H=4)
    assert bw(B=8, flags=gdn, **big) != bw(B=8, flags=gdn | direct, **big)       # 256
    assert bw(B=16, flags=gdn, **big) == bw(B=16, flags=gdn | direct, **big)     # 512
    assert bw(B=16, flags=gdn | chunk, **big) != bw(B=16, flags=gdn | direct, **big)
    for entry in (_lib.SDM_ENTRY_SCAN, _lib.SDM_ENTRY_SCAN_TRAIN):
        fw = lambda **kw: lib.sdm_workspace_bytes(ctypes.byref(_d(**kw)), entry)
        assert fw(B=32, flags=gdn, **big) == fw(B=32, flags=gdn | chunk, **big)   # 1024
        assert fw(B=64, flags=gdn, **big) == fw(B=64, flags=gdn | direct, **big)  # 2048
        assert fw(B=64, flags=gdn | chunk, **big) != fw(B=64, flags=gdn | direct, **big)
    # 8 slices of 16 columns for 2 x 2 walks of d_v = 128: 8 shares per dot product
    dg8 = _d(T=64, d_v=128, flags=_lib.SDM_FLAG_DELTA_GDN)
    ng8 = lib.sdm_workspace_bytes(ctypes.byref(dg8), _lib.SDM_ENTRY_SCAN_BACKWARD)
    assert ng8 >= dg8.B * dg8.T * dg8.H * (128 * 4 + 8 * (dg8.R * 4 + dg8.W * 8 + 4))
    # its inference walk keeps the raw read vectors for the norm pass (8 slices)
    assert lib.sdm_workspace_bytes(ctypes.byref(dg8), _lib.SDM_ENTRY_SCAN) >= \
        dg8.B * dg8.T * dg8.H * 128 * 4
    assert lib.sdm_workspace_bytes(ctypes.byref(_d(T=63, flags=_lib.SDM_FLAG_DELTA_GDN)),
                                   _lib.SDM_ENTRY_SCAN) == 0
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


def test_default_scan_schedule_by_walks(lib):
    # the per-slot rule's slot-owner schedules (with their bucketing workspace) from 16
    # tokens, the direct one (no workspace) below that or from 512 walks; the training
    # forward's two-phase one from 256 tokens below 512 walks
    ws = lambda **kw: lib.sdm_workspace_bytes(ctypes.byref(_d(**kw)), _lib.SDM_ENTRY_SCAN)
    assert ws(B=64, H=4, T=64) > 0 and ws(B=255, H=2, T=64) > 0
    assert ws(B=128, H=4, T=64) == 0 and ws(B=512, H=4, T=512) == 0
    assert ws(B=256, H=4, T=64, flags=_lib.SDM_FLAG_SCAN_TWO_PHASE) > 0
    assert ws(B=2, H=2, T=15) == 0
    tw = lambda **kw: lib.sdm_workspace_bytes(ctypes.byref(_d(**kw)), _lib.SDM_ENTRY_SCAN_TRAIN)
    assert tw(B=64, H=4, T=256) > 0
    assert tw(B=128, H=4, T=256) == 0


def test_default_backward_schedule_by_walks(lib):
    # the per-slot reverse walk: slot-owner (its workspace holds buckets and partial
    # dots) from 256 tokens while B H < 512, else the direct one (d_gamma partials only)
    bw = lambda **kw: lib.sdm_workspace_bytes(ctypes.byref(_d(**kw)), _lib.SDM_ENTRY_SCAN_BACKWARD)
    direct = lambda B, H, d_v=16: B * H * d_v * 4
    assert bw(B=64, H=4, T=512) > direct(64, 4)
    assert bw(B=128, H=4, T=512) == direct(128, 4)
    assert bw(B=128, H=4, T=512, flags=_lib.SDM_FLAG_SCAN_STREAM) > direct(128, 4)
    assert bw(B=2, H=2, T=255) == direct(2, 2)


def test_workspace_sizes_of_the_workloads(lib):
    for name, wl in synth.WORKLOADS.items():
        d = dims_for(wl)
        per_th = 4 * (2 * wl.W + 2 * wl.R + 2 * wl.d_v + 2)
        fwd = lib.sdm_workspace_bytes(ctypes.byref(d), _lib.SDM_ENTRY_FORWARD)
        assert fwd >= wl.tokens * wl.H * per_th, name
        sel = lib.sdm_workspace_bytes(ctypes.byref(d), _lib.SDM_ENTRY_SELECT)
        assert 0 < sel <= (1 << 30) + 256 or sel == wl.tokens * wl.H * 16 * wl.n, name


def test_noalloc_forward_validates_before_touching_the_device(lib):
    fwd = lambda d, x=FAKE: lib.sdm_forward_noalloc(ctypes.byref(d), x, FAKE, FAKE, FAKE, None,
                                                    FAKE, FAKE, None)
    assert fwd(_d(H=0)) == _lib.SDM_ERR_SHAPE
    assert fwd(_d(flags=_lib.SDM_FLAG_TIMING)) == _lib.SDM_ERR_UNSUPPORTED
    assert fwd(_d(), x=None) == _lib.SDM_ERR_NULL
    assert fwd(_d(), x=FAKE + 8) == _lib.SDM_ERR_ALIGN
    assert fwd(_d(B=0)) == _lib.SDM_OK                      # empty call: nothing enqueued
    # sizes whose forward workspace exceeds the fixed array are refused
    big = _d(B=8, T=4096, d_model=2048, H=4, n=362, W=64, R=64, d_v=128)
    assert lib.sdm_workspace_bytes(ctypes.byref(big), _lib.SDM_ENTRY_FORWARD) > \
        _lib.SDM_NOALLOC_SCRATCH_BYTES
    assert fwd(big) == _lib.SDM_ERR_WORKSPACE
    # the decode step (256 sequences x 1 token, N = 65536) fits
    dec = _d(B=256, T=1, d_model=2048, H=4, n=256, W=64, R=64, d_v=128)
    assert lib.sdm_workspace_bytes(ctypes.byref(dec), _lib.SDM_ENTRY_FORWARD) <= \
        _lib.SDM_NOALLOC_SCRATCH_BYTES


def test_select_backward_validates_first(lib):
    s = _sel()
    g = _lib.SdmSelectGrads(*([FAKE] * 6))
    back = lambda dd, fwd=s, grads=g, x=FAKE, dy=FAKE, ws=FAKE, nb=1 << 40: \
        lib.sdm_select_backward(ctypes.byref(dd), ctypes.byref(fwd), x, FAKE, FAKE, FAKE,
                                ctypes.byref(grads), dy, FAKE, FAKE, ws, nb, None)
    d = _d(T=64)
    # every gate activation is taken (SiLU's pre-activation is recomputed)
    assert back(_d(T=64, gate_act=_lib.SDM_GATE_SILU), x=None) == _lib.SDM_ERR_NULL
    assert back(d, x=None) == _lib.SDM_ERR_NULL
    assert back(d, dy=None) == _lib.SDM_ERR_NULL
    assert back(d, fwd=_sel(gate=None)) == _lib.SDM_ERR_NULL
    assert back(d, grads=_lib.SdmSelectGrads(*([FAKE] * 5 + [None]))) == _lib.SDM_ERR_NULL
    assert back(d, x=FAKE + 2) == _lib.SDM_ERR_ALIGN
    assert back(d, grads=_lib.SdmSelectGrads(*([FAKE] * 2 + [FAKE + 4] + [FAKE] * 3))) == \
        _lib.SDM_ERR_ALIGN
    need = lib.sdm_workspace_bytes(ctypes.byref(d), _lib.SDM_ENTRY_SELECT_BACKWARD)
    assert need >= d.B * d.T * d.H * 2 * 4
    assert back(d, ws=None) == _lib.SDM_ERR_WORKSPACE
    assert back(d, nb=need - 1) == _lib.SDM_ERR_WORKSPACE
    assert back(d, ws=FAKE + 8) == _lib.SDM_ERR_ALIGN
    assert back(_d(T=0), x=None, dy=None, ws=None, nb=0) == _lib.SDM_OK
    assert back(_d(H=0)) == _lib.SDM_ERR_SHAPE


def test_chunk_schedule_flag(lib):
    chunk, gdn = _lib.SDM_FLAG_SCAN_CHUNK, _lib.SDM_FLAG_DELTA_GDN
    d = _d(T=100, flags=chunk)
    need = lib.sdm_workspace_bytes(ctypes.byref(d), _lib.SDM_ENTRY_SCAN)
    # per token and head: L and links of the writes, L of the reads, y; per chunk A
    th = d.B * d.T * d.H
    assert need >= th * (2 * d.W + d.R + d.d_v) * 4 + d.B * d.H * 4 * 32 * 32 * 4
    assert lib.sdm_workspace_bytes(ctypes.byref(d), _lib.SDM_ENTRY_FORWARD) > need
    # the key-weighted rule adds the solve's matrices; it takes the schedule by default
    # from 64 tokens with an fp32 state, and not with a bf16 one or the direct flag
    dg = _d(T=100, flags=chunk | gdn)
    assert lib.sdm_workspace_bytes(ctypes.byref(dg), _lib.SDM_ENTRY_SCAN) > need
    assert lib.sdm_workspace_bytes(ctypes.byref(_d(T=64, flags=gdn)), _lib.SDM_ENTRY_SCAN) > 0
    assert lib.sdm_workspace_bytes(ctypes.byref(_d(T=63, flags=gdn)), _lib.SDM_ENTRY_SCAN) == 0
    for fl in (gdn | _lib.SDM_FLAG_SCAN_DIRECT, gdn | _lib.SDM_FLAG_STATE_BF16):
        assert lib.sdm_workspace_bytes(ctypes.byref(_d(T=512, flags=fl)), _lib.SDM_ENTRY_SCAN) == 0
    s = _sel()
    scan = lambda dd, ws=FAKE, nb=1 << 40: lib.sdm_scan(ctypes.byref(dd), ctypes.byref(s), None,
                                                        FAKE, FAKE, None, ws, nb, None)
    assert scan(d, ws=None) == _lib.SDM_ERR_WORKSPACE
    assert scan(d, nb=need - 1) == _lib.SDM_ERR_WORKSPACE
    assert scan(_d(T=100, flags=chunk | _lib.SDM_FLAG_STATE_BF16)) == _lib.SDM_ERR_UNSUPPORTED
    assert scan(_d(T=100, flags=chunk | _lib.SDM_FLAG_SCAN_TWO_PHASE)) == _lib.SDM_ERR_SHAPE
    # the training entries take it with an fp32 log only (its walk logs fp32 rows), and
    # size their workspace as the inference scan
    for lf in (_lib.SDM_FLAG_LOG_FP8, _lib.SDM_FLAG_LOG_INT4):
        assert lib.sdm_scan_train(ctypes.byref(_d(T=100, flags=chunk | lf)), ctypes.byref(s),
                                  None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                                  None) == _lib.SDM_ERR_UNSUPPORTED
    assert lib.sdm_workspace_bytes(ctypes.byref(d), _lib.SDM_ENTRY_SCAN_TRAIN) == need
    assert lib.sdm_scan_train(ctypes.byref(d), ctypes.byref(s), None, FAKE, FAKE, FAKE, FAKE,
                              None, None, 0, None) == _lib.SDM_ERR_WORKSPACE
