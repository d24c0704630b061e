"""ctypes binding of libsdm.so: argument marshalling only.

Every function here forwards to the C entry point of the same name.  Tensors are
used only as device memory (their data pointers) and the stream is torch's
current stream; all computation happens in the library's HIP kernels.  If the
library has not been built, the first call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsdm.so")

SDM_OK = 0
SDM_ERR_NULL, SDM_ERR_SHAPE, SDM_ERR_DTYPE, SDM_ERR_ALIGN = -1, -2, -3, -4
SDM_ERR_WORKSPACE, SDM_ERR_UNSUPPORTED, SDM_ERR_HIP = -5, -6, -7
SDM_DTYPE_F32, SDM_DTYPE_BF16 = 0, 1
SDM_GATE_NONE, SDM_GATE_SIGMOID, SDM_GATE_SILU = 0, 1, 2
SDM_ENTRY_SELECT, SDM_ENTRY_SCAN, SDM_ENTRY_FORWARD, SDM_ENTRY_SCAN_BACKWARD = 0, 1, 2, 3
SDM_ENTRY_SCAN_TRAIN, SDM_ENTRY_SELECT_FROM_SCORES, SDM_ENTRY_SELECT_BACKWARD = 4, 5, 6
SDM_MAX_COUNT, SDM_MAX_HALF = 128, 1024
SDM_NOALLOC_SCRATCH_BYTES = 64 << 20
SDM_FLAG_SCAN_DIRECT, SDM_FLAG_SCAN_STREAM, SDM_FLAG_SCAN_TWO_PHASE = 1, 2, 4
SDM_FLAG_TIMING = 8
SDM_FLAG_DELTA_GDN = 16
SDM_FLAG_STATE_BF16 = 32
SDM_FLAG_STATE_FP8 = 512
SDM_FLAG_LOG_FP8, SDM_FLAG_LOG_INT4 = 64, 128
SDM_FLAG_SCAN_CHUNK = 256

EXPORTS = ("sdm_abi_version", "sdm_status_string", "sdm_workspace_bytes", "sdm_select",
           "sdm_select_from_scores", "sdm_scan", "sdm_forward", "sdm_scan_shared_m0",
           "sdm_forward_shared_m0", "sdm_scan_train", "sdm_scan_backward",
           "sdm_slot_histogram", "sdm_timing_read", "sdm_forward_noalloc",
           "sdm_select_backward")


class SdmDims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("d_model", ctypes.c_int64),
                ("H", ctypes.c_int32), ("n", ctypes.c_int32), ("W", ctypes.c_int32),
                ("R", ctypes.c_int32), ("d_v", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("gate_act", ctypes.c_int32), ("eps", ctypes.c_float), ("flags", ctypes.c_int32)]


class SdmSel(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in
                ("idx_w", "wt_w", "idx_r", "wt_r", "v", "gate", "alpha", "beta", "scores")]


GRAD_FIELDS = ("d_wt_w", "d_wt_r", "d_v", "d_gate", "d_alpha", "d_beta", "d_norm_w")


class SdmScanGrads(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in GRAD_FIELDS]


SELECT_GRAD_FIELDS = ("d_wt_w", "d_wt_r", "d_v", "d_gate", "d_alpha", "d_beta")


class SdmSelectGrads(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in SELECT_GRAD_FIELDS]


class SdmKernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("ms", ctypes.c_float)]


class SdmError(RuntimeError):
    def __init__(self, code: int, text: str):
        super().__init__(f"sdm status {code}: {text}")
        self.code = code


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and type the shared library; raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run sparse_memory_linear_sdm_amd.build.build()")
    # torch carries its own HIP runtime.  Loaded first, it is the one the library binds
    # to; loaded after the library, it would be a second runtime, whose streams the
    # library's launches reject.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P, I32, I64, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.sdm_abi_version.restype = I32
    lib.sdm_abi_version.argtypes = []
    lib.sdm_status_string.restype = ctypes.c_char_p
    lib.sdm_status_string.argtypes = [I32]
    lib.sdm_workspace_bytes.restype = ctypes.c_size_t
    lib.sdm_workspace_bytes.argtypes = [P(SdmDims), I32]
    lib.sdm_select.restype = I32
    lib.sdm_select.argtypes = [P(SdmDims), VP, VP, VP, VP, P(SdmSel), VP, ctypes.c_size_t, VP]
    lib.sdm_select_from_scores.restype = I32
    lib.sdm_select_from_scores.argtypes = [P(SdmDims), VP, VP, VP, VP, VP, VP, ctypes.c_size_t,
                                           VP]
    lib.sdm_scan.restype = I32
    lib.sdm_scan.argtypes = [P(SdmDims), P(SdmSel), VP, VP, VP, VP, VP, ctypes.c_size_t, VP]
    lib.sdm_forward.restype = I32
    lib.sdm_forward.argtypes = [P(SdmDims), VP, VP, VP, VP, VP, VP, VP, P(SdmSel), VP,
                                ctypes.c_size_t, VP]
    lib.sdm_timing_read.restype = I32
    lib.sdm_timing_read.argtypes = [P(SdmKernelTime), I32]
    lib.sdm_scan_shared_m0.restype = I32
    lib.sdm_scan_shared_m0.argtypes = [P(SdmDims), P(SdmSel), VP, VP, VP, VP, VP, VP, VP,
                                       ctypes.c_size_t, VP]
    lib.sdm_forward_shared_m0.restype = I32
    lib.sdm_forward_shared_m0.argtypes = [P(SdmDims), VP, VP, VP, VP, VP, VP, VP, VP, VP, VP,
                                          ctypes.c_size_t, VP]
    lib.sdm_scan_train.restype = I32
    lib.sdm_scan_train.argtypes = [P(SdmDims), P(SdmSel), VP, VP, VP, VP, VP, VP, VP, ctypes.c_size_t,
                                   VP]
    lib.sdm_scan_backward.restype = I32
    lib.sdm_scan_backward.argtypes = [P(SdmDims), P(SdmSel), VP, VP, VP, VP, VP, VP, VP,
                                      P(SdmScanGrads), VP, ctypes.c_size_t, VP]
    lib.sdm_select_backward.restype = I32
    lib.sdm_select_backward.argtypes = [P(SdmDims), P(SdmSel), VP, VP, VP, VP, P(SdmSelectGrads),
                                        VP, VP, VP, VP, ctypes.c_size_t, VP]
    lib.sdm_forward_noalloc.restype = I32
    lib.sdm_forward_noalloc.argtypes = [P(SdmDims), VP, VP, VP, VP, VP, VP, VP, VP]
    lib.sdm_slot_histogram.restype = I32
    lib.sdm_slot_histogram.argtypes = [P(SdmDims), VP, VP, VP]
    del I64
    _lib = lib
    return lib


def dims(B, T, d_model, H, n, W, R, d_v, in_dtype=SDM_DTYPE_BF16, gate_act=SDM_GATE_SIGMOID,
         eps=1e-6, flags=0) -> SdmDims:
    return SdmDims(B, T, d_model, H, n, W, R, d_v, in_dtype, gate_act, eps, flags)


def _ptr(t):
    """Device address of a tensor (or None / a plain int address)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(code: int):
    if code != SDM_OK:
        raise SdmError(code, load().sdm_status_string(code).decode())


def sel_struct(idx_w, wt_w, idx_r, wt_r, v, gate, alpha, beta, scores=None) -> SdmSel:
    return SdmSel(*[_ptr(t) for t in (idx_w, wt_w, idx_r, wt_r, v, gate, alpha, beta, scores)])


def abi_version() -> int:
    return load().sdm_abi_version()


def status_string(code: int) -> str:
    return load().sdm_status_string(code).decode()


def workspace_bytes(d: SdmDims, entry: int) -> int:
    return load().sdm_workspace_bytes(ctypes.byref(d), entry)


def sdm_select(d: SdmDims, x, w_proj, A, b_dt, out: SdmSel, ws=None, ws_bytes=0, stream=None):
    _check(load().sdm_select(ctypes.byref(d), _ptr(x), _ptr(w_proj), _ptr(A), _ptr(b_dt),
                             ctypes.byref(out), _ptr(ws), ws_bytes, _stream(stream)))


def sdm_select_from_scores(d: SdmDims, scores, idx_w, wt_w, idx_r, wt_r, ws=None, ws_bytes=0,
                           stream=None):
    _check(load().sdm_select_from_scores(ctypes.byref(d), _ptr(scores), _ptr(idx_w), _ptr(wt_w),
                                         _ptr(idx_r), _ptr(wt_r), _ptr(ws), ws_bytes,
                                         _stream(stream)))


def sdm_scan(d: SdmDims, inp: SdmSel, norm_w, state, out, y_raw=None, ws=None, ws_bytes=0,
             stream=None):
    _check(load().sdm_scan(ctypes.byref(d), ctypes.byref(inp), _ptr(norm_w), _ptr(state),
                           _ptr(out), _ptr(y_raw), _ptr(ws), ws_bytes, _stream(stream)))


def sdm_forward(d: SdmDims, x, w_proj, A, b_dt, norm_w, state, out, debug: SdmSel | None = None,
                ws=None, ws_bytes=0, stream=None):
    _check(load().sdm_forward(ctypes.byref(d), _ptr(x), _ptr(w_proj), _ptr(A), _ptr(b_dt),
                              _ptr(norm_w), _ptr(state), _ptr(out),
                              ctypes.byref(debug) if debug is not None else None, _ptr(ws),
                              ws_bytes, _stream(stream)))


def sdm_select_backward(d: SdmDims, fwd: SdmSel, x, w_proj, A, b_dt, grads: SdmSelectGrads,
                        d_y, d_A, d_b_dt, ws=None, ws_bytes=0, stream=None):
    _check(load().sdm_select_backward(ctypes.byref(d), ctypes.byref(fwd), _ptr(x), _ptr(w_proj),
                                      _ptr(A), _ptr(b_dt), ctypes.byref(grads), _ptr(d_y),
                                      _ptr(d_A), _ptr(d_b_dt), _ptr(ws), ws_bytes,
                                      _stream(stream)))


def sdm_forward_noalloc(d: SdmDims, x, w_proj, A, b_dt, norm_w, state, out, stream=None):
    _check(load().sdm_forward_noalloc(ctypes.byref(d), _ptr(x), _ptr(w_proj), _ptr(A), _ptr(b_dt),
                                      _ptr(norm_w), _ptr(state), _ptr(out), _stream(stream)))


def sdm_scan_shared_m0(d: SdmDims, inp: SdmSel, norm_w, m0, state, touched, out, y_raw=None,
                       ws=None, ws_bytes=0, stream=None):
    _check(load().sdm_scan_shared_m0(ctypes.byref(d), ctypes.byref(inp), _ptr(norm_w), _ptr(m0),
                                     _ptr(state), _ptr(touched), _ptr(out), _ptr(y_raw), _ptr(ws),
                                     ws_bytes, _stream(stream)))


def sdm_forward_shared_m0(d: SdmDims, x, w_proj, A, b_dt, norm_w, m0, state, touched, out,
                          ws=None, ws_bytes=0, stream=None):
    _check(load().sdm_forward_shared_m0(ctypes.byref(d), _ptr(x), _ptr(w_proj), _ptr(A),
                                        _ptr(b_dt), _ptr(norm_w), _ptr(m0), _ptr(state),
                                        _ptr(touched), _ptr(out), _ptr(ws), ws_bytes,
                                        _stream(stream)))


def sdm_scan_train(d: SdmDims, inp: SdmSel, norm_w, state, out, y_raw, log, log_scale=None,
                   ws=None, ws_bytes=0, stream=None):
    _check(load().sdm_scan_train(ctypes.byref(d), ctypes.byref(inp), _ptr(norm_w), _ptr(state),
                                 _ptr(out), _ptr(y_raw), _ptr(log), _ptr(log_scale), _ptr(ws),
                                 ws_bytes, _stream(stream)))


def sdm_scan_backward(d: SdmDims, inp: SdmSel, norm_w, state, d_state, y_raw, log, log_scale,
                      d_out, grads: SdmScanGrads, ws=None, ws_bytes=0, stream=None):
    _check(load().sdm_scan_backward(ctypes.byref(d), ctypes.byref(inp), _ptr(norm_w),
                                    _ptr(state), _ptr(d_state), _ptr(y_raw), _ptr(log),
                                    _ptr(log_scale), _ptr(d_out), ctypes.byref(grads), _ptr(ws),
                                    ws_bytes, _stream(stream)))


def sdm_slot_histogram(d: SdmDims, idx_w, counts, stream=None):
    _check(load().sdm_slot_histogram(ctypes.byref(d), _ptr(idx_w), _ptr(counts), _stream(stream)))


def timing_read(max_records: int = 4096) -> list:
    """[(kernel name, ms)] of launches recorded under SDM_FLAG_TIMING, oldest first."""
    buf = (SdmKernelTime * max_records)()
    n = load().sdm_timing_read(buf, max_records)
    if n < 0:
        raise SdmError(n, load().sdm_status_string(n).decode())
    return [(buf[i].name.decode(), float(buf[i].ms)) for i in range(n)]
