"""Tensor-level calls of the SDM forward path.

Each function checks dtypes/devices/contiguity, allocates the outputs (and the
workspace, unless one is passed) with torch, and calls the C entry point of the
same name in libsdm.so.  Nothing here computes any part of the method.
"""
from __future__ import annotations

import contextlib
import functools

import torch

from . import _lib
from ._lib import SdmDims

PRODUCT_FIELDS = ("idx_w", "wt_w", "idx_r", "wt_r", "v", "gate", "alpha", "beta")


def _stream_ctx(stream):
    if stream is None:
        return contextlib.nullcontext()
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(stream)
    return torch.cuda.stream(s)


def _on_stream(fn):
    """Run the call with `stream` (when given) as torch's current stream, so that every
    tensor it allocates (outputs, workspace) belongs to the stream its kernels run on:
    the caching allocator then reuses that memory only after the stream's work."""
    @functools.wraps(fn)
    def call(*args, stream=None, **kw):
        with _stream_ctx(stream):
            return fn(*args, stream=stream, **kw)
    return call


def _need(t, dtype, shape, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def in_dtype(d: SdmDims):
    return torch.bfloat16 if d.in_dtype == _lib.SDM_DTYPE_BF16 else torch.float32


def alloc_products(d: SdmDims, device, with_scores=False) -> dict:
    B, T, H = d.B, d.T, d.H
    e = lambda *s, dt=torch.float32: torch.empty(s, dtype=dt, device=device)
    p = dict(idx_w=e(B, T, H, d.W, dt=torch.int32), wt_w=e(B, T, H, d.W),
             idx_r=e(B, T, H, d.R, dt=torch.int32), wt_r=e(B, T, H, d.R),
             v=e(B, T, H, d.d_v), gate=e(B, T, H, d.d_v), alpha=e(B, T, H), beta=e(B, T, H))
    if with_scores:
        p["scores"] = e(B, T, H, 4 * d.n)
    return p


def _sel(p: dict) -> _lib.SdmSel:
    return _lib.sel_struct(*(p[k] for k in PRODUCT_FIELDS), p.get("scores"))


def _check_params(d: SdmDims, x, w_proj, A, b_dt):
    P = 4 * d.n + 2 * d.d_v + 2
    _need(x, in_dtype(d), (d.B, d.T, d.d_model), "x")
    _need(w_proj, in_dtype(d), (d.H * P, d.d_model), "w_proj")
    _need(A, torch.float32, (d.H,), "A")
    _need(b_dt, torch.float32, (d.H,), "b_dt")


def _check_products(d: SdmDims, p: dict):
    shapes = dict(idx_w=(d.W,), wt_w=(d.W,), idx_r=(d.R,), wt_r=(d.R,), v=(d.d_v,),
                  gate=(d.d_v,), alpha=(), beta=())
    for k in PRODUCT_FIELDS:
        dt = torch.int32 if k.startswith("idx") else torch.float32
        _need(p[k], dt, (d.B, d.T, d.H) + shapes[k], k)


def _workspace(d: SdmDims, entry: int, device, ws=None):
    need = _lib.workspace_bytes(d, entry)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    elif ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace of {need} bytes needed")
    return ws, ws.numel() * ws.element_size()


@_on_stream
def select(d: SdmDims, x, w_proj, A, b_dt, with_scores=False, out=None, ws=None, stream=None):
    _check_params(d, x, w_proj, A, b_dt)
    p = out if out is not None else alloc_products(d, x.device, with_scores)
    _check_products(d, p)
    ws, nb = _workspace(d, _lib.SDM_ENTRY_SELECT, x.device, ws)
    _lib.sdm_select(d, x, w_proj, A, b_dt, _sel(p), ws, nb, stream)
    return p


@_on_stream
def select_from_scores(d: SdmDims, scores, stream=None):
    _need(scores, torch.float32, (d.B, d.T, d.H, 4 * d.n), "scores")
    p = alloc_products(d, scores.device)
    ws, nb = _workspace(d, _lib.SDM_ENTRY_SELECT_FROM_SCORES, scores.device)
    _lib.sdm_select_from_scores(d, scores, p["idx_w"], p["wt_w"], p["idx_r"], p["wt_r"], ws, nb,
                                stream)
    return {k: p[k] for k in ("idx_w", "wt_w", "idx_r", "wt_r")}


def state_dtype(d: SdmDims):
    if d.flags & _lib.SDM_FLAG_STATE_FP8:
        return torch.uint8
    return torch.bfloat16 if d.flags & _lib.SDM_FLAG_STATE_BF16 else torch.float32


def state_shape(d: SdmDims):
    """[B, H, N, d_v], or with SDM_FLAG_STATE_FP8 the byte count of its two planes."""
    N = d.n * d.n
    if d.flags & _lib.SDM_FLAG_STATE_FP8:
        return (d.B * d.H * N * d.d_v * 33 // 32,)
    return (d.B, d.H, N, d.d_v)


def fp8_state_planes(d: SdmDims, state):
    """Views of an fp8 state buffer: E4M3 codes [B, H, N, d_v] and block exponents
    [B, H, N, d_v / 32]."""
    N = d.n * d.n
    k = d.B * d.H * N * d.d_v
    return (state[:k].view(d.B, d.H, N, d.d_v), state[k:].view(d.B, d.H, N, d.d_v // 32))


@_on_stream
def scan(d: SdmDims, products: dict, norm_w, state, with_y_raw=False, out=None, ws=None,
         stream=None):
    _check_products(d, products)
    N = d.n * d.n
    _need(state, state_dtype(d), state_shape(d), "state")
    if norm_w is not None:
        _need(norm_w, torch.float32, (d.H, d.d_v), "norm_w")
    dev = state.device
    o = out if out is not None else torch.empty((d.B, d.T, d.H, d.d_v), device=dev)
    _need(o, torch.float32, (d.B, d.T, d.H, d.d_v), "out")
    y = torch.empty_like(o) if with_y_raw else None
    ws, nb = _workspace(d, _lib.SDM_ENTRY_SCAN, dev, ws)
    _lib.sdm_scan(d, _sel(products), norm_w, state, o, y, ws, nb, stream)
    return (o, y) if with_y_raw else o


@_on_stream
def forward(d: SdmDims, x, w_proj, A, b_dt, norm_w, state, debug=False, with_scores=False,
            out=None, ws=None, stream=None):
    """Whole path; state is updated in place.  Returns out (and the products if debug)."""
    _check_params(d, x, w_proj, A, b_dt)
    N = d.n * d.n
    _need(state, state_dtype(d), state_shape(d), "state")
    if norm_w is not None:
        _need(norm_w, torch.float32, (d.H, d.d_v), "norm_w")
    o = out if out is not None else torch.empty((d.B, d.T, d.H, d.d_v), device=x.device)
    _need(o, torch.float32, (d.B, d.T, d.H, d.d_v), "out")
    prod = alloc_products(d, x.device, with_scores) if debug else None
    ws, nb = _workspace(d, _lib.SDM_ENTRY_FORWARD, x.device, ws)
    _lib.sdm_forward(d, x, w_proj, A, b_dt, norm_w, state, o, _sel(prod) if prod else None, ws,
                     nb, stream)
    return (o, prod) if debug else o


def log_format(d: SdmDims) -> str:
    if d.flags & _lib.SDM_FLAG_LOG_FP8:
        return "fp8"
    return "int4" if d.flags & _lib.SDM_FLAG_LOG_INT4 else "fp32"


@_on_stream
def scan_train(d: SdmDims, products: dict, norm_w, state, out=None, ws=None, stream=None):
    """Training forward: scan() that also records the write log.  Returns
    (out, y_raw, log) with log a dict: "rows" ([B, T, H, W, d_v] fp32, or uint8 codes
    [.., d_v] (fp8) / [.., d_v / 2] (int4)) and "scale" ([B, T, H, W] absmax, or None)."""
    _check_products(d, products)
    N = d.n * d.n
    _need(state, torch.float32, (d.B, d.H, N, d.d_v), "state")
    if norm_w is not None:
        _need(norm_w, torch.float32, (d.H, d.d_v), "norm_w")
    dev = state.device
    o = out if out is not None else torch.empty((d.B, d.T, d.H, d.d_v), device=dev)
    _need(o, torch.float32, (d.B, d.T, d.H, d.d_v), "out")
    y = torch.empty_like(o)
    fmt = log_format(d)
    lead = (d.B, d.T, d.H, d.W)
    if fmt == "fp32":
        log = dict(rows=torch.empty(lead + (d.d_v,), device=dev), scale=None)
    else:
        width = d.d_v if fmt == "fp8" else d.d_v // 2
        log = dict(rows=torch.empty(lead + (width,), dtype=torch.uint8, device=dev),
                   scale=torch.empty(lead, device=dev))
    ws, nb = _workspace(d, _lib.SDM_ENTRY_SCAN_TRAIN, dev, ws)
    _lib.sdm_scan_train(d, _sel(products), norm_w, state, o, y, log["rows"], log["scale"], ws, nb,
                        stream)
    return o, y, log


@_on_stream
def scan_backward(d: SdmDims, products: dict, norm_w, state, d_state, y_raw, log, d_out,
                  with_d_norm_w=True, ws=None, stream=None):
    """Gradients of scan_train's call.  state (M_T -> M_0) and d_state (dL/dM_T ->
    dL/dM_0) are updated in place.  Returns a dict of gradient tensors."""
    _check_products(d, products)
    N = d.n * d.n
    B, T, H = d.B, d.T, d.H
    _need(state, torch.float32, (B, H, N, d.d_v), "state")
    _need(d_state, torch.float32, (B, H, N, d.d_v), "d_state")
    _need(y_raw, torch.float32, (B, T, H, d.d_v), "y_raw")
    fmt = log_format(d)
    if fmt == "fp32":
        _need(log["rows"], torch.float32, (B, T, H, d.W, d.d_v), "log rows")
    else:
        _need(log["rows"], torch.uint8,
              (B, T, H, d.W, d.d_v if fmt == "fp8" else d.d_v // 2), "log rows")
        _need(log["scale"], torch.float32, (B, T, H, d.W), "log scale")
    _need(d_out, torch.float32, (B, T, H, d.d_v), "d_out")
    if norm_w is not None:
        _need(norm_w, torch.float32, (H, d.d_v), "norm_w")
    e = lambda *s: torch.empty(s, dtype=torch.float32, device=state.device)
    g = dict(d_wt_w=e(B, T, H, d.W), d_wt_r=e(B, T, H, d.R), d_v=e(B, T, H, d.d_v),
             d_gate=e(B, T, H, d.d_v), d_alpha=e(B, T, H), d_beta=e(B, T, H),
             d_norm_w=e(H, d.d_v) if with_d_norm_w else None)
    ws, nb = _workspace(d, _lib.SDM_ENTRY_SCAN_BACKWARD, state.device, ws)
    gs = _lib.SdmScanGrads(*[_lib._ptr(g[k]) for k in _lib.GRAD_FIELDS])
    _lib.sdm_scan_backward(d, _sel(products), norm_w, state, d_state, y_raw, log["rows"],
                           log["scale"], d_out, gs, ws, nb, stream)
    return g


@_on_stream
def select_backward(d: SdmDims, products: dict, x, w_proj, A, b_dt, grads: dict, ws=None,
                    stream=None):
    """Backward of the selection pass: gradients of its products (grads: d_wt_w, d_wt_r,
    d_v, d_gate, d_alpha, d_beta, as scan_backward returns them) to the projection output.
    Returns (d_y [B, T, H*P], d_A [H], d_b_dt [H]); dx = d_y W_proj and dW_proj =
    d_y^T x are plain GEMMs left to the caller."""
    _check_params(d, x, w_proj, A, b_dt)
    _check_products(d, products)
    B, T, H = d.B, d.T, d.H
    shapes = dict(d_wt_w=(d.W,), d_wt_r=(d.R,), d_v=(d.d_v,), d_gate=(d.d_v,), d_alpha=(),
                  d_beta=())
    for k in _lib.SELECT_GRAD_FIELDS:
        _need(grads[k], torch.float32, (B, T, H) + shapes[k], k)
    P = 4 * d.n + 2 * d.d_v + 2
    dev = x.device
    d_y = torch.empty((B, T, H * P), dtype=torch.float32, device=dev)
    d_A = torch.empty((H,), dtype=torch.float32, device=dev)
    d_b_dt = torch.empty((H,), dtype=torch.float32, device=dev)
    ws, nb = _workspace(d, _lib.SDM_ENTRY_SELECT_BACKWARD, dev, ws)
    gs = _lib.SdmSelectGrads(*[_lib._ptr(grads[k]) for k in _lib.SELECT_GRAD_FIELDS])
    _lib.sdm_select_backward(d, _sel(products), x, w_proj, A, b_dt, gs, d_y, d_A, d_b_dt, ws, nb,
                             stream)
    return d_y, d_A, d_b_dt


def alloc_touched(d: SdmDims, device):
    """All-zero touched bitmaps [B, H, ceil(N/32)] (int32 words): every sequence at M0."""
    return torch.zeros((d.B, d.H, (d.n * d.n + 31) // 32), dtype=torch.int32, device=device)


def _check_shared(d: SdmDims, m0, state, touched):
    N = d.n * d.n
    _need(m0, state_dtype(d), (d.H, N, d.d_v), "m0")
    _need(state, state_dtype(d), state_shape(d), "state")
    _need(touched, torch.int32, (d.B, d.H, (N + 31) // 32), "touched")


@_on_stream
def scan_shared_m0(d: SdmDims, products: dict, norm_w, m0, state, touched, with_y_raw=False,
                   out=None, ws=None, stream=None):
    """scan() on the effective state (store rows whose touched bit is set, else m0)."""
    _check_products(d, products)
    _check_shared(d, m0, state, touched)
    if norm_w is not None:
        _need(norm_w, torch.float32, (d.H, d.d_v), "norm_w")
    o = out if out is not None else torch.empty((d.B, d.T, d.H, d.d_v), device=state.device)
    _need(o, torch.float32, (d.B, d.T, d.H, d.d_v), "out")
    y = torch.empty_like(o) if with_y_raw else None
    ws, nb = _workspace(d, _lib.SDM_ENTRY_SCAN, state.device, ws)
    _lib.sdm_scan_shared_m0(d, _sel(products), norm_w, m0, state, touched, o, y, ws, nb, stream)
    return (o, y) if with_y_raw else o


@_on_stream
def forward_shared_m0(d: SdmDims, x, w_proj, A, b_dt, norm_w, m0, state, touched, out=None,
                      ws=None, stream=None):
    """forward() on the effective state; state and touched are updated in place."""
    _check_params(d, x, w_proj, A, b_dt)
    _check_shared(d, m0, state, touched)
    if norm_w is not None:
        _need(norm_w, torch.float32, (d.H, d.d_v), "norm_w")
    o = out if out is not None else torch.empty((d.B, d.T, d.H, d.d_v), device=x.device)
    _need(o, torch.float32, (d.B, d.T, d.H, d.d_v), "out")
    ws, nb = _workspace(d, _lib.SDM_ENTRY_FORWARD, x.device, ws)
    _lib.sdm_forward_shared_m0(d, x, w_proj, A, b_dt, norm_w, m0, state, touched, o, ws, nb,
                               stream)
    return o


@_on_stream
def slot_histogram(d: SdmDims, idx_w, counts=None, stream=None):
    """Per-head slot-update counts [H, N] int32; accumulates into `counts` if given."""
    _need(idx_w, torch.int32, (d.B, d.T, d.H, d.W), "idx_w")
    N = d.n * d.n
    if counts is None:
        counts = torch.zeros((d.H, N), dtype=torch.int32, device=idx_w.device)
    _need(counts, torch.int32, (d.H, N), "counts")
    _lib.sdm_slot_histogram(d, idx_w, counts, stream)
    return counts
