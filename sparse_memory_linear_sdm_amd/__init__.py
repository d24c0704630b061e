"""MI355X-native forward path of the Sparse Delta Memory (SDM) layer.

  synth   seeded synthetic workloads (shapes and draws only)
  _lib    ctypes binding of libsdm.so (the C ABI declared in include/sdm.h)
  ops     tensor-level select / select_from_scores / scan / forward
  build   compiles libsdm.so for gfx950
"""
from ._lib import SdmError, SdmDims, SdmSel, dims, abi_version, status_string  # noqa: F401


def dims_for(wl, T=None, B=None):
    """SdmDims of a synth.Workload (optionally with another T or B)."""
    from . import _lib
    return _lib.dims(wl.B if B is None else B, wl.T if T is None else T, wl.d_model, wl.H, wl.n,
                     wl.W, wl.R, wl.d_v,
                     _lib.SDM_DTYPE_BF16 if wl.dtype == "bf16" else _lib.SDM_DTYPE_F32,
                     wl.gate_act, wl.eps)
