"""Seeded synthetic workloads for the SDM forward path.

This module holds the workload shapes and the random draws that both the
GPU path (tests, bench) and the CPU oracle are fed with.  It contains none of
the method's arithmetic: it only draws numbers and rounds them to the storage
type (bf16 by round-to-nearest-even), so that the two sides of every parity
check see bit-identical inputs.

Every tensor is drawn from numpy's PCG64 with a ``SeedSequence`` whose spawn key
names (workload, tensor, block), so any block can be regenerated on its own.

Distributions (the pages print none; these are the stated workload recipe):
  x       ~ N(0, 1)                      [B, T, d_model]
  W_proj  ~ N(0, 1/d_model)              [H*P, d_model], P = 4n + 2 d_v + 2
  A       = 1                            [H]
  b_dt    ~ U(-4, -1)                    [H]
  gamma   = 1                            [H, d_v]   (RMSNorm weight)
  M0      ~ N(0, 0.02^2)                 [H, N, d_v] fp32, shared across batch
The long-sequence workload repeats every 4096-token block once later: blocks
128..255 are a seeded permutation of blocks 0..127.
"""
from __future__ import annotations

import dataclasses
import numpy as np

# tensor tags for the spawn keys
_X, _W, _BDT, _M0, _PERM = 1, 2, 3, 4, 5
X_BLOCK = 4096  # tokens per independently seeded block of x


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    tag: int           # spawn-key id of this workload
    B: int
    T: int
    d_model: int
    H: int
    n: int             # sqrt(N): slots per head N = n*n
    W: int
    R: int
    d_v: int
    dtype: str         # "fp32" or "bf16" for x and W_proj
    steps: int = 1     # decode: number of T=1 calls (T holds the step count)
    repeat_block: int = 0  # long workload: block size whose copies recur later
    eps: float = 1e-6
    gate_act: int = 1  # 1 = sigmoid

    @property
    def N(self) -> int:
        return self.n * self.n

    @property
    def P(self) -> int:
        return 4 * self.n + 2 * self.d_v + 2

    @property
    def tokens(self) -> int:
        return self.B * self.T

    def slot_bytes_per_token_head(self, elem_bytes: int = 4) -> int:
        """Algorithmic slot-row bytes: W rows read + W rows written + R rows read
        (elements of elem_bytes: 4 for an fp32 state, 2 for bf16)."""
        return (2 * self.W + self.R) * self.d_v * elem_bytes


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 1, B=1, T=256, d_model=64, H=1, n=32, W=8, R=8, d_v=16, dtype="fp32"),
        Workload("layer1p4b", 2, B=8, T=4096, d_model=2048, H=4, n=362, W=64, R=64, d_v=128,
                 dtype="bf16"),
        Workload("long1m", 3, B=1, T=1048576, d_model=2048, H=4, n=512, W=64, R=64, d_v=128,
                 dtype="bf16", repeat_block=4096),
        Workload("layer8b", 4, B=4, T=8192, d_model=4096, H=8, n=1024, W=64, R=64, d_v=128,
                 dtype="bf16"),
        Workload("decode256", 5, B=256, T=64, d_model=2048, H=4, n=256, W=64, R=64, d_v=128,
                 dtype="bf16", steps=64),
    ]
}


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def bf16_round(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _as_storage(a32: np.ndarray, dtype: str):
    """Return (values as fp32, storage array).  For bf16 the storage is uint16 bits."""
    if dtype == "fp32":
        return a32, a32
    bits = bf16_round(a32)
    return bf16_to_f32(bits), bits


def gen_x_block(wl: Workload, b: int, block: int, seed: int = 0) -> np.ndarray:
    """fp32 draw of x[b, block*X_BLOCK : ...] before rounding, honouring repeats."""
    if wl.repeat_block:
        nblk = wl.T // wl.repeat_block
        half = nblk // 2
        if block >= half:
            perm = _rng(seed, wl.tag, _PERM, b).permutation(half)
            block = int(perm[block - half])
    rows = min(X_BLOCK, wl.T - block * X_BLOCK)
    return _rng(seed, wl.tag, _X, b, block).standard_normal((rows, wl.d_model), dtype=np.float32)


def gen_x(wl: Workload, seed: int = 0, t0: int = 0, t1: int | None = None, batches=None):
    """x[b, t0:t1, :] for b in batches -> (fp32 values [nb, t1-t0, d], storage array)."""
    t1 = wl.T if t1 is None else t1
    batches = range(wl.B) if batches is None else batches
    out = np.empty((len(batches), t1 - t0, wl.d_model), np.float32)
    for bi, b in enumerate(batches):
        blk0, blk1 = t0 // X_BLOCK, (t1 - 1) // X_BLOCK
        for blk in range(blk0, blk1 + 1):
            xb = gen_x_block(wl, b, blk, seed)
            lo = max(t0, blk * X_BLOCK)
            hi = min(t1, blk * X_BLOCK + xb.shape[0])
            out[bi, lo - t0:hi - t0] = xb[lo - blk * X_BLOCK:hi - blk * X_BLOCK]
    return _as_storage(out, wl.dtype)


def gen_params(wl: Workload, seed: int = 0):
    """Layer parameters: dict with w_proj (values, storage), A, b_dt, gamma."""
    w = _rng(seed, wl.tag, _W).standard_normal((wl.H * wl.P, wl.d_model), dtype=np.float32)
    w *= np.float32(1.0 / np.sqrt(wl.d_model))
    w_vals, w_store = _as_storage(w, wl.dtype)
    b_dt = _rng(seed, wl.tag, _BDT).uniform(-4.0, -1.0, size=wl.H).astype(np.float32)
    return dict(
        w_proj=w_vals,
        w_proj_store=w_store,
        A=np.ones(wl.H, np.float32),
        b_dt=b_dt,
        gamma=np.ones((wl.H, wl.d_v), np.float32),
    )


def gen_m0_head(wl: Workload, h: int, seed: int = 0) -> np.ndarray:
    """Initial state of head h, [N, d_v] fp32 ~ N(0, 0.02^2)."""
    m = _rng(seed, wl.tag, _M0, h).standard_normal((wl.N, wl.d_v), dtype=np.float32)
    m *= np.float32(0.02)
    return m


def gen_m0(wl: Workload, seed: int = 0) -> np.ndarray:
    return np.stack([gen_m0_head(wl, h, seed) for h in range(wl.H)])


def small(name: str = "tiny", **overrides) -> Workload:
    """A workload with some fields replaced (used for reduced-size parity cases)."""
    return dataclasses.replace(WORKLOADS[name], **overrides)
