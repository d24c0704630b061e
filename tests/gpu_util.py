"""Helpers of the GPU parity tests: device transfer of synthetic inputs and the
comparison rules (tolerances, near-tie accounting)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import sdm_oracle as O
from sparse_memory_linear_sdm_amd import synth

RTOL, ATOL = 1e-4, 1e-5        # fp32 state / outputs / weights vs the fp64 oracle
NEAR_TIE = 1e-6                # gap between the W-th and (W+1)-th oracle score


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_dev(a, dtype=None):
    if isinstance(a, np.ndarray) and a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev())
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev())


def host(t):
    return t.detach().cpu().numpy()


def layer_inputs(wl: synth.Workload, seed=0, with_state=True):
    """Synthetic inputs of a workload: host values (fp32) and device tensors."""
    x_vals, x_store = synth.gen_x(wl, seed)
    prm = synth.gen_params(wl, seed)
    h = dict(x=x_vals, w_proj=prm["w_proj"], A=prm["A"], b_dt=prm["b_dt"], gamma=prm["gamma"])
    d = dict(x=to_dev(x_store), w_proj=to_dev(prm["w_proj_store"]), A=to_dev(prm["A"]),
             b_dt=to_dev(prm["b_dt"]), gamma=to_dev(prm["gamma"]))
    if with_state:
        m0 = synth.gen_m0(wl, seed)
        h["m0"] = m0
        d["m0"] = to_dev(m0)
    return h, d


def broadcast_state(m0_dev, B):
    """A new [B, ...] state tensor holding B copies of m0 (never a view of m0: for
    B = 1 an expanded view would already be contiguous and alias it)."""
    return m0_dev.unsqueeze(0).repeat(B, *([1] * m0_dev.dim()))


def assert_close(got, exp, what, rtol=RTOL, atol=ATOL):
    got = np.asarray(got, np.float64)
    exp = np.asarray(exp, np.float64)
    err = np.abs(got - exp) - (atol + rtol * np.abs(exp))
    bad = np.argwhere(err > 0)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {bad.shape[0]} elements out of tolerance; first at {i}: "
                             f"got {got[i]!r} expected {exp[i]!r}")


def gemm_bound(x_rows, w, K):
    """Deterministic fp32-accumulation error bound of Y = x W^T for K terms."""
    return K * 2.0 ** -24 * (np.abs(np.asarray(x_rows, np.float64)) @ np.abs(np.asarray(w, np.float64)).T) + 1e-6


def random_products(rng, B, T, H, n, W, R, d_v, mode="random"):
    """Host-side selection products for scan tests (ids ascending and distinct).

    mode: "random" (independent tokens), "repeat" (runs of identical selections),
          "same" (every token selects the same slots).
    """
    N = n * n
    shp = (B, T, H)

    def ids(count):
        out = np.empty(shp + (count,), np.int32)
        for idx in np.ndindex(*shp):
            out[idx] = np.sort(rng.choice(N, count, replace=False))
        return out

    iw, ir = ids(W), ids(R)
    if mode == "repeat":
        for t in range(1, T):
            keep = rng.random((B, H)) < 0.7
            iw[:, t][keep] = iw[:, t - 1][keep]
            ir[:, t][keep] = ir[:, t - 1][keep]
        if R <= W:  # half of the tokens read exactly slots they write
            rd = rng.random(shp) < 0.5
            ir[rd] = iw[rd][:, :R]
    elif mode == "same":
        iw[:] = iw[:, :1]
        ir[:] = ir[:, :1]
    wt_w = rng.dirichlet(np.ones(W), shp).astype(np.float32)
    wt_r = rng.dirichlet(np.ones(R), shp).astype(np.float32)
    return dict(idx_w=iw, wt_w=wt_w, idx_r=ir, wt_r=wt_r,
                v=rng.standard_normal(shp + (d_v,)).astype(np.float32),
                gate=rng.uniform(0, 1, shp + (d_v,)).astype(np.float32),
                alpha=rng.uniform(0.3, 1.0, shp).astype(np.float32),
                beta=rng.uniform(0.0, 1.0, shp).astype(np.float32))


def strided_products(rng, B, T, H, n, W, R, d_v):
    """Distinct ids per token without a per-token loop: an offset and an odd stride
    modulo N = n^2 (a power of two), ascending."""
    N = n * n
    assert N & (N - 1) == 0 and max(W, R) <= N
    shp = (B, T, H)

    def ids(count):
        o = rng.integers(0, N, shp + (1,))
        st = rng.integers(0, N // 2, shp + (1,)) * 2 + 1
        return np.sort((o + st * np.arange(count)) % N, axis=-1).astype(np.int32)

    def wts(count):
        w = rng.uniform(0.05, 1.0, shp + (count,)).astype(np.float32)
        return (w / w.sum(-1, keepdims=True)).astype(np.float32)

    return dict(idx_w=ids(W), wt_w=wts(W), idx_r=ids(R), wt_r=wts(R),
                v=rng.standard_normal(shp + (d_v,)).astype(np.float32),
                gate=rng.uniform(0, 1, shp + (d_v,)).astype(np.float32),
                alpha=rng.uniform(0.3, 1.0, shp).astype(np.float32),
                beta=rng.uniform(0.0, 1.0, shp).astype(np.float32))


def oracle_walks(prod_h, m0_h, gamma, eps, walks, rule="slot", state="exact"):
    """Oracle scan + norm for the listed (b, h) walks from given products."""
    res = {}
    for b, h in walks:
        sel = {k: prod_h[k][b, :, h] for k in ("idx_w", "wt_w", "idx_r", "wt_r", "v", "gate",
                                                "alpha", "beta")}
        sel["g"] = sel.pop("gate")
        out, y, M = O.forward_walk(m0_h[b, h] if m0_h.ndim == 4 else m0_h[h], sel, gamma[h], eps,
                                   rule, state)
        res[(b, h)] = (out, y, M)
    return res


# ---- bf16 state storage ------------------------------------------------------------
# The kernels compute each update in fp32 and round it once to bf16; the oracle
# computes it in fp64 and rounds once.  The two stored values are equal unless the
# exact value lies within a few fp32 ulps (2^-22 relative) of a bf16 rounding
# boundary -- about 1e-5 of the element writes on these inputs -- and then they are
# one spacing apart.  Later writes carry such a difference scaled by alpha (1 - c)
# (and, in the key-weighted form, spread it over the write set with weights
# beta k_i alpha k_j summing to at most 1), so it never grows beyond the rounding
# steps it started from -- in absolute terms: an element that later shrinks towards
# zero keeps the difference of its larger past.  The bound is therefore two bf16
# spacings of the walk's largest state magnitude, and the differing elements must
# stay rare.  Reads of a differing element move y by at most that much (the read
# weights sum to 1).
BF16_MAX_DIFF_FRACTION = 1e-3


def bf16_spacing(x):
    """Distance between adjacent bf16 values around |x| (8 significant bits)."""
    _, e = np.frexp(np.abs(np.asarray(x, np.float64)))
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


def fp8_spacing(x):
    """Distance between adjacent E4M3 values around |x| (3 fraction bits) -- at the
    walk's scale, a bound for every block's elements (no block scale exceeds it)."""
    _, e = np.frexp(np.abs(np.asarray(x, np.float64)))
    return np.ldexp(1.0, e - 4)


def check_bf16_state(got, exp, scale, what, spacing=bf16_spacing):
    """Stored states equal but for a small fraction of elements, each at most two
    spacings of the format (bf16, or fp8 with spacing=fp8_spacing) at the walk's scale
    apart: roundings of values that lay within fp32 error of a rounding boundary."""
    got = np.asarray(got, np.float64)
    exp = np.asarray(exp, np.float64)
    diff = got != exp
    frac = float(diff.mean())
    assert frac <= BF16_MAX_DIFF_FRACTION, f"{what}: {frac:.2e} of the elements differ"
    if diff.any():
        worst = np.max(np.abs(got - exp)) / spacing(scale)
        assert worst <= 2.0, f"{what}: a difference of {worst:.2f} spacings of the state's scale"
    return int(diff.sum())


def check_bf16_reads(y_got, y_exp, out_got, gamma_h, gate, eps, scale, R, what,
                     spacing=bf16_spacing):
    """y: within the fp32 summation bound 2R 2^-24 scale (R weighted rows, weights
    summing to 1, plus the schedules' partial sums), or -- for tokens that read an
    element one rounding step apart -- within that plus two spacings of the scale;
    such tokens are a minority.  out: the norm and gate of the kernel's own y (given
    y, the normalised output is fixed; normalising a small y magnifies its absolute
    difference, so out is not compared with the oracle's out directly)."""
    y_got = np.asarray(y_got, np.float64)
    y_exp = np.asarray(y_exp, np.float64)
    err = np.abs(y_got - y_exp)
    fp32 = 2 * R * 2.0 ** -24 * scale + 1e-12
    ok = np.all(err <= fp32, axis=-1)
    assert (~ok).mean() <= 0.25, f"{what}: {(~ok).sum()} of {ok.size} tokens beyond the fp32 bound"
    delta = fp32 + 2 * spacing(scale)
    assert np.all(err <= delta), f"{what}: read beyond the storage format's bound"
    assert_close(out_got, O.rms_norm_gate(y_got, gamma_h, gate, eps), f"{what} norm/gate")
    # out against the oracle's out: with s = (mean(y^2) + eps)^(-1/2) and yhat = y s, the
    # norm's Jacobian d out_i / d y_j = gamma_i g_i s (delta_ij - yhat_i yhat_j / d_v)
    # bounds the change from a read error of at most delta per element by
    # |gamma_i g_i| s delta (1 + |yhat_i| mean_j |yhat_j|); half again for the second
    # order, plus the fp32 tolerance of the norm itself
    gate = np.asarray(gate, np.float64)
    o_exp = O.rms_norm_gate(y_exp, gamma_h, gate, eps)
    s = 1.0 / np.sqrt(np.mean(y_exp * y_exp, axis=-1, keepdims=True) + eps)
    yh = np.abs(y_exp) * s
    lim = (np.abs(np.asarray(gamma_h, np.float64) * gate) * s * delta *
           (1.0 + yh * np.mean(yh, axis=-1, keepdims=True)))
    oerr = np.abs(np.asarray(out_got, np.float64) - o_exp)
    okout = oerr <= 1.5 * lim + RTOL * np.abs(o_exp) + ATOL
    assert okout.all(), (f"{what}: out beyond the bound from the reads at "
                         f"{np.argwhere(~okout)[0]}, err {oerr[~okout].max():.3e}")
    return int((~ok).sum())
