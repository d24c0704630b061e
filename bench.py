"""Benchmark of the SDM layer forward path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload layer1p4b]
                    [--mode forward|train]

A step is one pass of the whole path (projection GEMM + gates, product-key
selection, recurrent sparse scan, RMSNorm + gate) over one batch of synthetic
input already resident in HBM.  Prints one JSON line with tokens/s, the
roofline of the dominant kernel (the scan, HBM-bound) and a CPU baseline (the
fp64 oracle timed on a bounded sample of the same workload on the host).

--mode train times the training path instead: a step is the selection pass, the
training forward of the scan (with the fp32 write log) and the scan backward
(random incoming gradients of out and of the final state), which leaves the state
at M0 again.  Its roofline is the reverse-walk kernel's; no CPU baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "SDM layer tokens/s at N=131072,W=R=64,d_v=128; effective HBM GB/s vs peak"
METRIC_TRAIN = ("SDM layer training tokens/s (selection, scan forward with write log, scan "
                "backward); reverse-walk HBM GB/s vs peak")
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
CSRC = os.path.join(ROOT, "sparse_memory_linear_sdm_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_traffic_layer1p4b.txt")
SCAN_SOURCE = os.path.join(CSRC, "scan_stream.hip")
MFMA_FILE = os.path.join(ROOT, "profiles", "proj_gemm_mfma_layer1p4b.txt")
BACK_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_backward_traffic_layer1p4b.txt")
BACK_SOURCE = os.path.join(CSRC, "scan_stream_backward.hip")
GEMM_SOURCE = os.path.join(CSRC, "proj_gemm.hip")


def _profile_fields(path: str, source: str):
    """Fields of a committed counter summary, if it was taken on the current source."""
    import hashlib
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.split()[0] if v.split() else ""
    cur = hashlib.sha256(open(source, "rb").read()).hexdigest()
    if fields.get("source_sha256") != cur:
        return None  # the kernel changed since the counters were taken
    return fields


def measured_traffic(workload: str):
    """Counter-measured HBM bytes of one scan launch, if taken on the current source."""
    f = _profile_fields(TRAFFIC_FILE, SCAN_SOURCE) if workload == "layer1p4b" else None
    return int(float(f["traffic_bytes"])) if f else None


def measured_back_traffic(workload: str):
    """Counter-measured HBM bytes of one reverse-walk launch (current source)."""
    f = _profile_fields(BACK_TRAFFIC_FILE, BACK_SOURCE) if workload == "layer1p4b" else None
    return int(float(f["traffic_bytes"])) if f else None


def measured_mfma_util(workload: str):
    """Counter-measured MFMA busy fraction of the projection GEMM (current source)."""
    f = _profile_fields(MFMA_FILE, GEMM_SOURCE) if workload == "layer1p4b" else None
    return float(f["mfma_util"]) if f else None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", default="layer1p4b")
    p.add_argument("--state", choices=("fp32", "bf16"), default="fp32",
                   help="state storage: fp32 (the method's precision) or bf16 with fp32 "
                        "arithmetic (SDM_FLAG_STATE_BF16)")
    p.add_argument("--mode", choices=("forward", "train"), default="forward")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-tokens", type=int, default=2048,
                   help="tokens of batch entry 0 in the oracle's timed sample")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="after the timed steps, copy MIB MiB device-to-device (the reference "
                        "kernel of known traffic for scaling hardware byte counters)")
    return p.parse_args()


def cpu_baseline(wl, ntok: int) -> dict:
    """The fp64 oracle, as it stands, on the first `ntok` tokens of batch entry 0."""
    from threadpoolctl import threadpool_limits

    from oracle import sdm_oracle as O
    from sparse_memory_linear_sdm_amd import synth

    x, _ = synth.gen_x(wl, seed=0, t0=0, t1=ntok, batches=[0])
    prm = synth.gen_params(wl, seed=0)
    m0 = synth.gen_m0(wl, seed=0)[None]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        O.forward(x, prm["w_proj"], prm["A"], prm["b_dt"], prm["gamma"], m0, wl.H, wl.n, wl.d_v,
                  wl.W, wl.R, wl.eps)
        dt = time.perf_counter() - t0
    return {"value": ntok / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{wl.name}: tokens 0..{ntok - 1} of batch entry 0, all {wl.H} heads, "
                      f"from x (fp64 projection, brute-force top-{wl.W}/{wl.R} over "
                      f"N={wl.N}, sequential scan, norm+gate); {dt:.1f} s on 1 host thread"}


def copy_calibration(mib: int, dev, res: dict) -> None:
    """A device-to-device copy of known size after the timed steps: the reference
    kernel for scaling hardware byte counters."""
    import torch
    nb = mib << 20
    src = torch.empty(nb // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    res["copy_calibration_bytes"] = {"read": nb, "write": nb}


def gemm_line(wl, kernels_ms, kernel, steps):
    """The projection GEMM against the dense MFMA peak of its dtype: algorithmic
    2 M N K flops over its event-timed duration per step, and the counted MFMA busy
    fraction from the committed rocprofv3 summary."""
    if kernel is None:
        return None
    ms = kernels_ms[kernel]["avg"] * kernels_ms[kernel]["launches"] / steps
    flops = 2.0 * wl.tokens * wl.H * wl.P * wl.d_model
    tf = flops / (ms * 1e-3) / 1e12
    peak = MFMA_BF16_PEAK_TFLOPS if kernel == "proj_gemm_bf16" else 157.3
    return {"kernel": kernel, "achieved": tf, "peak": peak, "unit": "TFLOP/s", "frac": tf / peak,
            "ms": ms, "mfma_util_counted": measured_mfma_util(wl.name)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the SDM walks "
              "of one GPU are measured at their real shape. Multi-GPU sharding is not built.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_memory_linear_sdm_amd import _lib, dims_for, ops, synth

    if args.mode == "train":
        return train_main(args)
    wl = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = dims_for(wl)
    bf16_state = args.state == "bf16"
    if bf16_state:
        d.flags |= _lib.SDM_FLAG_STATE_BF16

    # inputs resident in HBM before timing
    _, x_store = synth.gen_x(wl, seed=0)
    prm = synth.gen_params(wl, seed=0)
    m0 = synth.gen_m0(wl, seed=0)

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    x = to_dev(x_store)
    w = to_dev(prm["w_proj_store"])
    A, b_dt, gamma = to_dev(prm["A"]), to_dev(prm["b_dt"]), to_dev(prm["gamma"])
    m0_d = to_dev(m0)
    if bf16_state:
        m0_d = m0_d.to(torch.bfloat16)
    state = m0_d.unsqueeze(0).repeat(wl.B, *([1] * m0_d.dim()))  # a copy, also for B = 1
    del m0
    prod = ops.alloc_products(d, dev)
    out = torch.empty((wl.B, wl.T, wl.H, wl.d_v), device=dev)
    ws_sel = torch.empty(max(_lib.workspace_bytes(d, _lib.SDM_ENTRY_SELECT), 1), dtype=torch.uint8,
                         device=dev)
    ws_scan = torch.empty(max(_lib.workspace_bytes(d, _lib.SDM_ENTRY_SCAN), 1), dtype=torch.uint8,
                          device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        ops.select(d, x, w, A, b_dt, out=prod, ws=ws_sel, stream=stream)
        if ev:
            ev[1].record(stream)
        ops.scan(d, prod, gamma, state, out=out, ws=ws_scan, stream=stream)
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    _lib.timing_read()  # drop records of earlier calls

    # timed steps: the library brackets each of its kernel launches with HIP events
    # on `stream` (SDM_FLAG_TIMING), so every kernel's duration comes from this run
    d.flags |= _lib.SDM_FLAG_TIMING
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    d.flags &= ~_lib.SDM_FLAG_TIMING
    ms_sel = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    ms_scan = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    ms_step = float(np.mean([e[0].elapsed_time(e[2]) for e in evs]))
    ms_wall = wall * 1e3 / args.steps
    per_kernel = {}
    for name, ms in _lib.timing_read(1 << 16):
        per_kernel.setdefault(name, []).append(ms)
    kernels_ms = {k: {"avg": float(np.mean(v)), "launches": len(v)} for k, v in per_kernel.items()}
    scan_kernel = next(k for k in ("two_phase_scan", "stream_scan", "scan_direct") if k in kernels_ms)
    gemm_kernel = next((k for k in ("proj_gemm_bf16", "proj_gemm_f32") if k in kernels_ms), None)
    # launches per step (the scan can run in token chunks): time per step of that kernel
    scan_ms = kernels_ms[scan_kernel]["avg"] * kernels_ms[scan_kernel]["launches"] / args.steps

    tokens = wl.tokens
    slot_bytes = tokens * wl.H * wl.slot_bytes_per_token_head(2 if bf16_state else 4)
    achieved = slot_bytes / (scan_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": tokens / (ms_wall * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_wall,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16 projection, fp32 selection/scan, bf16 state storage" if bf16_state
                  else "bf16 projection, fp32 selection/scan"),
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "d_model": wl.d_model, "H": wl.H,
                   "N": wl.N, "n": wl.n, "W": wl.W, "R": wl.R, "d_v": wl.d_v,
                   "state": f"{args.state} [B,H,N,d_v]", "tokens_per_step": tokens},
        "phases_ms": {"select": ms_sel, "scan": ms_scan, "step_events": ms_step},
        "gemm": gemm_line(wl, kernels_ms, gemm_kernel, args.steps),
        "kernels_ms": kernels_ms,
        "effective_hbm_gbs_step": slot_bytes / (ms_wall * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "kernel": scan_kernel, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None if bf16_state else measured_traffic(wl.name),
                     "algorithmic_bytes_per_launch":
                         slot_bytes * args.steps / kernels_ms[scan_kernel]["launches"]},
    }
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, dev, res)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_tokens)
    print(json.dumps(res), flush=True)


def train_main(args):
    import torch

    from sparse_memory_linear_sdm_amd import _lib, dims_for, ops, synth

    if args.state != "fp32":
        print("--mode train keeps fp32 state", file=sys.stderr)
        sys.exit(2)
    wl = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = dims_for(wl)
    _, x_store = synth.gen_x(wl, seed=0)
    prm = synth.gen_params(wl, seed=0)
    m0 = synth.gen_m0(wl, seed=0)

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    x = to_dev(x_store)
    w = to_dev(prm["w_proj_store"])
    A, b_dt, gamma = to_dev(prm["A"]), to_dev(prm["b_dt"]), to_dev(prm["gamma"])
    state = to_dev(m0).unsqueeze(0).expand(wl.B, *m0.shape).contiguous()
    del m0
    gen = torch.Generator(device=dev).manual_seed(0)
    d_out = torch.randn((wl.B, wl.T, wl.H, wl.d_v), device=dev, generator=gen)
    d_state0 = torch.randn(state.shape, device=dev, generator=gen) * 0.1
    d_state = torch.empty_like(d_state0)
    prod = ops.alloc_products(d, dev)
    out = torch.empty((wl.B, wl.T, wl.H, wl.d_v), device=dev)
    ws_sel = torch.empty(max(_lib.workspace_bytes(d, _lib.SDM_ENTRY_SELECT), 1), dtype=torch.uint8,
                         device=dev)
    ws_fwd = torch.empty(max(_lib.workspace_bytes(d, _lib.SDM_ENTRY_SCAN_TRAIN), 1),
                         dtype=torch.uint8, device=dev)
    ws_bwd = torch.empty(max(_lib.workspace_bytes(d, _lib.SDM_ENTRY_SCAN_BACKWARD), 1),
                         dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        d_state.copy_(d_state0)
        ops.select(d, x, w, A, b_dt, out=prod, ws=ws_sel, stream=stream)
        _, y, log = ops.scan_train(d, prod, gamma, state, out=out, ws=ws_fwd, stream=stream)
        ops.scan_backward(d, prod, gamma, state, d_state, y, log, d_out, ws=ws_bwd, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    _lib.timing_read()
    d.flags |= _lib.SDM_FLAG_TIMING
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    d.flags &= ~_lib.SDM_FLAG_TIMING
    ms_wall = wall * 1e3 / args.steps
    per_kernel = {}
    for name, ms in _lib.timing_read(1 << 16):
        per_kernel.setdefault(name, []).append(ms)
    kernels_ms = {k: {"avg": float(np.mean(v)), "launches": len(v)} for k, v in per_kernel.items()}
    back = next(k for k in ("stream_backward", "scan_backward") if k in kernels_ms)
    back_ms = kernels_ms[back]["avg"] * kernels_ms[back]["launches"] / args.steps
    tokens = wl.tokens
    # per token and head: M and dM read, dM written per read; log and dM read, dM and M
    # written per write
    back_bytes = tokens * wl.H * (3 * wl.R + 4 * wl.W) * wl.d_v * 4
    achieved = back_bytes / (back_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC_TRAIN,
        "value": tokens / (ms_wall * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_wall,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 projection, fp32 selection/scan/gradients, fp32 write log",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "d_model": wl.d_model, "H": wl.H,
                   "N": wl.N, "n": wl.n, "W": wl.W, "R": wl.R, "d_v": wl.d_v,
                   "state": "fp32 [B,H,N,d_v]", "tokens_per_step": tokens,
                   "step": "select + scan_train + scan_backward"},
        "kernels_ms": kernels_ms,
        "roofline": {"bound": "hbm", "kernel": back, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_back_traffic(wl.name) if back == "stream_backward" else None,
                     "algorithmic_bytes_per_launch":
                         back_bytes * args.steps / kernels_ms[back]["launches"]},
    }
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, dev, res)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
