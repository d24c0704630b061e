"""Benchmark of the SDM layer forward path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload layer1p4b]
                    [--mode forward|train]

A step is one pass of the whole path (projection GEMM + gates, product-key
selection, recurrent sparse scan, RMSNorm + gate) over one batch of synthetic
input already resident in HBM.  Prints one JSON line with tokens/s, the
roofline of the dominant kernel (the scan, HBM-bound) and a CPU baseline (the
fp64 oracle timed on a bounded sample of the same workload on the host).

--decode-steps (decode workload) times the decode configuration as defined: each
step is one T=1 sdm_forward of all 256 sequences, the 64 steps captured in one HIP
graph and replayed; it reports microseconds per step and slot-row GB/s.

--rule gdn times the key-weighted (Gated DeltaNet form) write rule instead of the
pages' per-slot rule (its default scan schedule from 256 tokens is the chunkwise one);
--schedule forces a scan schedule.

--mode train times the training path instead: a step is the selection pass, the
training forward of the scan (with the fp32 write log), the scan backward (random
incoming gradients of out and of the final state), which leaves the state at M0
again, the selection-pass backward down to dY, and the two projection-gradient
GEMMs (dx, dW_proj; bf16 through the platform BLAS).  Its roofline is the
reverse-walk kernel's; no CPU baseline.  --schedule sets the training forward's
schedule (and the backward's: chunk picks by length as the default does).
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
METRIC_DECODE = ("SDM decode tokens/s (256 sequences, one token per step, N=65536, W=R=64, "
                 "d_v=128; graph-replayed steps); slot-row HBM GB/s vs peak")
METRIC_TRAIN = ("SDM layer training tokens/s (selection, scan forward with write log, scan "
                "backward, selection backward, projection gradients); reverse-walk HBM GB/s "
                "vs peak")
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
CSRC = os.path.join(ROOT, "sparse_memory_linear_sdm_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_traffic_layer1p4b.txt")
SCAN_SOURCE = os.path.join(CSRC, "scan_stream.hip")
MFMA_FILE = os.path.join(ROOT, "profiles", "proj_gemm_mfma_layer1p4b.txt")
BACK_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_backward_traffic_layer1p4b.txt")
BACK_SOURCE = os.path.join(CSRC, "scan_stream_backward.hip")
CHUNK_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "chunk_walk_traffic_layer1p4b_gdn.txt")
CHUNK_BACK_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "chunk_backward_traffic_layer1p4b_gdn.txt")
CHUNK_SOURCE = os.path.join(CSRC, "scan_chunk.hip")
GEMM_SOURCE = os.path.join(CSRC, "proj_gemm.hip")
SELECT_FILE = os.path.join(ROOT, "profiles", "select_valu_layer1p4b.txt")
SELECT_SOURCE = os.path.join(CSRC, "select.hip")
# VALU issue peak of MI355X: 256 CUs x 4 SIMDs, each issuing one wave64 VALU instruction
# every 2 cycles (32 lanes per cycle: the 157.3 TFLOP/s fp32 vector peak is 32 FMA lanes
# x 1024 SIMDs x 2.4 GHz), in wave64 instructions per second
VALU_PEAK_WAVE_INSTR_PER_S = 1024 * 2.4e9 / 2


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


def measured_chunk_traffic(workload: str, backward: bool):
    """Counter-measured HBM bytes of one key-weighted chunk-walk (or chunkwise reverse
    walk) launch, if taken on the current source."""
    path = CHUNK_BACK_TRAFFIC_FILE if backward else CHUNK_TRAFFIC_FILE
    f = _profile_fields(path, CHUNK_SOURCE) if workload == "layer1p4b" else None
    return int(float(f["traffic_bytes"])) if f else None


def measured_select_valu(workload: str):
    """Counted VALU instructions per launch of the selection kernel (current source)."""
    f = _profile_fields(SELECT_FILE, SELECT_SOURCE) if workload == "layer1p4b" else None
    return float(f["valu_instructions_per_launch"]) if f else None


def select_line(wl, kernels_ms, steps):
    """The selection kernel against the VALU issue roofline: counted VALU wave
    instructions per launch (committed rocprofv3 summary, current source) over the
    kernel's event-timed duration, against 1024 SIMDs x 2.4 GHz / 2 cycles."""
    if "select" not in kernels_ms:
        return None
    ms = kernels_ms["select"]["avg"]
    valu = measured_select_valu(wl.name)
    res = {"kernel": "select", "bound": "alu", "ms": ms,
           "problems_per_launch": wl.tokens * wl.H * 2 * steps // kernels_ms["select"]["launches"],
           "peak": VALU_PEAK_WAVE_INSTR_PER_S / 1e12, "unit": "T wave64 VALU instr/s"}
    if valu is not None:
        ach = valu / (ms * 1e-3)
        res.update(valu_instructions_per_launch=valu, achieved=ach / 1e12,
                   frac=ach / VALU_PEAK_WAVE_INSTR_PER_S)
    return res


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
    p.add_argument("--rule", choices=("slot", "gdn"), default="slot",
                   help="write rule: the pages' per-slot delta rule, or the key-weighted "
                        "(Gated DeltaNet form) variant")
    p.add_argument("--schedule", choices=("default", "direct", "stream", "two_phase", "chunk"),
                   default="default", help="scan schedule (default: the library's choice)")
    p.add_argument("--state", choices=("fp32", "bf16", "fp8"), default="fp32",
                   help="state storage: fp32 (the method's precision), bf16 with fp32 "
                        "arithmetic (SDM_FLAG_STATE_BF16), or fp8 E4M3 with a power-of-two "
                        "exponent per 32-column block (SDM_FLAG_STATE_FP8)")
    p.add_argument("--mode", choices=("forward", "train"), default="forward")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-tokens-per-core", type=int, default=2048,
                   help="tokens of batch entry 0 per host core in the oracle's timed sample")
    p.add_argument("--decode-steps", action="store_true",
                   help="decode workload as defined: every step one T=1 sdm_forward of all "
                        "sequences, the steps captured in one HIP graph and replayed")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="after the timed steps, copy MIB MiB device-to-device (the reference "
                        "kernel of known traffic for scaling hardware byte counters)")
    return p.parse_args()


# ---- CPU baseline: the fp64 oracle as it stands, spread over the host's cores ----------
# Worker processes (one BLAS thread each) regenerate the seeded inputs they need.  The
# selection pass runs the oracle's pass_a on token blocks; the scan runs the oracle's
# forward_walk, one (batch, head) walk per process.  Nothing of the oracle is changed.
_CPU = {}


def _cpu_init(name: str, with_m0: bool):
    from threadpoolctl import threadpool_limits

    from sparse_memory_linear_sdm_amd import synth
    threadpool_limits(limits=1)
    wl = synth.WORKLOADS[name]
    _CPU.update(wl=wl, prm=synth.gen_params(wl, seed=0))
    if with_m0:
        _CPU["m0"] = synth.gen_m0(wl, seed=0)


def _cpu_pass_a(block):
    from oracle import sdm_oracle as O
    from sparse_memory_linear_sdm_amd import synth
    wl, prm = _CPU["wl"], _CPU["prm"]
    b, t0, t1 = block
    x, _ = synth.gen_x(wl, seed=0, t0=t0, t1=t1, batches=[b])
    a = O.pass_a(x[0], prm["w_proj"], prm["A"], prm["b_dt"], wl.H, wl.n, wl.d_v, wl.W, wl.R)
    return {k: a[k] for k in ("idx_w", "wt_w", "idx_r", "wt_r", "v", "g", "alpha", "beta")}


def _cpu_walk(job):
    from oracle import sdm_oracle as O
    wl, prm = _CPU["wl"], _CPU["prm"]
    h, sel = job
    out, _, _ = O.forward_walk(_CPU["m0"][h], sel, prm["gamma"][h], wl.eps)
    return out.shape[0]


def cpu_baseline(wl, tokens_per_core: int) -> dict:
    """The fp64 oracle on the first tokens of the batch (whole sequences from entry 0 on,
    all heads, from x) over min(affinity, 16) processes: the selection by token blocks,
    then one process per (batch entry, head) walk."""
    import multiprocessing as mp

    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    ntok = min(wl.tokens, tokens_per_core * cores)
    nb = (ntok + wl.T - 1) // wl.T
    blocks = []
    per = max(1, -(-ntok // cores))
    for b in range(nb):
        tb = min(wl.T, ntok - b * wl.T)
        blocks += [(b, t, min(t + per, tb)) for t in range(0, tb, per)]
    ctx = mp.get_context("spawn")   # fresh interpreters: nothing of the GPU process is inherited
    with ctx.Pool(cores, initializer=_cpu_init, initargs=(wl.name, True)) as pool:
        pool.map(abs, range(cores))  # every worker started and initialised before timing
        t0 = time.perf_counter()
        parts = pool.map(_cpu_pass_a, blocks)
        t1 = time.perf_counter()
        jobs = []
        for b in range(nb):
            mine = [p for blk, p in zip(blocks, parts) if blk[0] == b]
            sel = {k: np.concatenate([p[k] for p in mine]) for k in mine[0]}
            jobs += [(h, {k: v[:, h] for k, v in sel.items()}) for h in range(wl.H)]
        pool.map(_cpu_walk, jobs)
        t2 = time.perf_counter()
    dt = t2 - t0
    return {"value": ntok / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{wl.name}: the first {ntok} tokens ({nb} batch entr"
                      f"{'y' if nb == 1 else 'ies'} from entry 0), all {wl.H} heads, from x "
                      f"(fp64 projection, brute-force top-{wl.W}/{wl.R} over N={wl.N}, "
                      f"sequential scan, norm+gate); {dt:.1f} s on {cores} processes "
                      f"(selection over {len(blocks)} token blocks {t1 - t0:.1f} s, then "
                      f"{len(jobs)} walks {t2 - t1:.1f} s), one BLAS thread each"}


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
    if args.decode_steps:
        return decode_main(args)
    wl = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = dims_for(wl)
    bf16_state = args.state == "bf16"
    fp8_state = args.state == "fp8"
    if bf16_state:
        d.flags |= _lib.SDM_FLAG_STATE_BF16
    if fp8_state:
        d.flags |= _lib.SDM_FLAG_STATE_FP8
    gdn = args.rule == "gdn"
    if gdn:
        d.flags |= _lib.SDM_FLAG_DELTA_GDN
    d.flags |= {"default": 0, "direct": _lib.SDM_FLAG_SCAN_DIRECT,
                "stream": _lib.SDM_FLAG_SCAN_STREAM, "two_phase": _lib.SDM_FLAG_SCAN_TWO_PHASE,
                "chunk": _lib.SDM_FLAG_SCAN_CHUNK}[args.schedule]

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
    if fp8_state:
        state = fp8_state_buffer(state)
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
    scan_kernel = next(k for k in ("two_phase_scan", "stream_scan", "chunk_walk", "gdn_slices",
                                   "scan_direct") if k in kernels_ms)
    gemm_kernel = next((k for k in ("proj_gemm_bf16", "proj_gemm_f32") if k in kernels_ms), None)
    # launches per step (the scan can run in token chunks): time per step of that kernel
    scan_ms = kernels_ms[scan_kernel]["avg"] * kernels_ms[scan_kernel]["launches"] / args.steps

    tokens = wl.tokens
    # (2W + R) rows per token and head for either write rule: the key-weighted
    # prediction and update use the same W row reads
    slot_bytes = tokens * wl.H * wl.slot_bytes_per_token_head(2 if bf16_state else 4)
    if fp8_state:  # a byte per element plus a block exponent byte per 32 columns
        slot_bytes = tokens * wl.H * (2 * wl.W + wl.R) * wl.d_v * 33 // 32
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
                  else "bf16 projection, fp32 selection/scan, fp8 (E4M3, 32-column block "
                       "exponents) state storage" if fp8_state
                  else "bf16 projection, fp32 selection/scan"),
        "rule": args.rule,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "d_model": wl.d_model, "H": wl.H,
                   "N": wl.N, "n": wl.n, "W": wl.W, "R": wl.R, "d_v": wl.d_v,
                   "state": f"{args.state} [B,H,N,d_v]", "tokens_per_step": tokens},
        "phases_ms": {"select": ms_sel, "scan": ms_scan, "step_events": ms_step},
        "gemm": gemm_line(wl, kernels_ms, gemm_kernel, args.steps),
        "select": select_line(wl, kernels_ms, args.steps),
        "kernels_ms": kernels_ms,
        "effective_hbm_gbs_step": slot_bytes / (ms_wall * 1e-3) / 1e9,
        "step_frac_of_peak": slot_bytes / (ms_wall * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm", "kernel": scan_kernel, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": (measured_traffic(wl.name)
                                 if args.state == "fp32" and not gdn and
                                 scan_kernel == "two_phase_scan" else
                                 measured_chunk_traffic(wl.name, False)
                                 if args.state == "fp32" and gdn and scan_kernel == "chunk_walk"
                                 else None),
                     "algorithmic_bytes_per_launch":
                         slot_bytes * args.steps / kernels_ms[scan_kernel]["launches"]},
    }
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, dev, res)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_tokens_per_core)
    print(json.dumps(res), flush=True)


def decode_main(args):
    """The decode workload as defined: each step is one sdm_forward with T = 1 for all
    B sequences, continuing their states.  The wl.T steps (each with its own input
    token) are captured in one HIP graph; a timed repetition replays the graph."""
    import torch

    from sparse_memory_linear_sdm_amd import _lib, dims_for, ops, synth

    wl = synth.WORKLOADS[args.workload]
    if args.state != "fp32":
        print("--decode-steps keeps fp32 state", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d1 = dims_for(wl, T=1)
    if args.rule == "gdn":
        d1.flags |= _lib.SDM_FLAG_DELTA_GDN
    _, x_store = synth.gen_x(wl, seed=0)
    prm = synth.gen_params(wl, seed=0)
    m0 = synth.gen_m0(wl, seed=0)

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # per-step inputs [steps, B, 1, d_model], each step's slice contiguous
    xs = to_dev(x_store).transpose(0, 1).contiguous().unsqueeze(2)
    w = to_dev(prm["w_proj_store"])
    A, b_dt, gamma = to_dev(prm["A"]), to_dev(prm["b_dt"]), to_dev(prm["gamma"])
    m0_d = to_dev(m0)
    del m0
    state = m0_d.unsqueeze(0).repeat(wl.B, *([1] * m0_d.dim()))
    outs = torch.empty((wl.T, wl.B, 1, wl.H, wl.d_v), device=dev)
    ws = torch.empty(max(_lib.workspace_bytes(d1, _lib.SDM_ENTRY_FORWARD), 1), dtype=torch.uint8,
                     device=dev)

    def steps(stream):
        for t in range(wl.T):
            ops.forward(d1, xs[t], w, A, b_dt, gamma, state, out=outs[t], ws=ws, stream=stream)

    # eager pass with kernel timing (HIP events around every launch on the stream)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    _lib.timing_read()
    d1.flags |= _lib.SDM_FLAG_TIMING
    with torch.cuda.stream(side):
        steps(side)
    torch.cuda.synchronize()
    d1.flags &= ~_lib.SDM_FLAG_TIMING
    per_kernel = {}
    for name, ms in _lib.timing_read(1 << 16):
        per_kernel.setdefault(name, []).append(ms)
    kernels_ms = {k: {"avg": float(np.mean(v)), "launches": len(v)} for k, v in per_kernel.items()}

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n_steps = args.steps * wl.T
    us_step = wall * 1e6 / n_steps
    step_bytes = wl.B * wl.H * wl.slot_bytes_per_token_head(4)
    scan_kernel = next(k for k in ("scan_direct", "gdn_slices", "two_phase_scan", "stream_scan")
                       if k in kernels_ms)
    scan_ms = kernels_ms[scan_kernel]["avg"] * kernels_ms[scan_kernel]["launches"] / wl.T
    achieved = step_bytes / (scan_ms * 1e-3) / 1e9
    gemm_kernel = next((k for k in ("proj_gemm_bf16", "proj_gemm_f32") if k in kernels_ms), None)
    res = {
        "metric": METRIC_DECODE,
        "value": wl.B / (us_step * 1e-6),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": n_steps,
        "warmup": args.warmup * wl.T,
        "ms_per_step": us_step * 1e-3,
        "us_per_step": us_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 projection, fp32 selection/scan",
        "data": "synthetic",
        "rule": args.rule,
        "config": {"workload": wl.name, "B": wl.B, "T": 1, "decode_steps": wl.T,
                   "d_model": wl.d_model, "H": wl.H, "N": wl.N, "n": wl.n, "W": wl.W, "R": wl.R,
                   "d_v": wl.d_v, "state": "fp32 [B,H,N,d_v]", "tokens_per_step": wl.B,
                   "replays": args.steps, "steps_per_replay": wl.T},
        "effective_hbm_gbs_step": step_bytes / (us_step * 1e-6) / 1e9,
        "step_frac_of_peak": step_bytes / (us_step * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "kernels_ms_eager": kernels_ms,
        "gemm": gemm_line(dataclass_replace(wl, T=1), kernels_ms, gemm_kernel, wl.T),
        "roofline": {"bound": "hbm", "kernel": scan_kernel, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None, "algorithmic_bytes_per_launch": step_bytes},
    }
    print(json.dumps(res), flush=True)


def fp8_state_buffer(m):
    """[B, H, N, d_v] fp32 -> the SDM_FLAG_STATE_FP8 buffer of the nearest stored
    values: E4M3 codes (torch's float8_e4m3fn conversion of x 2^-e, exact scaling),
    then per 32-column block the E8M0 byte of e, the least e >= -127 with
    absmax <= 448 2^e."""
    import torch
    blk = m.reshape(*m.shape[:-1], m.shape[-1] // 32, 32)
    mant, k = torch.frexp(blk.abs().amax(-1))
    e = (k - 1) - 8 + (2 * mant > 1.75).to(k.dtype)
    e = torch.where(mant > 0, e.clamp(min=-127), torch.full_like(e, -127))
    codes = torch.ldexp(blk, (-e).unsqueeze(-1).to(blk.dtype)).to(torch.float8_e4m3fn)
    return torch.cat([codes.view(torch.uint8).reshape(-1), (e + 127).to(torch.uint8).reshape(-1)])


def dataclass_replace(wl, **kw):
    import dataclasses
    return dataclasses.replace(wl, **kw)


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
    gdn = args.rule == "gdn"
    if gdn:  # the key-weighted rule: chunk schedule from 256 tokens, else direct
        d.flags |= _lib.SDM_FLAG_DELTA_GDN
    if args.schedule != "default":  # the training forward's schedule (and the backward's)
        d.flags |= {"direct": _lib.SDM_FLAG_SCAN_DIRECT, "stream": _lib.SDM_FLAG_SCAN_STREAM,
                    "two_phase": _lib.SDM_FLAG_SCAN_TWO_PHASE,
                    "chunk": _lib.SDM_FLAG_SCAN_CHUNK}[args.schedule]
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
    ws_sb = torch.empty(max(_lib.workspace_bytes(d, _lib.SDM_ENTRY_SELECT_BACKWARD), 1),
                        dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    gemm_ms = []

    def step(timed=False):
        d_state.copy_(d_state0)
        ops.select(d, x, w, A, b_dt, out=prod, ws=ws_sel, stream=stream)
        _, y, log = ops.scan_train(d, prod, gamma, state, out=out, ws=ws_fwd, stream=stream)
        g = ops.scan_backward(d, prod, gamma, state, d_state, y, log, d_out, ws=ws_bwd,
                              stream=stream)
        d_y, _, _ = ops.select_backward(d, prod, x, w, A, b_dt, g, ws=ws_sb, stream=stream)
        # dx = dY W_proj and dW_proj = dY^T x: plain GEMMs of the projection, in bf16
        # through the platform BLAS
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        dyb = d_y.view(-1, d_y.shape[-1]).to(w.dtype)
        torch.mm(dyb, w)
        torch.mm(dyb.t(), x.view(-1, x.shape[-1]))
        if timed:
            e1.record(stream)
            gemm_ms.append((e0, e1))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    _lib.timing_read()
    d.flags |= _lib.SDM_FLAG_TIMING
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(timed=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    d.flags &= ~_lib.SDM_FLAG_TIMING
    ms_wall = wall * 1e3 / args.steps
    per_kernel = {}
    for name, ms in _lib.timing_read(1 << 16):
        per_kernel.setdefault(name, []).append(ms)
    kernels_ms = {k: {"avg": float(np.mean(v)), "launches": len(v)} for k, v in per_kernel.items()}
    kernels_ms["proj_grad_gemms_blas"] = {
        "avg": float(np.mean([a.elapsed_time(b) for a, b in gemm_ms])), "launches": len(gemm_ms)}
    back = next(k for k in ("stream_backward", "chunk_backward", "gdn_slices_backward",
                            "scan_backward") if k in kernels_ms)
    back_ms = kernels_ms[back]["avg"] * kernels_ms[back]["launches"] / args.steps
    tokens = wl.tokens
    # per token and head: M and dM read, dM written per read; log and dM read, dM and M
    # written per write
    # (either write rule)
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
        "rule": args.rule,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "T": wl.T, "d_model": wl.d_model, "H": wl.H,
                   "N": wl.N, "n": wl.n, "W": wl.W, "R": wl.R, "d_v": wl.d_v,
                   "state": "fp32 [B,H,N,d_v]", "tokens_per_step": tokens,
                   "schedule": args.schedule,
                   "step": "select + scan_train + scan_backward + select_backward + "
                           "dx/dW_proj GEMMs (bf16, platform BLAS)"},
        "kernels_ms": kernels_ms,
        "roofline": {"bound": "hbm", "kernel": back, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": (measured_back_traffic(wl.name) if back == "stream_backward"
                                 else measured_chunk_traffic(wl.name, True)
                                 if back == "chunk_backward" else None),
                     "algorithmic_bytes_per_launch":
                         back_bytes * args.steps / kernels_ms[back]["launches"]},
    }
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, dev, res)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
