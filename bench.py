#!/usr/bin/env python3
"""Throughput of the Gemma-4 26B-A4B mixture-of-experts block on one MI355X.

One step = one pass of the experts-only hot path over one batch of decode
tokens: route (router + dispatch) -> expert gate_up -> expert down -> combine,
each a call into libmoe (the C ABI) on the current stream.  The workload is the 26B-A4B
layer's experts (128 experts, top-8, hidden 2816, expert intermediate 704,
bf16 weights, fp32 router) at a decode batch of 64 tokens; batches of 1, 8 and
32 and a 4096-token prefill are measured the same way and reported in the same
line.

Inputs are seeded and synthetic, generated on the GPU: x ~ N(0,1) bf16,
gate_up / down ~ N(0, 0.02) bf16, router weight N(0, 0.02) fp32,
router_scale = 1, per_expert_scale ~ U(0.5, 1.5).  The 256 MB Infinity Cache
would hold one copy of the weights a small batch touches, so the steps rotate
over several weight copies and several input batches: every step streams its
experts from HBM.

Timing: W untimed warm-up steps, then K steps bracketed by device
synchronisation; HIP events between the calls give each kernel's average
duration on the stream it runs on.  The oracle (CPU) is timed on a bounded
sample of the same workload as a reported baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-block tokens/s on 1 MI355X; % HBM BW (decode) / % bf16 MFMA (prefill)"
H, E, K, I = 2816, 128, 8, 704
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
GATE_UP_BYTES = 2 * I * H * 2     # one expert's gate_up, bf16
DOWN_BYTES = H * I * 2            # one expert's down, bf16
ROUTER_BYTES = E * H * 4 + H * 4 + E * 4
KERNEL_SRC = os.path.join(ROOT, "sparse_moe_transformer_router_amd", "csrc", "expert_stream.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_decode_b64_traffic.txt")
SEGMENTS = ("route", "gate_up", "down", "combine")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--batch", type=int, default=64, help="decode tokens per step (headline)")
    ap.add_argument("--sweep", default="1,8,32", help="other decode batches to report")
    ap.add_argument("--prefill", type=int, default=4096, help="prefill tokens (0 = skip)")
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated over")
    ap.add_argument("--xbatches", type=int, default=16, help="input batches rotated over")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (for counter calibration)")
    ap.add_argument("--seed", type=int, default=0)
    return ap.parse_args()


class Workload:
    """Resident weights (several copies) and input batches on the GPU."""

    def __init__(self, torch, lib, copies, seed):
        self.torch, self.lib = torch, lib
        dev = torch.device("cuda")
        self.copies = []
        for c in range(copies):
            g = torch.Generator(device=dev)
            g.manual_seed(1_000_003 * seed + 7919 * c + 1)
            gu = torch.randn(E, 2 * I, H, generator=g, device=dev).mul_(0.02).to(torch.bfloat16)
            dn = torch.randn(E, H, I, generator=g, device=dev).mul_(0.02).to(torch.bfloat16)
            rw = torch.randn(E, H, generator=g, device=dev).mul_(0.02)
            rs = torch.ones(H, device=dev)
            pes = torch.rand(E, generator=g, device=dev).add_(0.5)
            self.copies.append((rw, rs, pes, gu, dn))
        torch.cuda.synchronize()
        self.dims = lib.dims(H, E, K, I, 0, 1e-6, lib.MOE_BF16, lib.MOE_F32)

    def batches(self, T, n, seed):
        torch = self.torch
        g = torch.Generator(device="cuda")
        g.manual_seed(1_000_033 * seed + T)
        return [torch.randn(T, H, generator=g, device="cuda").to(torch.bfloat16) for _ in range(n)]


class Runner:
    """Buffers for one batch size and the per-step call sequence."""

    def __init__(self, wl: Workload, T: int):
        torch, lib = wl.torch, wl.lib
        self.wl, self.T = wl, T
        S = T * K
        self.ws = lib.workspace(wl.dims, T)
        self.idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
        self.w = torch.empty(T, K, dtype=torch.float32, device="cuda")
        self.counts = torch.empty(E, dtype=torch.int32, device="cuda")
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        self.sorted = torch.empty(S, dtype=torch.int32, device="cuda")
        self.h = torch.empty(S, I, dtype=torch.bfloat16, device="cuda")
        self.y = torch.empty(S, H, dtype=torch.float32, device="cuda")
        self.out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")

    def step(self, x, copy, ev=None):
        lib, d, T = self.wl.lib, self.wl.dims, self.T
        rw, rs, pes, gu, dn = copy
        rec = (lambda j: ev[j].record()) if ev is not None else (lambda j: None)
        rec(0)
        lib.moe_route(d, T, x, rw, rs, pes, None, self.idx, self.w, self.counts, self.offsets,
                      self.sorted, self.ws)
        rec(1)
        lib.moe_expert_gate_up(d, T, x, gu, self.offsets, self.sorted, self.h)
        rec(2)
        lib.moe_expert_down(d, T, self.h, dn, self.w, self.offsets, self.sorted, self.y)
        rec(3)
        lib.moe_combine(d, T, self.y, None, self.out)
        rec(4)


def time_steps(torch, runner, xs, copies, steps, warmup):
    """Warm-up, then `steps` timed steps; returns (ms per step, per-segment ms, pairs used)."""
    n_ev = len(SEGMENTS) + 1
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(steps)]
    for i in range(warmup):
        runner.step(xs[i % len(xs)], copies[i % len(copies)])
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pairs = []
    start.record()
    for i in range(steps):
        j = warmup + i
        pairs.append((j % len(xs), j % len(copies)))
        runner.step(xs[j % len(xs)], copies[j % len(copies)], events[i])
    end.record()
    torch.cuda.synchronize()
    total = start.elapsed_time(end)
    seg = {name: sum(events[i][s].elapsed_time(events[i][s + 1]) for i in range(steps)) / steps
           for s, name in enumerate(SEGMENTS)}
    return total / steps, seg, pairs


def distinct_experts(torch, runner, xs, copies, pairs):
    """Average number of distinct experts a step touches (from its routing)."""
    us = []
    for xi, ci in sorted(set(pairs)):
        runner.step(xs[xi], copies[ci])
        torch.cuda.synchronize()
        us.append(int((runner.counts > 0).sum().item()))
    return sum(us) / len(us)


def decode_measure(torch, wl, T, steps, warmup, xbatches, seed):
    runner = Runner(wl, T)
    xs = wl.batches(T, xbatches, seed)
    ms, seg, pairs = time_steps(torch, runner, xs, wl.copies, steps, warmup)
    U = distinct_experts(torch, runner, xs, wl.copies, pairs)
    gate_up_bytes = U * GATE_UP_BYTES + T * H * 2
    step_bytes = U * (GATE_UP_BYTES + DOWN_BYTES) + ROUTER_BYTES + 2 * T * H * 2
    return {
        "tokens": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
        "distinct_experts": U, "kernel_ms": seg,
        "step_hbm_frac": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "gate_up_gbs": gate_up_bytes / (seg["gate_up"] * 1e-3) / 1e9,
        "gate_up_bytes": gate_up_bytes,
    }, runner, xs


def prefill_measure(torch, wl, T, steps, warmup, seed):
    runner = Runner(wl, T)
    xs = wl.batches(T, 2, seed + 1)
    ms, seg, _ = time_steps(torch, runner, xs, wl.copies, steps, warmup)
    flops = T * K * 6 * H * I
    gemm_ms = seg["gate_up"] + seg["down"]
    return {
        "tokens": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "kernel_ms": seg,
        "grouped_gemm_tflops": flops / (gemm_ms * 1e-3) / 1e12,
        "grouped_gemm_mfma_frac": flops / (gemm_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "gate_up_tflops": flops * 2 / 3 / (seg["gate_up"] * 1e-3) / 1e12,
        "down_tflops": flops / 3 / (seg["down"] * 1e-3) / 1e12,
    }


def cpu_baseline(torch, wl, xs, T, seconds):
    """The oracle as it stands, on the host cores: router + sparse experts for
    the first decode batch, repeated for about `seconds`."""
    import numpy as np
    import oracle

    rw, rs, pes, gu, dn = wl.copies[0]
    f = lambda t: t.float().cpu().numpy()  # noqa: E731
    x = f(xs[0])
    args = (f(rw), f(rs), f(pes))
    gu32, dn32 = f(gu), f(dn)
    n, t0 = 0, time.perf_counter()
    while True:
        idx, w = oracle.router(x, *args, K)
        oracle.experts(x, gu32, dn32, idx, w)
        n += T
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    del gu32, dn32
    return {"value": n / el, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"router + sparse experts (fp64 loop) on the first {T}-token decode batch of "
                      f"weight copy 0, repeated {n // T}x over {el:.1f} s"}


def traffic_from_profile():
    """HBM bytes per gate_up launch from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        rec = json.loads(open(TRAFFIC_FILE).read().split("---json---")[1])
    except (IndexError, ValueError):
        return None
    sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    return rec.get("bytes_per_launch") if rec.get("kernel_src_sha256") == sha else None


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures a single MI355X: the path is built and measured on one GPU "
              "(no collectives or sharding); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_moe_transformer_router_amd import lib

    torch.cuda.set_device(0)
    wl = Workload(torch, lib, args.copies, args.seed)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    head, runner, xs = decode_measure(torch, wl, args.batch, args.steps, args.warmup,
                                      args.xbatches, args.seed)
    sweep = {}
    for b in [int(v) for v in args.sweep.split(",") if v.strip()]:
        if b != args.batch:
            r, _, _ = decode_measure(torch, wl, b, args.steps, args.warmup, args.xbatches,
                                     args.seed)
            sweep[str(b)] = r
    prefill = None
    if args.prefill > 0:
        prefill = prefill_measure(torch, wl, args.prefill, max(5, args.steps // 5),
                                  max(2, args.warmup // 5), args.seed)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(torch, wl, xs, args.batch, args.cpu_seconds)

    achieved = head["gate_up_gbs"]
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"Gemma-4 26B-A4B MoE experts, decode batch {args.batch} tokens",
                   "tokens": args.batch, "experts": E, "top_k": K, "hidden": H,
                   "expert_inter": I, "weights": "bf16", "router": "fp32",
                   "weight_copies_rotated": args.copies, "input_batches_rotated": args.xbatches},
        "roofline": {"bound": "hbm", "kernel": "gate_up_stream_kernel (expert gate_up + GELU, decode)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_from_profile(),
                     "algorithmic_bytes_per_launch": head["gate_up_bytes"],
                     "avg_launch_ms": head["kernel_ms"]["gate_up"]},
        "cpu_baseline": cpu,
        "decode": {str(args.batch): head, **sweep},
        "prefill": prefill,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
