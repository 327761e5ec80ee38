#!/usr/bin/env python3
"""Throughput of the Gemma-4 26B-A4B mixture-of-experts block on one MI355X.

One step = one pass of the experts-only hot path over one batch of decode
tokens: route (router + dispatch) -> expert gate_up -> expert down -> combine,
each a call into libmoe (the C ABI) on the current stream.  The workload is the 26B-A4B
layer's experts (128 experts, top-8, hidden 2816, expert intermediate 704,
bf16 weights, fp32 router) at a decode batch of 64 tokens; batches of 1, 8 and
32 and a 4096-token prefill are measured the same way and reported in the same
line.

Inputs are seeded and synthetic: x ~ N(0,1) bf16, gate_up / down ~ N(0, 0.02)
bf16, router weight N(0, 0.02) fp32, router_scale = 1, per_expert_scale ~
U(0.5, 1.5).  Weight copy 0 and the first input batch of each leg come from
the same seeded generator as the parity tests (synth.py), and the CPU-baseline
leg checks the GPU's result on those exact bits against the oracle; the
other copies and batches are drawn on the GPU.  The 256 MB Infinity Cache
would hold one copy of the weights a small batch touches, so the steps rotate
over several weight copies and several input batches: every step streams its
experts from HBM.

Also reported in the same line: the tiny fp32 configuration (16 tokens,
hidden 64, 8 experts, top-2); the whole FFN block (pre-norms, router on the
normed input, experts, gated dense MLP of width 2112, five norms, residual,
layer scalar) at 2048 tokens; and a stack of 30 independently seeded blocks
(decode: 64 tokens, each step's input the previous step's output; prefill:
8192 tokens once through the stack).  Block norm gains are 1 + N(0, 0.02),
dense weights N(0, 0.02) bf16, layer scalar 0.06.

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
GATE_UP_SAMPLE = 5  # the timed region times gate_up on every 5th step
D = 2112                          # dense MLP width of the block
DENSE_BYTES = 3 * D * H * 2       # dense gate, up, down, bf16
LAYERS = 30


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--batch", type=int, default=64, help="decode tokens per step (headline)")
    ap.add_argument("--sweep", default="1,8,32,128,256", help="other decode batches to report")
    ap.add_argument("--prefill", type=int, default=4096, help="prefill tokens (0 = skip)")
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated over")
    ap.add_argument("--xbatches", type=int, default=16, help="input batches rotated over")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (for counter calibration)")
    ap.add_argument("--block", type=int, default=2048, help="whole-block tokens (0 = skip)")
    ap.add_argument("--stack", type=int, default=LAYERS, help="layers in the stack run (0 = skip)")
    ap.add_argument("--stack-steps", type=int, default=128, help="timed decode steps of the stack")
    ap.add_argument("--stack-prefill", type=int, default=8192, help="stack prefill tokens (0 = skip)")
    ap.add_argument("--dense-mask", type=int, default=1,
                    help="time the all-experts ablation at the decode and prefill sizes (0 = skip)")
    ap.add_argument("--quant", type=int, default=1,
                    help="time the int8 / E4M3 / MXFP4 expert legs (0 = skip)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--clock-warmup", type=float, default=1.0,
                    help="seconds of untimed decode steps before the first leg, so that the "
                         "GPU clock has left its idle level (0 = none)")
    return ap.parse_args()


def _upload_bf16(torch, t):
    """A synth bf16 tensor (its bit pattern) on the GPU."""
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(t.bf16).view(np.int16)).cuda().view(
        torch.bfloat16)


class Workload:
    """Resident weights (several copies) and input batches on the GPU.

    Copy 0 and the first input batch of every size are drawn by the seeded
    generator the parity tests use (synth.py, numpy PCG64 per tensor), so the
    timed configuration is the one the tests check against the oracle, bit
    for bit; the other copies and batches (there only to keep the 256 MB
    Infinity Cache from serving the weights) are drawn on the GPU with the
    same distributions."""

    def __init__(self, torch, lib, copies, seed):
        from sparse_moe_transformer_router_amd import synth

        self.torch, self.lib, self.seed = torch, lib, seed
        dev = torch.device("cuda")
        rw, rs, pes = synth.moe_router_weights(seed)
        gu, dn = synth.moe_expert_weights(seed)
        self.copies = [(torch.from_numpy(rw).cuda(), torch.from_numpy(rs).cuda(),
                        torch.from_numpy(pes).cuda(), _upload_bf16(torch, gu),
                        _upload_bf16(torch, dn))]
        del gu, dn
        for c in range(1, copies):
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

    def batches(self, T, n, seed, skew=False):
        """n input batches of T tokens; the first is synth's x of this seed."""
        from sparse_moe_transformer_router_amd import synth

        torch = self.torch
        g = torch.Generator(device="cuda")
        g.manual_seed(1_000_033 * seed + T)
        xs = [_upload_bf16(torch, synth.moe_x(T, seed, skew=skew))]
        xs += [torch.randn(T, H, generator=g, device="cuda").to(torch.bfloat16)
               for _ in range(n - 1)]
        if skew:
            for x in xs[1:]:
                x[:, 0] = 1.0
        return xs


class Runner:
    """Buffers for one batch size and the per-step call sequence.  Events 1
    and 2 of a step (gate_up's start and end) are recorded by the gate_up
    kernel's own dispatch (moe_expert_gate_up_timed), so they put no packets
    between the launches."""

    timed_gate_up = True

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
        rec = (lambda j: ev[j] is not None and ev[j].record()) if ev is not None \
            else (lambda j: None)
        rec(0)
        lib.moe_route(d, T, x, rw, rs, pes, None, self.idx, self.w, self.counts, self.offsets,
                      self.sorted, self.ws)
        if ev is not None and ev[1] is not None and ev[2] is not None:
            lib.moe_expert_gate_up_timed(d, T, x, gu, self.offsets, self.sorted, self.h, ev[1],
                                         ev[2])
        else:
            lib.moe_expert_gate_up(d, T, x, gu, self.offsets, self.sorted, self.h)
        lib.moe_expert_down(d, T, self.h, dn, self.w, self.offsets, self.sorted, self.y)
        rec(3)
        lib.moe_combine(d, T, self.y, None, self.out)
        rec(4)


def time_steps(torch, runner, xs, copies, steps, warmup, leg=None):
    """Warm-up, then `steps` timed steps, then `steps` instrumented steps.

    The timed region's only HIP events, besides the two around the whole
    region, are gate_up's start and end (the roofline kernel) on every
    GATE_UP_SAMPLE-th step, recorded by the kernel's own dispatch when the
    runner supports it.  Any event attached to a launch leaves the GPU idle
    around it (~6.5 us before gate_up and ~4.6 us after it in the kernel
    trace, against none between unrecorded launches), so recording every step
    would understate the step rate by ~4%.  The other segments' times come
    from the instrumented pass that follows.  Returns (ms per step,
    per-segment ms with gate_up from the timed region's sampled launches when
    the runner times it there, pairs of input / weight copy used in the timed
    region)."""
    n_ev = len(SEGMENTS) + 1
    timed = getattr(runner, "timed_gate_up", False)
    for i in range(warmup):
        runner.step(xs[i % len(xs)], copies[i % len(copies)])
    torch.cuda.synchronize()
    gev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(steps)]
    for e in [e for row in gev + events for e in row]:
        e.record()  # torch creates an event at its first record
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pairs = []
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        j = warmup + i
        pairs.append((j % len(xs), j % len(copies)))
        sampled = timed and i % GATE_UP_SAMPLE == 0
        runner.step(xs[j % len(xs)], copies[j % len(copies)],
                    [None, gev[i][0], gev[i][1]] + [None] * (n_ev - 3) if sampled else None)
    end.record()
    torch.cuda.synchronize()
    if leg is not None:
        WINDOWS[leg] = (t0, time.perf_counter())
    total = start.elapsed_time(end)
    for i in range(steps):
        j = warmup + steps + i
        runner.step(xs[j % len(xs)], copies[j % len(copies)], events[i])
    torch.cuda.synchronize()
    seg = {name: sum(events[i][s].elapsed_time(events[i][s + 1]) for i in range(steps)) / steps
           for s, name in enumerate(SEGMENTS)}
    if timed:
        samp = [g[0].elapsed_time(g[1]) for i, g in enumerate(gev) if i % GATE_UP_SAMPLE == 0]
        seg["gate_up"] = sum(samp) / len(samp)
    return total / steps, seg, pairs


def distinct_experts(torch, runner, xs, copies, pairs):
    """Average over the given steps (pairs of input / weight copy) of the
    number of distinct experts a step touches (from its routing)."""
    u = {}
    for xi, ci in sorted(set(pairs)):
        runner.step(xs[xi], copies[ci])
        torch.cuda.synchronize()
        u[(xi, ci)] = int((runner.counts > 0).sum().item())
    return sum(u[p] for p in pairs) / len(pairs)


def decode_measure(torch, wl, T, steps, warmup, xbatches, seed):
    runner = Runner(wl, T)
    xs = wl.batches(T, xbatches, seed)
    ms, seg, pairs = time_steps(torch, runner, xs, wl.copies, steps, warmup, f"decode_{T}")
    U = distinct_experts(torch, runner, xs, wl.copies, pairs)
    # the gate_up launches timed are those of every GATE_UP_SAMPLE-th step
    U_timed = distinct_experts(torch, runner, xs, wl.copies, pairs[::GATE_UP_SAMPLE])
    gate_up_bytes = U_timed * GATE_UP_BYTES + T * H * 2
    step_bytes = U * (GATE_UP_BYTES + DOWN_BYTES) + ROUTER_BYTES + 2 * T * H * 2
    return {
        "tokens": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
        "distinct_experts": U, "distinct_experts_gate_up_timed": U_timed, "kernel_ms": seg,
        "step_hbm_frac": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "gate_up_gbs": gate_up_bytes / (seg["gate_up"] * 1e-3) / 1e9,
        "gate_up_bytes": gate_up_bytes,
    }, runner, xs


def skewed_inputs(torch, wl, T, seed):
    """Two input batches and the weight copies with the per-expert logit bias
    b_e ~ N(0, 1) realised through the data (channel 0 of every token = 1,
    router weight column 0 = b).  Batch 0 with copy 0 is synth's skewed case
    of this seed, the inputs the 4096-token parity test checks."""
    from sparse_moe_transformer_router_amd import synth

    xs = wl.batches(T, 2, seed, skew=True)
    rw_skew, _, _ = synth.moe_router_weights(seed, skew=True)
    bias = torch.from_numpy(rw_skew[:, 0].copy()).cuda()
    copies = []
    for rw, rs, pes, gu, dn in wl.copies:
        rwb = rw.clone()
        rwb[:, 0] = bias
        copies.append((rwb, rs, pes, gu, dn))
    return xs, copies


def prefill_measure(torch, wl, T, steps, warmup, seed):
    """The prefill batch with imbalanced expert load: a per-expert logit bias
    b_e ~ N(0, 1), realised through the data as channel 0 of every token set
    to 1 and router weight column 0 set to b."""
    runner = Runner(wl, T)
    xs, copies = skewed_inputs(torch, wl, T, seed)
    ms, seg, _ = time_steps(torch, runner, xs, copies, steps, warmup, f"prefill_{T}")
    runner.step(xs[0], copies[0])
    torch.cuda.synchronize()
    counts = runner.counts.cpu()
    flops = T * K * 6 * H * I
    gemm_ms = seg["gate_up"] + seg["down"]
    return {
        "tokens": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), "kernel_ms": seg,
        "expert_load": {"max": int(counts.max()), "empty": int((counts == 0).sum()),
                        "top8_share": float(counts.sort(descending=True).values[:8].sum() / (T * K))},
        "grouped_gemm_tflops": flops / (gemm_ms * 1e-3) / 1e12,
        "grouped_gemm_mfma_frac": flops / (gemm_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "gate_up_tflops": flops * 2 / 3 / (seg["gate_up"] * 1e-3) / 1e12,
        "down_tflops": flops / 3 / (seg["down"] * 1e-3) / 1e12,
    }


class DenseMaskRunner:
    """The all-experts form on the same kernels: route (top-K), the
    all-experts slot layout (every expert takes every token, weight 0 outside
    the token's top-K), the experts over all T * E slots, and the combine
    over E slots per token."""

    def __init__(self, wl: Workload, T: int):
        torch, lib = wl.torch, wl.lib
        self.wl, self.T = wl, T
        self.sparse = Runner(wl, T)
        self.dd = lib.dims(H, E, E, I, 0, 1e-6, lib.MOE_BF16, lib.MOE_F32)
        self.ws = lib.workspace(self.dd, T)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        self.sorted = torch.empty(T * E, dtype=torch.int32, device="cuda")
        self.wd = torch.empty(T * E, dtype=torch.float32, device="cuda")
        self.y = torch.empty(T * E, H, dtype=torch.float32, device="cuda")
        self.out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")

    def step(self, x, copy, ev=None):
        lib, d, T, sp = self.wl.lib, self.wl.dims, self.T, self.sparse
        rw, rs, pes, gu, dn = copy
        rec = (lambda j: ev[j] is not None and ev[j].record()) if ev is not None \
            else (lambda j: None)
        rec(0)
        lib.moe_route(d, T, x, rw, rs, pes, None, sp.idx, sp.w, sp.counts, sp.offsets,
                      sp.sorted, sp.ws)
        lib.moe_dense_mask_dispatch(d, T, sp.idx, sp.w, self.offsets, self.sorted, self.wd)
        rec(1)
        lib.moe_expert_ffn(self.dd, T, x, gu, dn, self.wd, self.offsets, self.sorted, self.y,
                           self.ws)
        rec(2)
        rec(3)
        lib.moe_combine(self.dd, T, self.y, None, self.out)
        rec(4)


def dense_mask_measure(torch, wl, T, steps, warmup, xbatches, seed, sparse_ms):
    """The all-experts ablation at T tokens against the sparse path's step time."""
    runner = DenseMaskRunner(wl, T)
    xs = wl.batches(T, xbatches, seed)
    ms, seg, _ = time_steps(torch, runner, xs, wl.copies, steps, warmup, f"all_experts_{T}")
    flops = T * E * 6 * H * I
    return {
        "tokens": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
        "kernel_ms": {"route_and_layout": seg["route"], "experts": seg["gate_up"],
                      "combine": seg["combine"]},
        "expert_flops_executed": flops, "expert_flops_useful": flops * K // E,
        "experts_tflops_executed": flops / (seg["gate_up"] * 1e-3) / 1e12,
        "experts_mfma_frac_executed": flops / (seg["gate_up"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "sparse_ms_per_step": sparse_ms,
        "sparse_speedup": ms / sparse_ms,
    }


QUANT_FORMATS = {
    # name: (format code, weights per byte, scale bytes per weight row of length n, description)
    "int8": (1, 1, lambda n: 4, "int8 per-channel symmetric"),
    "fp8": (2, 1, lambda n: 4, "E4M3 per-channel (OCP FP8)"),
    "mxfp4": (3, 2, lambda n: n // 32, "MXFP4 (E2M1, E8M0 scale per 32 weights)"),
}


def quant_decode_measure(torch, lib, wl, name, T, steps, warmup, xbatches, seed, native=False,
                         skew=False):
    """Decode with the experts' weights quantized on the GPU (from the same
    weight copies) into one of QUANT_FORMATS: route, experts, combine.  With
    native, the experts run on the 8-bit / 4-bit matrix instructions with
    MXFP8 activations (moe_expert_ffn_mx) instead of widening the codes.
    With skew, the inputs and router weights of the skewed prefill leg."""
    fmt, per_byte, sbytes, desc = QUANT_FORMATS[name]
    experts = lib.moe_expert_ffn_mx if native else lib.moe_expert_ffn_q

    def quant(wt):
        rows, n = wt.numel() // wt.shape[-1], wt.shape[-1]
        q = torch.empty(rows * n // per_byte, dtype=torch.uint8, device="cuda")
        if fmt == 3:
            sc = torch.empty(rows * n // 32, dtype=torch.uint8, device="cuda")
        else:
            sc = torch.empty(rows, dtype=torch.float32, device="cuda")
        lib.moe_quantize(fmt, wt, q, sc)
        return q, sc

    if skew:
        xs, copies = skewed_inputs(torch, wl, T, seed)
    else:
        xs, copies = wl.batches(T, xbatches, seed), wl.copies
    qcopies = []
    for rw, rs, pes, gu, dn in copies:
        qcopies.append((rw, rs, pes, *quant(gu), *quant(dn)))
    torch.cuda.synchronize()
    r = Runner(wl, T)
    d = wl.dims

    def step(i, ev=None):
        rw, rs, pes, guq, gus, dnq, dns = qcopies[i % len(qcopies)]
        x = xs[i % len(xs)]
        if ev is not None:
            ev[0].record()
        lib.moe_route(d, T, x, rw, rs, pes, None, r.idx, r.w, r.counts, r.offsets, r.sorted, r.ws)
        if ev is not None:
            ev[1].record()
        experts(d, fmt, T, x, guq, gus, dnq, dns, r.w, r.offsets, r.sorted, r.y, r.ws)
        if ev is not None:
            ev[2].record()
        lib.moe_combine(d, T, r.y, None, r.out)
        if ev is not None:
            ev[3].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for i in range(steps):
        step(warmup + i)
    b.record()
    torch.cuda.synchronize()
    WINDOWS[f"{name}{'_native' if native else ''}_decode_{T}"] = (t0, time.perf_counter())
    ms = a.elapsed_time(b) / steps
    # per-segment times from an instrumented pass after the timed region
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        step(warmup + steps + i, evs[i])
    torch.cuda.synchronize()
    seg = {nm: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps
           for j, nm in enumerate(("route", "experts", "combine"))}
    us = []
    for i in range(len(qcopies)):
        step(i)
        torch.cuda.synchronize()
        us.append(int((r.counts > 0).sum().item()))
    U = sum(us) / len(us)
    # codes + scales of one expert's gate_up (2I rows of H) and down (H rows of I)
    per_expert = (2 * I * H + H * I) // per_byte + 2 * I * sbytes(H) + H * sbytes(I)
    expert_bytes = U * per_expert + T * H * 2
    step_bytes = U * per_expert + ROUTER_BYTES + 2 * T * H * 2
    flops = T * K * 6 * H * I
    # dense matrix peak (TFLOP/s): 8-bit / 4-bit-by-8-bit, or bf16 for the
    # widened codes
    peak = 5000.0 if native else 2500.0
    extra = {}
    if T > 256:
        tf = flops / (seg["experts"] * 1e-3) / 1e12
        extra = {"experts_tflops": tf,
                 ("experts_frac_of_fp8_mfma_peak" if native
                  else "experts_frac_of_bf16_mfma_peak"): tf / peak}
    return {"tokens": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3), **extra,
            "distinct_experts": U, "kernel_ms": seg, "weights": desc,
            "matrix_path": ("8-bit / 4-bit scaled matrix instructions, MXFP8 activations"
                            if native else "codes widened to bf16, bf16 matrix instructions"),
            "expert_bytes_per_expert": per_expert,
            "experts_gbs": expert_bytes / (seg["experts"] * 1e-3) / 1e9,
            "experts_hbm_frac": expert_bytes / (seg["experts"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "step_hbm_frac": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


class BlockLayer:
    """One block's weights (resident on the GPU) and its C-ABI weight struct."""

    def __init__(self, torch, lib, seed, layer):
        dev = torch.device("cuda")
        g = torch.Generator(device=dev)
        g.manual_seed(1_000_037 * seed + 104_729 * layer + 17)
        rnd = lambda *shape: torch.randn(*shape, generator=g, device=dev)  # noqa: E731
        self.gains = [rnd(H).mul_(0.02).add_(1.0) for _ in range(5)]
        self.dense = [rnd(D, H).mul_(0.02).to(torch.bfloat16), rnd(D, H).mul_(0.02).to(torch.bfloat16),
                      rnd(H, D).mul_(0.02).to(torch.bfloat16)]
        self.rw = rnd(E, H).mul_(0.02)
        self.rs = torch.ones(H, device=dev)
        self.pes = torch.rand(E, generator=g, device=dev).add_(0.5)
        self.gu = rnd(E, 2 * I, H).mul_(0.02).to(torch.bfloat16)
        self.dn = rnd(E, H, I).mul_(0.02).to(torch.bfloat16)
        self.w = lib.ffn_weights(*self.gains, *self.dense, self.rw, self.rs, self.pes, self.gu,
                                 self.dn, 0.06)


class BlockRunner:
    """Buffers for the whole block at T tokens."""

    def __init__(self, torch, lib, T):
        self.lib, self.T = lib, T
        self.dims = lib.dims(H, E, K, I, D, 1e-6, lib.MOE_BF16, lib.MOE_F32)
        self.ws = lib.workspace(self.dims, T)
        self.idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
        self.w = torch.empty(T, K, dtype=torch.float32, device="cuda")

    def step(self, x, layer, out):
        self.lib.gemma4_ffn_block(self.dims, self.T, x, layer.w, out, None, self.idx, self.w,
                                  self.ws)


def block_bytes(U, T):
    """Algorithmic HBM bytes of one block call: the touched experts, the dense
    MLP, the router, the input and the output."""
    return U * (GATE_UP_BYTES + DOWN_BYTES) + DENSE_BYTES + ROUTER_BYTES + 2 * T * H * 2


def block_flops(T):
    return T * K * 6 * H * I + T * 6 * H * D


def block_measure(torch, lib, T, steps, warmup, seed, layers):
    """The whole block at T tokens, rotating over the given layers' weights."""
    br = BlockRunner(torch, lib, T)
    g = torch.Generator(device="cuda")
    g.manual_seed(1_000_039 * seed + T)
    xs = [torch.randn(T, H, generator=g, device="cuda").to(torch.bfloat16) for _ in range(2)]
    out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    for i in range(warmup):
        br.step(xs[i % 2], layers[i % len(layers)], out)
    torch.cuda.synchronize()
    us = []
    for i in range(len(layers)):
        br.step(xs[0], layers[i], out)
        torch.cuda.synchronize()
        us.append(int(torch.unique(br.idx).numel()))
    U = sum(us) / len(us)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        br.step(xs[i % 2], layers[i % len(layers)], out)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    byts, fl = block_bytes(U, T), block_flops(T)
    return {"tokens": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
            "distinct_experts": U, "hbm_bytes": byts, "flops": fl,
            "hbm_frac": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "mfma_frac": fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "binding": "hbm" if byts / HBM_PEAK_GBS * 1e3 > fl / BF16_PEAK_TFLOPS else "mfma"}


def block_quant_measure(torch, lib, layers, T, steps, warmup, seed):
    """The whole layer at a decode batch with its expert and dense-MLP weights
    in each of QUANT_FORMATS (gemma4_ffn_block_q), quantized on the GPU from
    the layers' bf16 weights, beside the bf16 layer on the same weights."""
    res = {"bf16": block_measure(torch, lib, T, steps, warmup, seed, layers)}
    dims = lib.dims(H, E, K, I, D, 1e-6, lib.MOE_BF16, lib.MOE_F32)
    ws = lib.workspace(dims, T)
    g = torch.Generator(device="cuda")
    g.manual_seed(1_000_039 * seed + T)
    xs = [torch.randn(T, H, generator=g, device="cuda").to(torch.bfloat16) for _ in range(2)]
    out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    for name, (fmt, per_byte, sbytes, desc) in QUANT_FORMATS.items():
        def quant(wt):
            rows, n = wt.numel() // wt.shape[-1], wt.shape[-1]
            q = torch.empty(rows * n // per_byte, dtype=torch.uint8, device="cuda")
            sc = (torch.empty(rows * n // 32, dtype=torch.uint8, device="cuda") if fmt == 3
                  else torch.empty(rows, dtype=torch.float32, device="cuda"))
            lib.moe_quantize(fmt, wt, q, sc)
            return q, sc
        qlayers = []
        for ly in layers:
            mats = [*quant(ly.dense[0]), *quant(ly.dense[1]), *quant(ly.dense[2])]
            exp = [*quant(ly.gu), *quant(ly.dn)]
            keep = (*ly.gains, *mats, ly.rw, ly.rs, ly.pes, *exp)
            qlayers.append((keep, lib.ffn_weights_q(fmt, *keep, 0.06)))
        torch.cuda.synchronize()

        def step(i):
            lib.gemma4_ffn_block_q(dims, T, xs[i % 2], qlayers[i % len(qlayers)][1], out, None,
                                   idx, None, ws)
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        us = []
        for i in range(len(qlayers)):
            step(i)
            torch.cuda.synchronize()
            us.append(int(torch.unique(idx).numel()))
        U = sum(us) / len(us)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        a.record()
        for i in range(steps):
            step(i)
        b.record()
        torch.cuda.synchronize()
        WINDOWS[f"block_{name}_{T}"] = (t0, time.perf_counter())
        ms = a.elapsed_time(b) / steps
        per_expert = (2 * I * H + H * I) // per_byte + 2 * I * sbytes(H) + H * sbytes(I)
        dense = (3 * D * H) // per_byte + 2 * D * sbytes(H) + H * sbytes(D)
        byts = U * per_expert + dense + ROUTER_BYTES + 2 * T * H * 2
        res[name] = {"tokens": T, "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
                     "distinct_experts": U, "weights": desc, "hbm_bytes": byts,
                     "hbm_frac": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "speedup_vs_bf16": res["bf16"]["ms_per_step"] / ms}
        del qlayers
        torch.cuda.empty_cache()
    return res


def stack_measure(torch, lib, layers, T_dec, steps, T_pre, seed):
    """A stack of independently seeded blocks: decode steps whose input is the
    previous step's output, and one prefill pass."""
    n = len(layers)
    res = {"layers": n}
    g = torch.Generator(device="cuda")
    g.manual_seed(1_000_081 * seed + 5)
    br = BlockRunner(torch, lib, T_dec)
    x = torch.randn(T_dec, H, generator=g, device="cuda").to(torch.bfloat16)
    bufs = [x.clone(), torch.empty_like(x)]

    def one_step(cur):
        for li, layer in enumerate(layers):
            br.step(bufs[(cur + li) % 2], layer, bufs[(cur + li + 1) % 2])
        return (cur + n) % 2

    cur = 0
    us = []
    for li, layer in enumerate(layers):  # warm-up step; distinct experts per layer
        br.step(bufs[(cur + li) % 2], layer, bufs[(cur + li + 1) % 2])
        us.append(int(torch.unique(br.idx).numel()))
    cur = n % 2
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        cur = one_step(cur)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    finite = bool(torch.isfinite(bufs[cur].float()).all().item())
    U = sum(us) / len(us)
    byts = n * block_bytes(U, T_dec)
    res["decode"] = {"tokens": T_dec, "steps": steps, "ms_per_step": ms,
                     "tokens_per_s": T_dec / (ms * 1e-3), "output_finite": finite,
                     "distinct_experts_per_layer": U, "hbm_bytes_per_step": byts,
                     "per_layer_hbm_frac": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    del br, bufs
    if T_pre > 0:
        br = BlockRunner(torch, lib, T_pre)
        x = torch.randn(T_pre, H, generator=g, device="cuda").to(torch.bfloat16)
        bufs = [x, torch.empty_like(x)]
        for li, layer in enumerate(layers):  # warm-up pass
            br.step(bufs[li % 2], layer, bufs[(li + 1) % 2])
        torch.cuda.synchronize()
        a.record()
        for li, layer in enumerate(layers):
            br.step(bufs[li % 2], layer, bufs[(li + 1) % 2])
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        fl = n * block_flops(T_pre)
        res["prefill"] = {"tokens": T_pre, "ms": ms, "tokens_per_s": T_pre / (ms * 1e-3),
                          "flops": fl, "mfma_frac": fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
        del br, bufs
    return res


def stack_quant_decode(torch, lib, layers, T, steps, seed, name="int8"):
    """The stack's decode steps with every layer's expert and dense-MLP weights
    quantized on the GPU (gemma4_ffn_block_q), each step's input the previous
    step's output, as in stack_measure."""
    fmt, per_byte, sbytes, desc = QUANT_FORMATS[name]
    dims = lib.dims(H, E, K, I, D, 1e-6, lib.MOE_BF16, lib.MOE_F32)
    ws = lib.workspace(dims, T)

    def quant(wt):
        rows, n = wt.numel() // wt.shape[-1], wt.shape[-1]
        q = torch.empty(rows * n // per_byte, dtype=torch.uint8, device="cuda")
        sc = (torch.empty(rows * n // 32, dtype=torch.uint8, device="cuda") if fmt == 3
              else torch.empty(rows, dtype=torch.float32, device="cuda"))
        lib.moe_quantize(fmt, wt, q, sc)
        return q, sc
    ql = []
    for ly in layers:
        keep = (*ly.gains, *quant(ly.dense[0]), *quant(ly.dense[1]), *quant(ly.dense[2]), ly.rw,
                ly.rs, ly.pes, *quant(ly.gu), *quant(ly.dn))
        ql.append((keep, lib.ffn_weights_q(fmt, *keep, 0.06)))
    g = torch.Generator(device="cuda")
    g.manual_seed(1_000_081 * seed + 7)
    bufs = [torch.randn(T, H, generator=g, device="cuda").to(torch.bfloat16), None]
    bufs[1] = torch.empty_like(bufs[0])
    n = len(ql)

    def one_step(cur):
        for li, (_, w) in enumerate(ql):
            lib.gemma4_ffn_block_q(dims, T, bufs[(cur + li) % 2], w, bufs[(cur + li + 1) % 2],
                                   None, None, None, ws)
        return (cur + n) % 2
    cur = one_step(0)  # warm-up step
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(steps):
        cur = one_step(cur)
    b.record()
    torch.cuda.synchronize()
    WINDOWS[f"stack_{name}_decode_{T}"] = (t0, time.perf_counter())
    ms = a.elapsed_time(b) / steps
    finite = bool(torch.isfinite(bufs[cur].float()).all().item())
    del ql
    torch.cuda.empty_cache()
    return {"layers": n, "tokens": T, "steps": steps, "weights": desc, "ms_per_step": ms,
            "tokens_per_s": T / (ms * 1e-3), "output_finite": finite}


def tiny_measure(torch, lib, steps, warmup):
    """The tiny fp32 configuration (16 tokens, hidden 64, 8 experts, top-2,
    intermediate 32) through moe_forward."""
    from sparse_moe_transformer_router_amd import synth
    c = synth.tiny_case(seed=0)
    f = lambda a: torch.from_numpy(a).cuda()  # noqa: E731
    d = lib.dims(c.H, c.E, c.K, c.I, 0, c.eps, lib.MOE_F32, lib.MOE_F32)
    ws = lib.workspace(d, c.T)
    x, rw, rs, pes = f(c.x.f32), f(c.router_w), f(c.router_scale), f(c.per_expert_scale)
    gu, dn = f(c.gate_up.f32), f(c.down.f32)
    out = torch.empty(c.T, c.H, device="cuda")
    idx = torch.empty(c.T, c.K, dtype=torch.int32, device="cuda")
    w = torch.empty(c.T, c.K, device="cuda")
    call = lambda: lib.moe_forward(d, c.T, x, rw, rs, pes, gu, dn, out, idx, w, ws)  # noqa: E731
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    return {"tokens": c.T, "ms_per_step": ms, "tokens_per_s": c.T / (ms * 1e-3),
            "dtype": "f32", "timing": "host clock around the launches (launch-bound)"}


def clock_warmup(torch, wl, T, seconds, seed):
    """Untimed decode steps for `seconds`: the GPU clock starts from its idle
    level and takes a while to rise under load, which the few warmup steps of
    each leg do not cover.  Returns the number of steps run."""
    if seconds <= 0:
        return 0
    runner = Runner(wl, T)
    xs = wl.batches(T, 4, seed + 99)
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(64):
            runner.step(xs[n % len(xs)], wl.copies[n % len(wl.copies)])
            n += 1
        torch.cuda.synchronize()
    return n


def achievable(torch):
    """Measured ceilings of this GPU (libmoe_probe): a 4 GiB streaming read and
    a register-only bf16 MFMA loop (32x32x16, 8 independent accumulators per
    wave, 1024 blocks of 4 waves)."""
    from sparse_moe_transformer_router_amd import probe

    buf = torch.ones(1 << 30, dtype=torch.int32, device="cuda")
    bx = torch.empty(probe.read_blocks(), dtype=torch.int32, device="cuda")
    for _ in range(3):
        probe.stream_read(buf, bx)
    n = 10
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(n):
        probe.stream_read(buf, bx)
    b.record()
    torch.cuda.synchronize()
    WINDOWS["probe_hbm_read"] = (t0, time.perf_counter())
    read_gbs = n * buf.numel() * 4 / (a.elapsed_time(b) * 1e-3) / 1e9
    del buf
    blocks, iters = 1024, 2000
    out = torch.empty(blocks * 4, dtype=torch.float32, device="cuda")
    for _ in range(2):
        probe.mfma(blocks, iters, out)
    t0 = time.perf_counter()
    a.record()
    for _ in range(5):
        probe.mfma(blocks, iters, out)
    b.record()
    torch.cuda.synchronize()
    WINDOWS["probe_mfma"] = (t0, time.perf_counter())
    mfma_tflops = 5 * probe.mfma_flops(blocks, iters) / (a.elapsed_time(b) * 1e-3) / 1e12
    assert bool((out == 16.0 * iters).all()), "MFMA probe result wrong"
    return {"hbm_read_gbs": read_gbs, "mfma_bf16_tflops": mfma_tflops,
            "probe": "libmoe_probe: 4 GiB streaming read (a contiguous chunk per block, "
                     "32-B lane spans); register-only "
                     "v_mfma_f32_32x32x16_bf16 loop"}


class ClockSampler:
    """GPU clock and socket power read from sysfs every few milliseconds in a
    background thread (no child process): the gfx clock level the driver
    marks current in pp_dpm_sclk, and hwmon power1_input.  Each leg reports
    the samples that fall inside its timed region."""

    def __init__(self, period_s=0.005):
        import glob
        import threading
        cards = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.sclk = cards[0] if cards else None
        pw = sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input"))
        self.power = pw[0] if pw else None
        self.samples = []  # (t, MHz, W)
        self.error = None if self.sclk else "no pp_dpm_sclk in sysfs"
        self._stop = threading.Event()
        self._period = period_s
        self._thread = threading.Thread(target=self._run, daemon=True)
        if self.sclk:
            self._thread.start()

    def _read(self):
        mhz = None
        with open(self.sclk) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    mhz = float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
        watts = None
        if self.power:
            with open(self.power) as f:
                watts = int(f.read().strip()) / 1e6
        return mhz, watts

    def _run(self):
        while not self._stop.is_set():
            try:
                mhz, watts = self._read()
                self.samples.append((time.perf_counter(), mhz, watts))
            except (OSError, ValueError, IndexError) as e:
                self.error = f"{type(e).__name__}: {e}"[:200]
                return
            self._stop.wait(self._period)

    def stop(self):
        self._stop.set()
        if self._thread.is_alive():
            self._thread.join(timeout=5)

    def summary(self, windows):
        """Per leg: mean / min / max gfx clock and power over its timed window."""
        if not self.samples:
            return {"error": self.error or "no samples"}
        out = {"source": f"{self.sclk} (current level), {self.power}",
               "period_ms": self._period * 1e3}
        for leg, (t0, t1) in windows.items():
            sel = [(m, w) for t, m, w in self.samples if t0 <= t <= t1 and m is not None]
            if not sel:
                continue
            ms = [m for m, _ in sel]
            ws = [w for _, w in sel if w is not None]
            out[leg] = {"samples": len(sel),
                        "gfx_clk_mhz": {"mean": sum(ms) / len(ms), "min": min(ms), "max": max(ms)}}
            if ws:
                out[leg]["socket_power_w"] = {"mean": sum(ws) / len(ws), "min": min(ws),
                                              "max": max(ws)}
        return out


WINDOWS = {}  # leg -> (start, end) of its timed region, host clock


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(torch, wl, xs, T, seconds, runner):
    """The oracle as it stands, on the host cores: router + sparse experts for
    the first decode batch, repeated for about `seconds`.  The same batch (and
    weight copy 0) through one GPU step is compared with the oracle's result:
    routing bit for bit, the output as max |err| / RMS."""
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
        ref = oracle.experts(x, gu32, dn32, idx, w)
        n += T
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    del gu32, dn32
    runner.step(xs[0], wl.copies[0])
    torch.cuda.synchronize()
    got = runner.out.float().cpu().numpy().astype(np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    parity = {"inputs": f"synth seed {wl.seed}: weight copy 0, first {T}-token batch",
              "routing_exact": bool(np.array_equal(runner.idx.cpu().numpy(), idx)),
              "max_err_over_rms": float(np.max(np.abs(got - ref))) / rms, "bar": 2e-2}
    return {"value": n / el, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"router + sparse experts (fp64 loop) on the first {T}-token decode batch of "
                      f"weight copy 0, repeated {n // T}x over {el:.1f} s",
            "parity_of_timed_inputs": parity}


def prefill_routing_check(torch, wl, T, seed):
    """Routing of synth's skewed prefill batch (the timed leg's batch 0 with
    copy 0) on the GPU against the oracle router, bit for bit."""
    import numpy as np
    import oracle

    runner = Runner(wl, T)
    xs, copies = skewed_inputs(torch, wl, T, seed)
    runner.step(xs[0], copies[0])
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy()  # noqa: E731
    rw, rs, pes = (f(t) for t in copies[0][:3])
    idx, _ = oracle.router(f(xs[0]), rw, rs, pes, K)
    counts = np.bincount(idx.ravel(), minlength=E)
    return {"inputs": f"synth seed {seed}, skewed, {T} tokens",
            "routing_exact": bool(np.array_equal(runner.idx.cpu().numpy(), idx)),
            "counts_exact": bool(np.array_equal(runner.counts.cpu().numpy(), counts))}


def _oracle_experts_rate(x, args, gu32, dn32, seconds):
    import oracle

    n, t0 = 0, time.perf_counter()
    while True:
        idx, w = oracle.router(x, *args, K)
        oracle.experts(x, gu32, dn32, idx, w)
        n += x.shape[0]
        el = time.perf_counter() - t0
        if el >= seconds:
            return n / el, n // x.shape[0], el


def cpu_oracle_configs(torch, wl, xs, T, layers, prefill_T, seed, seconds, stack_steps,
                       stack_prefill):
    """Oracle rates on the other configurations (bounded samples): the decode
    batch on one thread, 64 tokens of the skewed prefill batch, the tiny fp32
    experts-only case, the whole block on 16 tokens, and the 30-layer stack
    extrapolated from layers 0, 14 and 29 timed on 16 tokens each."""
    layer = layers[0] if layers else None
    import oracle
    from sparse_moe_transformer_router_amd import synth

    res = {"cores": oracle.num_threads(), "kind": "oracle", "cpu_model": cpu_model()}
    f = lambda t: t.float().cpu().numpy()  # noqa: E731
    rw, rs, pes, gu, dn = wl.copies[0]
    gu32, dn32 = f(gu), f(dn)
    cores = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        v, calls, el = _oracle_experts_rate(f(xs[0]), (f(rw), f(rs), f(pes)), gu32, dn32,
                                            seconds / 4)
    finally:
        oracle.set_num_threads(cores)
    res["decode_single_thread"] = {"tokens_per_s": v, "threads": 1,
                                   "sample": f"router + sparse experts on the {T}-token decode "
                                             f"batch, {calls} calls over {el:.1f} s"}
    if prefill_T:
        pxs, pcopies = skewed_inputs(torch, wl, prefill_T, seed)
        prw, prs, ppes, _, _ = pcopies[0]
        v, calls, el = _oracle_experts_rate(f(pxs[0][:64]), (f(prw), f(prs), f(ppes)), gu32,
                                            dn32, seconds / 4)
        res["prefill_sample"] = {"tokens_per_s": v,
                                 "sample": f"router + sparse experts on the first 64 tokens of "
                                           f"the skewed {prefill_T}-token batch, {calls} calls "
                                           f"over {el:.1f} s"}
    del gu32, dn32
    c = synth.tiny_case(seed=0)
    n, t0 = 0, time.perf_counter()
    while True:
        idx, w = oracle.router(c.x.f32, c.router_w, c.router_scale, c.per_expert_scale, c.K)
        oracle.experts(c.x.f32, c.gate_up.f32, c.down.f32, idx, w)
        n += c.T
        el = time.perf_counter() - t0
        if el >= seconds / 4:
            break
    res["tiny_f32"] = {"tokens_per_s": n / el, "sample": f"{n // c.T} calls of the 16-token case"}
    if layer is not None:
        f = lambda t: t.float().cpu().numpy()  # noqa: E731
        g = torch.Generator(device="cuda")
        g.manual_seed(7)
        x = f(torch.randn(16, H, generator=g, device="cuda").to(torch.bfloat16))
        args = [f(t) for t in (*layer.gains, *layer.dense, layer.rw, layer.rs, layer.pes, layer.gu,
                               layer.dn)]
        n, t0 = 0, time.perf_counter()
        while True:
            oracle.block(x, *args, 0.06, K)
            n += x.shape[0]
            el = time.perf_counter() - t0
            if el >= seconds / 4:
                break
        res["block"] = {"tokens_per_s": n / el,
                        "sample": f"whole block on 16 tokens, {n // 16} calls over {el:.1f} s"}
        del args
    if layers is not None and len(layers) >= LAYERS:
        # the stack: layers 0, 14 and 29 on 16 tokens each (the oracle's cost
        # is linear in the tokens and equal for every layer of these shapes);
        # the stack's rates are extrapolated from their mean per-token time
        per = []
        for li in (0, 14, LAYERS - 1):
            ly = layers[li]
            args = [f(t) for t in (*ly.gains, *ly.dense, ly.rw, ly.rs, ly.pes, ly.gu, ly.dn)]
            t0 = time.perf_counter()
            oracle.block(x, *args, 0.06, K)
            per.append((time.perf_counter() - t0) / x.shape[0])
            del args
        layer_s = sum(per) / len(per)
        res["stack_extrapolated"] = {
            "sample": "layers 0, 14 and 29 of the stack, one call on 16 tokens each; the "
                      f"stack's figures are extrapolated to {LAYERS} layers (labelled "
                      "extrapolation, not measured end to end)",
            "seconds_per_token_per_layer": per,
            "decode_tokens_per_s": 1.0 / (LAYERS * layer_s),
            "decode_seconds_for_the_gpu_run": stack_steps * T * LAYERS * layer_s,
            "prefill_tokens_per_s": 1.0 / (LAYERS * layer_s),
            "prefill_seconds_for_the_gpu_run": stack_prefill * LAYERS * layer_s}
    return res


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
    clocks_sampler = ClockSampler()
    wl = Workload(torch, lib, args.copies, args.seed)
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def done(leg):
        print(f"bench: {leg} done", file=sys.stderr, flush=True)

    warm_steps = clock_warmup(torch, wl, args.batch, args.clock_warmup, args.seed)
    done(f"clock warm-up ({warm_steps} untimed decode steps)")
    ach = achievable(torch)
    done("achievable read / MFMA rates")

    head, runner, xs = decode_measure(torch, wl, args.batch, args.steps, args.warmup,
                                      args.xbatches, args.seed)
    done(f"decode {args.batch}")
    sweep = {}
    for b in [int(v) for v in args.sweep.split(",") if v.strip()]:
        if b != args.batch:
            r, _, _ = decode_measure(torch, wl, b, args.steps, args.warmup, args.xbatches,
                                     args.seed)
            sweep[str(b)] = r
            done(f"decode {b}")
    prefill = None
    if args.prefill > 0:
        prefill = prefill_measure(torch, wl, args.prefill, max(5, args.steps // 5),
                                  max(2, args.warmup // 5), args.seed)
        done(f"prefill {args.prefill}")

    dense_mask = {}
    if args.dense_mask:
        dense_mask[str(args.batch)] = dense_mask_measure(
            torch, wl, args.batch, max(5, args.steps // 5), max(2, args.warmup // 5),
            args.xbatches, args.seed, head["ms_per_step"])
        done(f"all-experts ablation {args.batch}")
        if prefill is not None:
            dense_mask[str(args.prefill)] = dense_mask_measure(
                torch, wl, args.prefill, 5, 2, 2, args.seed, prefill["ms_per_step"])
            done(f"all-experts ablation {args.prefill}")

    quant = {}
    for name in (QUANT_FORMATS if args.quant else ()):
        quant[name] = quant_decode_measure(torch, lib, wl, name, args.batch, args.steps,
                                           args.warmup, args.xbatches, args.seed)
        done(f"{name} experts decode")
    native = {}
    for name in (("fp8", "mxfp4") if args.quant else ()):
        native[name] = {}
        for b in sorted({1, 8, args.batch, 256}):
            native[name][str(b)] = quant_decode_measure(torch, lib, wl, name, b, args.steps,
                                                        args.warmup, args.xbatches, args.seed,
                                                        native=True)
        if args.prefill > 0:
            native[name][f"{args.prefill}_skewed"] = quant_decode_measure(
                torch, lib, wl, name, args.prefill, max(5, args.steps // 5),
                max(2, args.warmup // 5), 2, args.seed, native=True, skew=True)
        done(f"{name} experts on the 8/4-bit matrix instructions")
    quant_prefill = {}
    for name in (QUANT_FORMATS if args.quant and args.prefill > 0 else ()):
        quant_prefill[name] = quant_decode_measure(
            torch, lib, wl, name, args.prefill, max(5, args.steps // 5), max(2, args.warmup // 5),
            2, args.seed, skew=True)
        done(f"{name} experts at {args.prefill} skewed tokens (tiled, widened codes)")

    tiny = tiny_measure(torch, lib, args.steps, args.warmup)
    done("tiny fp32")

    block, layers = None, []
    if args.block > 0 or args.stack > 0:
        layers = [BlockLayer(torch, lib, args.seed, l) for l in range(max(2, args.stack))]
        torch.cuda.synchronize()
    if args.block > 0:
        block = block_measure(torch, lib, args.block, max(5, args.steps // 5),
                              max(2, args.warmup // 5), args.seed, layers[:2])
        done(f"layer {args.block}")
    block_q = None
    if args.block > 0:
        block_q = block_quant_measure(torch, lib, layers[:2], args.batch,
                                      max(10, args.steps // 2), max(2, args.warmup // 2),
                                      args.seed)
        done(f"layer {args.batch}, quantized weights")
    stack = None
    if args.stack > 0:
        stack = stack_measure(torch, lib, layers[:args.stack], args.batch, args.stack_steps,
                              args.stack_prefill, args.seed)
        stack["decode_int8"] = stack_quant_decode(torch, lib, layers[:args.stack], args.batch,
                                                  args.stack_steps, args.seed)
        done(f"stack of {args.stack} layers")

    clocks_sampler.stop()
    clocks = clocks_sampler.summary(WINDOWS)
    # A probe figure is a ceiling only if no kernel of this run beat it; the
    # fractions against it are reported only then.
    best_read = max([r["gate_up_gbs"] for r in [head, *sweep.values()]] +
                    [r["experts_gbs"] for r in quant.values()] +
                    [v["experts_gbs"] for m in native.values() for v in m.values()])
    ach["read_probe_is_ceiling"] = ach["hbm_read_gbs"] >= best_read
    ach["best_kernel_read_gbs"] = best_read
    read_ceiling = ach["hbm_read_gbs"] if ach["read_probe_is_ceiling"] else None
    for r in [head, *sweep.values()]:
        r["gate_up_frac_of_achievable_read"] = (r["gate_up_gbs"] / read_ceiling
                                                if read_ceiling else None)
    if prefill is not None:
        prefill["grouped_gemm_frac_of_achievable_mfma"] = (prefill["grouped_gemm_tflops"] /
                                                           ach["mfma_bf16_tflops"])
    for r in [*quant.values(), *[v for m in native.values() for v in m.values()]]:
        r["experts_frac_of_achievable_read"] = (r["experts_gbs"] / read_ceiling
                                                if read_ceiling else None)

    cpu = None
    cpu_configs = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(torch, wl, xs, args.batch, args.cpu_seconds, runner)
        if prefill is not None:
            prefill["routing_vs_oracle"] = prefill_routing_check(torch, wl, args.prefill,
                                                                 args.seed)
        cpu_configs = cpu_oracle_configs(torch, wl, xs, args.batch, layers or None,
                                         args.prefill, args.seed, args.cpu_seconds,
                                         args.stack_steps, args.stack_prefill)
        done("cpu baselines")

    achieved = head["gate_up_gbs"]
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_warmup": {"seconds": args.clock_warmup, "untimed_decode_steps": warm_steps},
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
                     "frac_of_achievable": achieved / read_ceiling if read_ceiling else None,
                     "algorithmic_bytes_per_launch": head["gate_up_bytes"],
                     "avg_launch_ms": head["kernel_ms"]["gate_up"]},
        "cpu_baseline": cpu,
        "achievable": ach,
        "gpu_clock_power": clocks,
        "decode": {str(args.batch): head, **sweep},
        "prefill": prefill,
        "dense_masked_ablation": dense_mask or None,
        "quantized_experts_decode": quant,
        "quantized_experts_native_decode": native or None,
        "quantized_experts_prefill": quant_prefill or None,
        "tiny_f32": tiny,
        "block": block,
        "block_decode_quantized": block_q,
        "stack": stack,
        "cpu_oracle_other_configs": cpu_configs,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
