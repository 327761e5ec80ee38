"""moe_expert_gate_up_timed: the gate_up kernel launched with the caller's
events on its own dispatch.  Its output must equal moe_expert_gate_up's bit
for bit on each of the three gate_up kernels (decode streaming, prefill
grouped GEMM, fp32), and the events must bracket the kernel: a positive
duration no longer than that of ordinary events recorded around the call."""
import numpy as np
import pytest
import torch

import oracle
from sparse_moe_transformer_router_amd import synth
from tests.gpu_util import dev_tensor, note

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sparse_moe_transformer_router_amd import lib
else:
    lib = None


@pytest.mark.parametrize("name,T,kw,bf16", [
    ("decode streaming, 26B shapes", 64, {}, True),
    ("prefill grouped GEMM", 300, dict(H=256, E=16, K=4, I=64), True),
    ("fp32 path", 40, dict(H=128, E=8, K=2, I=32), False),
])
def test_timed_gate_up_matches_and_brackets_the_kernel(name, T, kw, bf16):
    c = synth.moe_case(T, seed=21, bf16=bf16, **kw) if kw else synth.moe_case(T, seed=21)
    note(f"timed gate_up: {name}")
    idx, _ = oracle.router(c.x.f32, c.router_w, c.router_scale, c.per_expert_scale, c.K, c.eps)
    _, offsets, sorted_slots = oracle.dispatch(idx, c.E)
    act = lib.MOE_BF16 if c.bf16 else lib.MOE_F32
    d = lib.dims(c.H, c.E, c.K, c.I, 0, c.eps, act, lib.MOE_F32)
    x, gu = dev_tensor(c.x, c.bf16), dev_tensor(c.gate_up, c.bf16)
    off = torch.from_numpy(np.ascontiguousarray(offsets, np.int32)).cuda()
    ss = torch.from_numpy(np.ascontiguousarray(sorted_slots, np.int32)).cuda()
    dt = torch.bfloat16 if c.bf16 else torch.float32
    h0 = torch.empty(T * c.K, c.I, dtype=dt, device="cuda")
    h1 = torch.full_like(h0, 7.0)
    lib.moe_expert_gate_up(d, T, x, gu, off, ss, h0)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record()  # torch creates its events at the first record
    torch.cuda.synchronize()
    ev[0].record()
    lib.moe_expert_gate_up_timed(d, T, x, gu, off, ss, h1, ev[1], ev[2])
    ev[3].record()
    torch.cuda.synchronize()
    assert torch.equal(h0.view(torch.int16 if c.bf16 else torch.int32),
                       h1.view(torch.int16 if c.bf16 else torch.int32))
    kernel_ms, outer_ms = ev[1].elapsed_time(ev[2]), ev[0].elapsed_time(ev[3])
    assert 0.0 < kernel_ms <= outer_ms, (kernel_ms, outer_ms)
