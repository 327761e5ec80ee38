"""bf16 per-slot outputs (moe_dims.slot_dtype = MOE_BF16).  The down kernels
compute each slot output in fp32 and round it once on the store, so every
bf16 slot must equal the fp32 path's slot rounded to nearest-even, bit for
bit; the combine must then return, for every token, the fp32 sum of its bf16
slots in slot order from +0, rounded once to bf16, bit for bit.  With the
fp32-slot path held to the oracle elsewhere, these two exact checks pin the
option down completely (its extra error against the oracle is exactly one
rounding of each slot, which the 2e-2 bar of the fp32-slot path does not
budget for: the option sits outside that bar, one 64-token 26B case reaches
0.026 x RMS).  Against the oracle the option is held to its own derived
per-element bound: the bf16 path's bound plus one bf16 rounding of each slot.
Covers the decode streaming down (both activation sources), the tiled down's
LDS-staged epilogue and the combine."""
import numpy as np
import pytest
import torch

import oracle
from sparse_moe_transformer_router_amd import synth
from tests.gpu_util import bf16_path_bound, dev_f32, dev_tensor, host, note

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sparse_moe_transformer_router_amd import lib
else:
    lib = None


def _run(c, idx, w, slot):
    d = lib.dims(c.H, c.E, c.K, c.I, 0, c.eps, lib.MOE_BF16, slot)
    ws = lib.workspace(d, c.T)
    T, K, E = c.T, c.K, c.E
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    ss = torch.empty(T * K, dtype=torch.int32, device="cuda")
    lib.moe_dispatch(d, T, torch.from_numpy(idx).cuda(), counts, offsets, ss, ws)
    ydt = torch.bfloat16 if slot == lib.MOE_BF16 else torch.float32
    y = torch.empty(T, K, c.H, dtype=ydt, device="cuda")
    out = torch.empty(T, c.H, dtype=torch.bfloat16, device="cuda")
    lib.moe_expert_ffn(d, T, dev_tensor(c.x, True), dev_tensor(c.gate_up, True),
                       dev_tensor(c.down, True), dev_f32(w), offsets, ss, y, ws)
    lib.moe_combine(d, T, y, None, out)
    torch.cuda.synchronize()
    return y, host(out)


@pytest.mark.parametrize("name,T,kw", [
    ("decode, global activations", 8, {}),
    ("decode, activations in LDS", 64, {}),
    ("tiled GEMM", 300, dict(H=512, E=16, K=4, I=128)),
])
def test_bf16_slots_are_the_rounded_fp32_slots(name, T, kw):
    c = synth.moe_case(T, seed=31, **kw)
    note(f"bf16 slots: {name} T={T}")
    idx, w = oracle.router(c.x.f32, c.router_w, c.router_scale, c.per_expert_scale, c.K, c.eps)
    y32, _ = _run(c, idx, w, lib.MOE_F32)
    y16, out = _run(c, idx, w, lib.MOE_BF16)
    assert torch.equal(y32.to(torch.bfloat16).view(torch.int16), y16.view(torch.int16))
    slots = host(y16).astype(np.float32)            # [T, K, H], exact
    acc = np.zeros((c.T, c.H), np.float32)
    for k in range(c.K):
        acc = acc + slots[:, k]                     # fp32, slot order, from +0
    want = torch.from_numpy(acc).to(torch.bfloat16).float().numpy()
    assert np.array_equal(out, want)
    # against the oracle, at the option's own bound
    ref = oracle.experts(c.x.f32, c.gate_up.f32, c.down.f32, idx, w)
    bound, exact = bf16_path_bound(c.x.f32, c.gate_up.f32, c.down.f32, idx, w, bf16_slots=True)
    np.testing.assert_allclose(exact, ref, rtol=1e-9, atol=1e-12)
    assert np.all(np.abs(out - ref) <= bound), float(np.max(np.abs(out - ref) / bound))
