"""GPU parity of the experts with weights stored below bf16 past the decode
sizes: int8 per-channel (page "Porting a 128-expert MoE (Gemma-4 26B-A4B) to
AWS Inferentia2", section "Can it run on a smaller box? Yes, no, and "deeper
than it looks"") and E4M3 / MXFP4 (its section "The fp4 rabbit hole (two of
them, both dead ends)").

Past 256 tokens moe_expert_ffn_q runs the tiled grouped GEMMs: the codes sit
in the LDS ring as stored and widen exactly to bf16 after the LDS reads, so
the result is the bf16 path on the dequantized weights.  The oracle runs its
quantized expert loop on the same codes; every row of the output is held to
the per-element bound of the bf16 path's roundings (computed on the oracle's
dequantized weights), and so is the first slot on its own (no output
rounding)."""
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

# name -> (ABI code, quantizer, dequantizer, quantized expert loop)
FORMATS = {
    "int8": (1, oracle.quantize_int8, oracle.dequantize_int8, oracle.experts_int8),
    "fp8": (2, oracle.quantize_fp8, oracle.dequantize_fp8, oracle.experts_fp8),
    "mxfp4": (3, oracle.quantize_mxfp4, oracle.dequantize_mxfp4, oracle.experts_mxfp4),
}


def _q_path(c, fmt, T, x, idx, w, q):
    d = lib.dims(c.H, c.E, c.K, c.I, 0, c.eps, lib.MOE_BF16, lib.MOE_F32)
    ws = lib.workspace(d, T)
    counts = torch.empty(c.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(c.E + 1, dtype=torch.int32, device="cuda")
    ss = torch.empty(T * c.K, dtype=torch.int32, device="cuda")
    lib.moe_dispatch(d, T, torch.from_numpy(idx).cuda(), counts, offsets, ss, ws)
    y = torch.empty(T, c.K, c.H, dtype=torch.float32, device="cuda")
    out = torch.empty(T, c.H, dtype=torch.bfloat16, device="cuda")
    dq = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in q]
    lib.moe_expert_ffn_q(d, fmt, T, dev_tensor(x, True), *dq, dev_f32(w), offsets, ss, y, ws)
    lib.moe_combine(d, T, y, None, out)
    torch.cuda.synchronize()
    return host(y), host(out)


def _check(name, c, x, idx, w, q, y, out):
    _, _, deq, loop = FORMATS[name]
    gu, dn = deq(q[0], q[1]), deq(q[2], q[3])
    ref = loop(x, *q, idx, w)
    bound, exact = bf16_path_bound(x, gu, dn, idx, w)
    np.testing.assert_allclose(exact, ref, rtol=1e-9, atol=1e-12)
    err = np.abs(out - ref)
    note(f"  max err / bound = {float(np.max(err / bound)):.3f}")
    assert np.all(err <= bound), float(np.max(err / bound))
    ref0 = loop(x, *q, idx[:, :1], w[:, :1])
    b0, e0 = bf16_path_bound(x, gu, dn, idx[:, :1], w[:, :1], out_rounded=False)
    np.testing.assert_allclose(e0, ref0, rtol=1e-9, atol=1e-12)
    assert np.all(np.abs(y[:, 0] - ref0) <= b0), float(np.max(np.abs(y[:, 0] - ref0) / b0))


@pytest.mark.parametrize("name", list(FORMATS))
def test_experts_q_tiled_small_ragged(name):
    """300 tokens, 8 experts of ragged size, a gate_up width (96) that fills
    part of one 128-column tile and a down contraction of three k-tiles."""
    fmt, quant, _, _ = FORMATS[name]
    c = synth.tiny_case(seed=12, T=300, H=256, E=8, K=2, I=96, bf16=True)
    q = (*quant(c.gate_up.f32), *quant(c.down.f32))
    idx, w = oracle.router(c.x.f32, c.router_w, c.router_scale, c.per_expert_scale, c.K, c.eps)
    note(f"experts {name} tiled, small ragged")
    y, out = _q_path(c, fmt, c.T, c.x, idx, w, q)
    _check(name, c, c.x.f32, idx, w, q, y, out)


@pytest.fixture(scope="module")
def skew26b():
    c = synth.moe_case(4096, seed=0, skew=True)
    idx, w = oracle.router(c.x.f32, c.router_w, c.router_scale, c.per_expert_scale, c.K, c.eps)
    return c, idx, w


@pytest.mark.parametrize("name", list(FORMATS))
def test_experts_q_26b_prefill_skewed(skew26b, name):
    """26B experts at 4096 skewed tokens (hottest expert ~3100 slots, a dozen
    experts empty), every row."""
    c, idx, w = skew26b
    fmt, quant, _, _ = FORMATS[name]
    note(f"experts {name} 26B prefill 4096 skewed: oracle quantization")
    q = (*quant(c.gate_up.f32), *quant(c.down.f32))
    note(f"experts {name} 26B prefill 4096 skewed")
    y, out = _q_path(c, fmt, c.T, c.x, idx, w, q)
    _check(name, c, c.x.f32, idx, w, q, y, out)


@pytest.mark.parametrize("name", list(FORMATS))
@pytest.mark.parametrize("H,I", [(8192, 256), (256, 8192)])
def test_experts_q_tiled_longest_contraction(name, H, I):
    """The longest contraction the ABI takes (8192) on either GEMM, past 256
    tokens: 256 k-tiles, and for MXFP4 a full 256-byte block-scale row per
    weight row staged in LDS."""
    fmt, quant, _, _ = FORMATS[name]
    c = synth.tiny_case(seed=14, T=264, H=H, E=4, K=2, I=I, bf16=True)
    q = (*quant(c.gate_up.f32), *quant(c.down.f32))
    idx, w = oracle.router(c.x.f32, c.router_w, c.router_scale, c.per_expert_scale, c.K, c.eps)
    note(f"experts {name} tiled, H={H} I={I}")
    y, out = _q_path(c, fmt, c.T, c.x, idx, w, q)
    _check(name, c, c.x.f32, idx, w, q, y, out)
