"""GPU parity of the int8-expert path (per-channel symmetric int8 weights, the
int8-expert variant of "Porting a 128-expert MoE (Gemma-4 26B-A4B) to AWS
Inferentia2", section "Can it run on a smaller box?"): the quantizer's codes
and scales bit-exact against the oracle's, and the int8 expert FFN at decode
batches within 2e-2 x RMS of the oracle's sparse loop on the oracle's own
dequantized weights."""
import numpy as np
import pytest
import torch

import oracle
from sparse_moe_transformer_router_amd import synth
from tests.gpu_util import (BF16_TOL, bf16_path_bound, dev_f32, dev_tensor, host, note,
                            rel_max_err)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sparse_moe_transformer_router_amd import lib
else:
    lib = None


def _gpu_quantize(wt: torch.Tensor):
    q = torch.empty(wt.shape, dtype=torch.int8, device="cuda")
    s = torch.empty(wt.shape[:-1], dtype=torch.float32, device="cuda")
    lib.moe_quantize_int8(wt, q, s)
    torch.cuda.synchronize()
    return host(q), host(s)


def _bf16_tensor(a: np.ndarray) -> synth.Tensor:
    bits = synth.f32_to_bf16_bits(a.astype(np.float32))
    return synth.Tensor(synth.bf16_bits_to_f32(bits), bits)


def test_quantize_special_rows_bit_exact():
    rows = np.zeros((6, 64), np.float32)
    rows[1, :9] = np.array([127, 63.5, -62.5, 0.5, -0.5, 1.5, 2.5, 0, -127]) / 16  # exact ties
    rng = np.random.default_rng(3)
    rows[2] = rng.standard_normal(64)
    rows[3] = -rows[2]
    rows[4] = rows[2] * 2.0 ** -20
    rows[5, 7] = -3.0  # a single nonzero
    t = _bf16_tensor(rows)
    note("quantize special rows")
    gq, gs = _gpu_quantize(dev_tensor(t, True))
    oq, os_ = oracle.quantize_int8(t.f32)
    assert np.array_equal(gq, oq)
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32))


@pytest.fixture(scope="module")
def case26b_q():
    c = synth.moe_case(256, seed=0)
    guq, gus = oracle.quantize_int8(c.gate_up.f32)
    dnq, dns = oracle.quantize_int8(c.down.f32)
    return c, (guq, gus, dnq, dns)


def test_quantize_26b_experts_bit_exact(case26b_q):
    c, (guq, gus, dnq, dns) = case26b_q
    note("quantize 26B gate_up / down")
    gq, gs = _gpu_quantize(dev_tensor(c.gate_up, True))
    assert np.array_equal(gq, guq)
    assert np.array_equal(gs.view(np.uint32), gus.view(np.uint32))
    gq, gs = _gpu_quantize(dev_tensor(c.down, True))
    assert np.array_equal(gq, dnq)
    assert np.array_equal(gs.view(np.uint32), dns.view(np.uint32))


def _int8_path(c, T, idx, w, q):
    d = lib.dims(c.H, c.E, c.K, c.I, 0, c.eps, lib.MOE_BF16, lib.MOE_F32)
    ws = lib.workspace(d, T)
    counts = torch.empty(c.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(c.E + 1, dtype=torch.int32, device="cuda")
    ss = torch.empty(T * c.K, dtype=torch.int32, device="cuda")
    lib.moe_dispatch(d, T, torch.from_numpy(idx).cuda(), counts, offsets, ss, ws)
    y = torch.empty(T, c.K, c.H, dtype=torch.float32, device="cuda")
    out = torch.empty(T, c.H, dtype=torch.bfloat16, device="cuda")
    guq, gus, dnq, dns = [torch.from_numpy(a).cuda() for a in q]
    x = dev_tensor(synth.Tensor(c.x.f32[:T], c.x.bf16[:T]), True)
    lib.moe_expert_ffn_int8(d, T, x, guq, gus, dnq, dns, dev_f32(w), offsets, ss, y, ws)
    lib.moe_combine(d, T, y, None, out)
    torch.cuda.synchronize()
    return host(y), host(out)


@pytest.fixture(scope="module")
def deq26b(case26b_q):
    _, (guq, gus, dnq, dns) = case26b_q
    return oracle.dequantize_int8(guq, gus), oracle.dequantize_int8(dnq, dns)


# 128 and 256 straddle the switch of gate_up to 32-row tiles; 256 tokens is
# the largest batch the quantized experts take
@pytest.mark.parametrize("T", [1, 8, 64, 128, 256])
def test_experts_int8_26b_decode(case26b_q, deq26b, T):
    """As the bf16 experts: the output within the per-element bound of its bf16
    roundings (on the oracle's dequantized weights) at every size and within
    2e-2 x RMS up to 128 tokens, the first slot within 2e-2 x RMS."""
    c, q = case26b_q
    x = c.x.f32[:T]
    idx, w = oracle.router(x, c.router_w, c.router_scale, c.per_expert_scale, c.K, c.eps)
    note(f"experts int8 26B decode T={T}")
    y, out = _int8_path(c, T, idx, w, q)
    ref = oracle.experts_int8(x, *q, idx, w)
    bound, exact = bf16_path_bound(x, *deq26b, idx, w)
    np.testing.assert_allclose(exact, ref, rtol=1e-9, atol=1e-12)
    assert np.all(np.abs(out - ref) <= bound), float(np.max(np.abs(out - ref) / bound))
    if T <= 128:
        assert rel_max_err(out, ref) <= BF16_TOL
    refk = oracle.experts_int8(x, *q, idx[:, :1], w[:, :1])
    assert rel_max_err(y[:, 0], refk) <= BF16_TOL


def test_experts_int8_small_ragged():
    """A small layer with ragged row groups (some experts empty) and
    unit-variance weights, held to the per-element bf16 rounding bound of the
    path (computed on the oracle's dequantized weights)."""
    c = synth.tiny_case(seed=9, T=37, H=128, E=16, K=3, I=64, bf16=True)
    q = (*oracle.quantize_int8(c.gate_up.f32), *oracle.quantize_int8(c.down.f32))
    idx, w = oracle.router(c.x.f32, c.router_w, c.router_scale, c.per_expert_scale, c.K, c.eps)
    note("experts int8 small ragged")
    y, out = _int8_path(c, c.T, idx, w, q)
    ref = oracle.experts_int8(c.x.f32, *q, idx, w)
    gu, dn = oracle.dequantize_int8(q[0], q[1]), oracle.dequantize_int8(q[2], q[3])
    bound, exact = bf16_path_bound(c.x.f32, gu, dn, idx, w)
    np.testing.assert_allclose(exact, ref, rtol=1e-9, atol=1e-12)
    assert np.all(np.abs(out - ref) <= bound), float(np.max(np.abs(out - ref) / bound))
