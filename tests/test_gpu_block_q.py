"""GPU parity of the layer with its expert and dense-MLP weights below bf16
(gemma4_ffn_block_q; the int8 option of the page "Porting a 128-expert MoE
(Gemma-4 26B-A4B) to AWS Inferentia2", section "Can it run on a smaller box?
Yes, no, and "deeper than it looks"", and the E4M3 / MXFP4 formats of its
section "The fp4 rabbit hole (two of them, both dead ends)").

Every matrix of a 26B-shaped layer (the experts' gate_up and down, the dense
gate, up and down) is quantized by the oracle (whose codes and scales the GPU
quantizer matches bit for bit, tests/test_gpu_int8.py and test_gpu_lowp.py);
the GPU runs the layer on those codes, and the oracle runs its layer on the
dequantized weights.  Routing is bit-exact (the router stays fp32); the
layer output and its pre-residual part are within 2e-2 x RMS, every row, at
one token, at a decode batch (64 tokens), at the largest batch of the
weight-streaming kernels (256 tokens) and past it (640 tokens: the tiled
grouped GEMMs for the experts and the dense branch)."""
import numpy as np
import pytest
import torch

import oracle
from sparse_moe_transformer_router_amd import synth
from tests.gpu_util import BF16_TOL, dev_f32, dev_tensor, host, note, rel_max_err

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sparse_moe_transformer_router_amd import lib
else:
    lib = None

# format name -> (ABI code, oracle quantizer, oracle dequantizer)
FORMATS = {
    "int8": (1, oracle.quantize_int8, oracle.dequantize_int8),
    "fp8": (2, oracle.quantize_fp8, oracle.dequantize_fp8),
    "mxfp4": (3, oracle.quantize_mxfp4, oracle.dequantize_mxfp4),
}
MATRICES = ("dense_gate", "dense_up", "dense_down", "gate_up", "down")


@pytest.fixture(scope="module")
def case():
    return synth.block_case(640, seed=8)


def _weights(b, name):
    return getattr(b.moe, name) if name in ("gate_up", "down") else getattr(b, name)


def _run(b, fmt, T, q):
    m = b.moe
    d = lib.dims(m.H, m.E, m.K, m.I, b.D, m.eps, lib.MOE_BF16, lib.MOE_F32)
    ws = lib.workspace(d, T)
    dq = {n: [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in q[n]] for n in MATRICES}
    keep = [dev_f32(b.g_pre), dev_f32(b.g_pre2), dev_f32(b.g_post1), dev_f32(b.g_post2),
            dev_f32(b.g_post), *dq["dense_gate"], *dq["dense_up"], *dq["dense_down"],
            dev_f32(m.router_w), dev_f32(m.router_scale), dev_f32(m.per_expert_scale),
            *dq["gate_up"], *dq["down"]]
    wts = lib.ffn_weights_q(fmt, *keep, b.layer_scalar)
    x = dev_tensor(synth.Tensor(m.x.f32[:T], m.x.bf16[:T]), True)
    out = torch.empty(T, m.H, dtype=torch.bfloat16, device="cuda")
    ffn = torch.empty(T, m.H, dtype=torch.float32, device="cuda")
    idx = torch.empty(T, m.K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, m.K, dtype=torch.float32, device="cuda")
    lib.gemma4_ffn_block_q(d, T, x, wts, out, ffn, idx, w, ws)
    torch.cuda.synchronize()
    return host(out), host(ffn), host(idx), host(w)


@pytest.mark.parametrize("name", list(FORMATS))
def test_quantized_layer_26b(case, name):
    b = case
    m = b.moe
    fmt, quant, deq = FORMATS[name]
    note(f"quantized layer {name}: oracle quantization")
    q = {n: quant(_weights(b, n).f32) for n in MATRICES}
    dq = {n: deq(*q[n]) for n in MATRICES}
    for T in (1, 64, 256, 640):
        note(f"quantized layer {name} T={T}")
        out, ffn, idx, w = _run(b, fmt, T, q)
        r = oracle.block(m.x.f32[:T], b.g_pre, b.g_pre2, b.g_post1, b.g_post2, b.g_post,
                         dq["dense_gate"], dq["dense_up"], dq["dense_down"], m.router_w,
                         m.router_scale, m.per_expert_scale, dq["gate_up"], dq["down"],
                         b.layer_scalar, m.K)
        assert np.array_equal(idx, r["idx"])
        np.testing.assert_allclose(w, r["w"], rtol=1e-6)
        e_ffn, e_out = rel_max_err(ffn, r["o"]), rel_max_err(out, r["out"])
        note(f"quantized layer {name} T={T}: ffn {e_ffn:.4f} out {e_out:.4f} x RMS")
        assert e_ffn <= BF16_TOL
        assert e_out <= BF16_TOL
