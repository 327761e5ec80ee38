"""moe_forward_noalloc (the library's own device scratch array as workspace)
against moe_forward with a caller workspace: the same kernels, so the same
bits.  Two calls in a row on the shared array, the second with a smaller
input; the routing it returns as well.  Also the refusal of a size whose
workspace exceeds the array."""
import ctypes

import numpy as np
import pytest
import torch

from sparse_moe_transformer_router_amd import synth
from tests.gpu_util import dev_f32, dev_tensor, note

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sparse_moe_transformer_router_amd import lib
else:
    lib = None


def _both(c, T, ws_path_first):
    d = lib.dims(c.H, c.E, c.K, c.I, 0, c.eps, lib.MOE_BF16 if c.bf16 else lib.MOE_F32)
    x = dev_tensor(synth.Tensor(c.x.f32[:T], None if c.x.bf16 is None else c.x.bf16[:T]),
                   c.bf16)
    args = (dev_f32(c.router_w), dev_f32(c.router_scale), dev_f32(c.per_expert_scale),
            dev_tensor(c.gate_up, c.bf16), dev_tensor(c.down, c.bf16))
    odt = torch.bfloat16 if c.bf16 else torch.float32
    res = {}
    for which in (("ws", "noalloc") if ws_path_first else ("noalloc", "ws")):
        out = torch.empty(T, c.H, dtype=odt, device="cuda")
        idx = torch.empty(T, c.K, dtype=torch.int32, device="cuda")
        w = torch.empty(T, c.K, dtype=torch.float32, device="cuda")
        if which == "ws":
            ws = lib.workspace(d, T)
            lib.moe_forward(d, T, x, *args, out, idx, w, ws)
        else:
            lib.moe_forward_noalloc(d, T, x, *args, out, idx, w)
        torch.cuda.synchronize()
        res[which] = (out.view(torch.int16 if c.bf16 else torch.int32).cpu().numpy(),
                      idx.cpu().numpy(), w.view(torch.int32).cpu().numpy())
    return res


@pytest.mark.parametrize("name,make,sizes", [
    ("26B-A4B bf16", lambda: synth.moe_case(64, seed=0), (64, 9)),
    ("small fp32", lambda: synth.tiny_case(seed=5, T=300, H=256, E=16, K=4, I=64), (300, 37)),
    ("small bf16", lambda: synth.tiny_case(seed=6, T=520, H=128, E=8, K=2, I=64, bf16=True),
     (520, 130)),
])
def test_noalloc_forward_equals_workspace_forward(name, make, sizes):
    c = make()
    for i, T in enumerate(sizes):
        note(f"noalloc forward {name} T={T} (call {i + 1})")
        r = _both(c, T, ws_path_first=(i % 2 == 1))
        for a, b in zip(r["ws"], r["noalloc"]):
            assert np.array_equal(a, b)


def test_noalloc_rejects_sizes_beyond_its_array():
    d = lib.dims(2816, 128, 8, 704, 0)
    L = lib.raw()
    fake = ctypes.c_void_p(0x10000)
    rc = L.moe_forward_noalloc(ctypes.byref(d), 539, fake, fake, fake, fake, fake, fake, fake,
                               None, None, None)
    assert rc == lib.MOE_ERR_WORKSPACE and "scratch" in lib.last_error()
