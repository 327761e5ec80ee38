"""GPU parity at the limits the C ABI accepts (include/moe.h): the largest
hidden size and expert width, the largest expert count with the largest
top-K the router takes, the smallest layer, and the largest batch.  Each is
held to the same bars as the other parity tests: router logits bit for bit,
routing and dispatch exact, the fp32 path within 1e-4 x RMS, the bf16 path
within its per-element rounding bound (small layers) or 2e-2 x RMS (26B
shapes)."""
import numpy as np
import pytest
import torch

import oracle
from sparse_moe_transformer_router_amd import synth
from tests.gpu_util import (BF16_TOL, F32_TOL, bf16_path_bound, dev_f32, dev_tensor, host, note,
                            rel_max_err)
from tests.test_gpu_parity import _check_router, _dims, _expert_path

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sparse_moe_transformer_router_amd import lib
else:
    lib = None


@pytest.mark.parametrize("seed,T,H,E,K,I", [
    (11, 40, 8192, 8, 2, 64),     # largest hidden size, weight-streaming kernels
    (12, 70, 8192, 8, 2, 64),     # largest hidden size, tiled GEMMs
    (13, 50, 128, 256, 32, 32),   # most experts, largest top-K, streaming
    (14, 300, 128, 256, 32, 32),  # most experts, largest top-K, tiled
    (15, 9, 64, 1, 1, 32),        # smallest layer: one expert, top-1
    (16, 33, 64, 5, 5, 8192),     # widest experts (I = 8192), streaming, K = E
    (17, 100, 64, 5, 2, 8192),    # widest experts, tiled
])
def test_limits_small_layers(seed, T, H, E, K, I):
    for bf in (False, True):
        c = synth.tiny_case(seed=seed, T=T, H=H, E=E, K=K, I=I, bf16=bf)
        note(f"limits T={T} H={H} E={E} K={K} I={I} bf16={bf}")
        idx, w = _check_router(c)
        y, out = _expert_path(c, idx, w)
        ref = oracle.experts(c.x.f32, c.gate_up.f32, c.down.f32, idx, w)
        if not bf:
            assert rel_max_err(out, ref) <= F32_TOL
            continue
        bound, exact = bf16_path_bound(c.x.f32, c.gate_up.f32, c.down.f32, idx, w)
        np.testing.assert_allclose(exact, ref, rtol=1e-9, atol=1e-12)
        assert np.all(np.abs(out - ref) <= bound), float(np.max(np.abs(out - ref) / bound))


def test_largest_batch_26b():
    """65536 tokens (the largest T; 524288 token-slots) through the router,
    the dispatch and the tiled expert GEMMs at 26B shapes: logits bit for bit,
    routing and dispatch exact, sampled rows of the output within 2e-2 x RMS
    of the oracle, and whole row tiles slot by slot within the per-element
    rounding bound (the hottest expert's ragged last tile, every row of the
    rarest expert, the first tile)."""
    T = 65536
    c = synth.moe_case(T, seed=6)
    note(f"largest batch T={T}: router and dispatch")
    d = _dims(c)
    ws = lib.workspace(d, T)
    x = dev_tensor(c.x, True)
    rw, rs, pes = dev_f32(c.router_w), dev_f32(c.router_scale), dev_f32(c.per_expert_scale)
    idx = torch.empty(T, c.K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, c.K, dtype=torch.float32, device="cuda")
    counts = torch.empty(c.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(c.E + 1, dtype=torch.int32, device="cuda")
    ss = torch.empty(T * c.K, dtype=torch.int32, device="cuda")
    lib.moe_route(d, T, x, rw, rs, pes, None, idx, w, counts, offsets, ss, ws)
    torch.cuda.synchronize()
    oi, ow = oracle.router(c.x.f32, c.router_w, c.router_scale, c.per_expert_scale, c.K, c.eps)
    assert np.array_equal(host(idx), oi)
    np.testing.assert_allclose(host(w), ow, rtol=1e-6, atol=0)
    oc, oo, os_ = oracle.dispatch(oi, c.E)
    assert np.array_equal(host(counts), oc)
    assert np.array_equal(host(offsets), oo)
    assert np.array_equal(host(ss), os_)
    note(f"largest batch T={T}: experts")
    y = torch.empty(T, c.K, c.H, dtype=torch.float32, device="cuda")
    out = torch.empty(T, c.H, dtype=torch.bfloat16, device="cuda")
    lib.moe_expert_ffn(d, T, x, dev_tensor(c.gate_up, True), dev_tensor(c.down, True), w,
                       offsets, ss, y, ws)
    lib.moe_combine(d, T, y, None, out)
    torch.cuda.synchronize()
    rows = np.array(sorted(set(np.random.default_rng(2).choice(T, 24, replace=False)) |
                           {0, T - 1}))
    ref = oracle.experts(c.x.f32[rows], c.gate_up.f32, c.down.f32, oi[rows], ow[rows])
    assert rel_max_err(host(out)[rows], ref) <= BF16_TOL
    # whole row tiles: the last 256 sorted rows (the ragged tail) of the
    # hottest expert and every row of the rarest one, slot by slot
    hot, rare = int(np.argmax(oc)), int(np.argmin(oc))
    picks = np.concatenate([os_[oo[hot + 1] - 256:oo[hot + 1]], os_[oo[rare]:oo[rare + 1]],
                            os_[:64]])
    tok, kk = picks // c.K, picks % c.K
    yh = host(y.view(T * c.K, c.H)[torch.from_numpy(picks.astype(np.int64)).cuda()])
    ref = oracle.experts(c.x.f32[tok], c.gate_up.f32, c.down.f32, oi[tok, kk][:, None],
                         ow[tok, kk][:, None])
    bound, exact = bf16_path_bound(c.x.f32[tok], c.gate_up.f32, c.down.f32,
                                   oi[tok, kk][:, None], ow[tok, kk][:, None], out_rounded=False)
    np.testing.assert_allclose(exact, ref, rtol=1e-9, atol=1e-12)
    assert np.all(np.abs(yh - ref) <= bound), float(np.max(np.abs(yh - ref) / bound))
