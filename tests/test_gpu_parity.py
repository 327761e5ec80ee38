"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: routing indices, per-expert counts, offsets and the slot permutation
bit-exact (and the router's fp32 logits bit-identical); expert / block
outputs within 2e-2 x RMS(oracle) on the bf16 path and 1e-4 x RMS(oracle) on
the fp32 path (max |err| over the whole compared tensor).
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_moe_transformer_router_amd import synth
from tests.gpu_util import (BF16_TOL, F32_TOL, bf16_path_bound, dev_f32, dev_tensor, host, note,
                            rel_max_err, ws_logits_view)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sparse_moe_transformer_router_amd import lib
else:  # collected on CPU-only hosts but every test here is marked gpu
    lib = None


def _dims(c, dense=0, slot=None):
    act = lib.MOE_BF16 if c.bf16 else lib.MOE_F32
    return lib.dims(c.H, c.E, c.K, c.I, dense, c.eps, act, lib.MOE_F32 if slot is None else slot)


def _run_router(c, pre_gain=None):
    # the router does not use the expert width; the toy's I=1 is below the ABI's minimum
    d = lib.dims(c.H, c.E, c.K, max(32, c.I), 0, c.eps, lib.MOE_BF16 if c.bf16 else lib.MOE_F32)
    ws = lib.workspace(d, c.T)
    x = dev_tensor(c.x, c.bf16)
    idx = torch.empty(c.T, c.K, dtype=torch.int32, device="cuda")
    w = torch.empty(c.T, c.K, dtype=torch.float32, device="cuda")
    lib.moe_router(d, c.T, x, dev_f32(c.router_w), dev_f32(c.router_scale),
                   dev_f32(c.per_expert_scale), None if pre_gain is None else dev_f32(pre_gain),
                   idx, w, ws)
    torch.cuda.synchronize()
    return host(idx), host(w), host(ws_logits_view(ws, c.T, c.E))


def _check_router(c, pre_gain=None):
    note(f"router T={c.T} H={c.H} E={c.E} K={c.K} bf16={c.bf16} pre={pre_gain is not None}")
    gi, gw, gl = _run_router(c, pre_gain)
    oi, ow, ol = oracle.router(c.x.f32, c.router_w, c.router_scale, c.per_expert_scale, c.K,
                               c.eps, pre_gain=pre_gain, want_logits=True)
    assert np.array_equal(gl.view(np.uint32), ol.view(np.uint32)), "logits differ in bits"
    assert np.array_equal(gi, oi), "routing indices differ"
    np.testing.assert_allclose(gw, ow, rtol=1e-6, atol=0)
    return gi, gw


# ---------------------------------------------------------------------------
# router
# ---------------------------------------------------------------------------
def test_router_toy():
    gi, gw = _check_router(synth.toy_case())
    assert gi.tolist() == [[0, 1], [0, 1]]


def test_router_tiny_fp32():
    _check_router(synth.tiny_case())


# up to 448 tokens the chunk-parallel logits kernel, past it the chunk-split
# kernel (four wave groups here)
@pytest.mark.parametrize("T", [1, 2, 3, 8, 9, 32, 63, 64, 200, 448, 449])
def test_router_decode_sizes(T):
    _check_router(synth.moe_case(T, seed=T, I=32, router_scale_std=0.05))


# the chunk-split kernel at 26B shapes: 257 and 2048 tokens its 16-token form
# (six wave groups; 2048: 256 blocks, the largest grid of that form), 2049
# and 4096 its 32-token four-group form (130 and 256 blocks), 4128 its
# two-group form (258 blocks)
@pytest.mark.parametrize("T,skew", [(257, False), (2048, True), (2049, False), (4096, True),
                                    (4128, False)])
def test_router_prefill_sizes(T, skew):
    _check_router(synth.moe_case(T, seed=11, I=32, skew=skew))


@pytest.mark.parametrize("T", [5, 300, 700])
def test_router_with_pre_norm(T):
    c = synth.moe_case(T, seed=12, I=32, router_scale_std=0.05)
    g = (1 + 0.05 * np.random.default_rng(0).standard_normal(c.H)).astype(np.float32)
    _check_router(c, pre_gain=g)


@pytest.mark.parametrize("T,H,E,K,bf16", [
    (600, 128, 6, 2, False),    # E % 4 != 0: lane-per-token tiled kernel
    # chunk-split kernel: 16-token blocks with 6 groups while their grid fits
    # 256 blocks, else 32-token blocks with 4 groups while theirs does, else 2
    (600, 192, 132, 4, True),   # 16-token, 3 chunks (groups 3-5 idle), ragged expert block
    (1000, 320, 64, 4, False),  # 16-token, 5 chunks: group 5 idle
    (1000, 832, 64, 4, True),   # 16-token, 13 chunks: a last round with one group
    (1500, 576, 132, 4, False), # 32-token (282 16-token blocks), 4 groups, 9 chunks
    (4100, 64, 256, 8, False),  # 2 groups, 1 chunk, ragged token tail
    (9000, 192, 128, 8, True),  # 2 groups, 3 chunks: a last round with one group
])
def test_router_large_batch_kernels(T, H, E, K, bf16):
    _check_router(synth.tiny_case(seed=T + E, T=T, H=H, E=E, K=K, I=32, bf16=bf16))


def test_router_fp32_large_hidden_and_k_equals_e():
    c = synth.tiny_case(seed=3, T=70, H=4608, E=16, K=16, I=32)
    _check_router(c)


@pytest.mark.parametrize("T,skew,pre", [(1, False, False), (13, False, True), (64, False, False),
                                        (65, False, False), (128, False, False),
                                        (129, False, False), (300, True, True),
                                        (600, False, True)])
def test_route_fused(T, skew, pre):
    """moe_route (router + dispatch in one call) against the oracle's router
    and dispatch: the dispatch inside the top-K kernel up to 1024 slots (128
    tokens at top-8), the dispatch kernels after it past that, after the
    chunk-parallel logits (<= 448 tokens) or the chunk-split kernel."""
    c = synth.moe_case(T, seed=20 + T, I=32, skew=skew, router_scale_std=0.05)
    g = (1 + 0.05 * np.random.default_rng(1).standard_normal(c.H)).astype(np.float32) if pre \
        else None
    note(f"route T={T} skew={skew} pre={pre}")
    d = _dims(c)
    ws = lib.workspace(d, c.T)
    idx = torch.empty(T, c.K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, c.K, dtype=torch.float32, device="cuda")
    counts = torch.empty(c.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(c.E + 1, dtype=torch.int32, device="cuda")
    ss = torch.empty(T * c.K, dtype=torch.int32, device="cuda")
    lib.moe_route(d, T, dev_tensor(c.x, True), dev_f32(c.router_w), dev_f32(c.router_scale),
                  dev_f32(c.per_expert_scale), None if g is None else dev_f32(g), idx, w, counts,
                  offsets, ss, ws)
    torch.cuda.synchronize()
    oi, ow = oracle.router(c.x.f32, c.router_w, c.router_scale, c.per_expert_scale, c.K, c.eps,
                           pre_gain=g)
    assert np.array_equal(host(idx), oi)
    np.testing.assert_allclose(host(w), ow, rtol=1e-6, atol=0)
    oc, oo, os_ = oracle.dispatch(oi, c.E)
    assert np.array_equal(host(counts), oc)
    assert np.array_equal(host(offsets), oo)
    assert np.array_equal(host(ss), os_)


# ---------------------------------------------------------------------------
# dispatch
# ---------------------------------------------------------------------------
def _random_routing(T, E, K, seed, zipf=False):
    rng = np.random.default_rng(seed)
    p = None
    if zipf:
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p = rng.permutation(p / p.sum())
    return np.stack([rng.choice(E, K, replace=False, p=p) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,K,zipf", [(1, 128, 8, False), (7, 8, 2, False), (64, 128, 8, False),
                                        (128, 128, 8, False), (129, 128, 8, False),
                                        (1000, 256, 3, True), (4096, 128, 8, True),
                                        (3, 1, 1, False)])
def test_dispatch_bit_exact(T, E, K, zipf):
    note(f"dispatch T={T} E={E} K={K} zipf={zipf}")
    idx = _random_routing(T, E, K, seed=T + E, zipf=zipf)
    d = lib.dims(64, E, K, 32)
    ws = lib.workspace(d, T)
    di = torch.from_numpy(idx).cuda()
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    ss = torch.empty(T * K, dtype=torch.int32, device="cuda")
    lib.moe_dispatch(d, T, di, counts, offsets, ss, ws)
    torch.cuda.synchronize()
    oc, oo, os_ = oracle.dispatch(idx, E)
    assert np.array_equal(host(counts), oc)
    assert np.array_equal(host(offsets), oo)
    assert np.array_equal(host(ss), os_)


# ---------------------------------------------------------------------------
# experts (moe_expert_ffn + moe_combine), routed by the oracle
# ---------------------------------------------------------------------------
def _expert_path(c, idx, w, slot_bf16=None):
    slot = None if slot_bf16 is None else (lib.MOE_BF16 if slot_bf16 else lib.MOE_F32)
    d = _dims(c, slot=slot)
    ws = lib.workspace(d, c.T)
    E, T, K = c.E, c.T, c.K
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    ss = torch.empty(T * K, dtype=torch.int32, device="cuda")
    di, dw = torch.from_numpy(idx).cuda(), dev_f32(w)
    lib.moe_dispatch(d, T, di, counts, offsets, ss, ws)
    ydt = torch.float32 if (d.slot_dtype == lib.MOE_F32) else torch.bfloat16
    adt = torch.bfloat16 if c.bf16 else torch.float32
    y = torch.empty(T, K, c.H, dtype=ydt, device="cuda")
    out = torch.empty(T, c.H, dtype=adt, device="cuda")
    lib.moe_expert_ffn(d, T, dev_tensor(c.x, c.bf16), dev_tensor(c.gate_up, c.bf16),
                       dev_tensor(c.down, c.bf16), dw, offsets, ss, y, ws)
    lib.moe_combine(d, T, y, None, out)
    torch.cuda.synchronize()
    return host(y), host(out)


def test_experts_tiny_fp32():
    c = synth.tiny_case()
    note("experts tiny fp32")
    idx, w = oracle.router(c.x.f32, c.router_w, c.router_scale, c.per_expert_scale, c.K, c.eps)
    y, out = _expert_path(c, idx, w)
    ref = oracle.experts(c.x.f32, c.gate_up.f32, c.down.f32, idx, w)
    assert rel_max_err(out, ref) <= F32_TOL
    ref0 = oracle.experts(c.x.f32, c.gate_up.f32, c.down.f32, idx[:, :1], w[:, :1])
    assert rel_max_err(y[:, 0], ref0) <= F32_TOL


@pytest.mark.parametrize("seed,T,H,E,K,I", [(1, 37, 128, 16, 4, 64), (2, 200, 192, 8, 2, 96),
                                            (3, 5, 64, 4, 4, 32), (4, 64, 128, 4, 2, 64),
                                            (5, 16, 64, 2, 1, 32), (6, 30, 256, 3, 3, 96)])
def test_experts_small_bf16_and_fp32(seed, T, H, E, K, I):
    """Small shapes with unit-variance weights: the fp32 path is held to
    1e-4 x RMS; the bf16 path, whose two bf16 roundings exceed 2e-2 x RMS on
    such heavy-tailed small layers, to the per-element rounding bound."""
    for bf in (False, True):
        c = synth.tiny_case(seed=seed, T=T, H=H, E=E, K=K, I=I, bf16=bf)
        note(f"experts small T={T} H={H} E={E} K={K} I={I} bf16={bf}")
        idx, w = oracle.router(c.x.f32, c.router_w, c.router_scale, c.per_expert_scale, K, c.eps)
        y, out = _expert_path(c, idx, w)
        ref = oracle.experts(c.x.f32, c.gate_up.f32, c.down.f32, idx, w)
        if not bf:
            assert rel_max_err(out, ref) <= F32_TOL
            continue
        bound, exact = bf16_path_bound(c.x.f32, c.gate_up.f32, c.down.f32, idx, w)
        np.testing.assert_allclose(exact, ref, rtol=1e-9, atol=1e-12)
        assert np.all(np.abs(out - ref) <= bound), float(np.max(np.abs(out - ref) / bound))


@pytest.fixture(scope="module")
def case26b():
    return synth.moe_case(256, seed=0)


# 8 and 9 straddle the switch of the decode down kernel to activation rows
# staged in LDS, 64 and 65 the switch of gate_up to 32-row tiles; 256 tokens
# (16 rows per expert) is the largest batch the weight-streaming kernels take
@pytest.mark.parametrize("T", [1, 8, 9, 16, 64, 65, 128, 256])
def test_experts_26b_decode(case26b, T):
    """The expert output (bf16) within its per-element rounding bound at every
    size, and each fp32 slot within 2e-2 x RMS.  The combined output is also
    held to 2e-2 x RMS up to 128 tokens; at 256 tokens (720k outputs) the tail
    of its two bf16 roundings (h before the down projection, then the output)
    alone goes past the bar: a CPU model of exactly those roundings gives
    0.0208 x RMS on this case, rounding the exact result alone 0.0124.  The bar
    is stated for the layer's output, which test_block_26b_decode checks at
    256 tokens, every row."""
    c = synth.MoECase(T, case26b.H, case26b.E, case26b.K, case26b.I, True, case26b.eps,
                      synth.Tensor(case26b.x.f32[:T], case26b.x.bf16[:T]), case26b.router_w,
                      case26b.router_scale, case26b.per_expert_scale, case26b.gate_up,
                      case26b.down)
    note(f"experts 26B decode T={T}")
    idx, w = oracle.router(c.x.f32, c.router_w, c.router_scale, c.per_expert_scale, c.K, c.eps)
    y, out = _expert_path(c, idx, w)
    ref = oracle.experts(c.x.f32, c.gate_up.f32, c.down.f32, idx, w)
    bound, exact = bf16_path_bound(c.x.f32, c.gate_up.f32, c.down.f32, idx, w)
    np.testing.assert_allclose(exact, ref, rtol=1e-9, atol=1e-12)
    assert np.all(np.abs(out - ref) <= bound), float(np.max(np.abs(out - ref) / bound))
    if T <= 128:
        assert rel_max_err(out, ref) <= BF16_TOL
    # each slot on its own (slot k = the k-th ranked expert's weighted output)
    for k in (0, c.K - 1):
        refk = oracle.experts(c.x.f32, c.gate_up.f32, c.down.f32, idx[:, k:k + 1],
                              w[:, k:k + 1])
        assert rel_max_err(y[:, k], refk) <= BF16_TOL


def _per_slot_refs(c, idx, w):
    """The oracle's output of each slot on its own: [T, K, H] fp64."""
    return np.stack([oracle.experts(c.x.f32, c.gate_up.f32, c.down.f32, idx[:, k:k + 1],
                                    w[:, k:k + 1]) for k in range(c.K)], 1)


def test_experts_26b_prefill_skewed_all_rows():
    """4096 skewed tokens (hottest expert ~3100 slots, a dozen experts empty),
    every row of every slot, through moe_route, moe_expert_ffn and moe_combine
    (the calls of moe_forward).

    - routing, counts, offsets and the slot permutation exact;
    - the in-order fp32 sum of each token's slots within 2e-2 x RMS of the
      oracle, and every fp32 slot within its per-element rounding bound;
    - the bf16 output equal to that sum rounded once to nearest-even, bit for
      bit, and within the per-element rounding bound of the bf16 path.
    The whole-tensor bar is not put on the bf16 output itself: under this
    load the largest outputs reach ~13 x RMS, so rounding the exact result to
    bf16 alone moves it by 0.026 x RMS.  Nor on a single slot: h rounded to
    bf16 before the down projection moves the first slot by up to 0.023 x its
    RMS here (a CPU model of that one rounding gives the same), while the sum
    of the eight slots, the experts' result, stays near 0.015."""
    c = synth.moe_case(4096, seed=0, skew=True)
    note("experts 26B prefill 4096 skewed, all rows")
    d = _dims(c)
    T, K, E = c.T, c.K, c.E
    ws = lib.workspace(d, T)
    x = dev_tensor(c.x, True)
    idx = torch.empty(T, K, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    ss = torch.empty(T * K, dtype=torch.int32, device="cuda")
    lib.moe_route(d, T, x, dev_f32(c.router_w), dev_f32(c.router_scale),
                  dev_f32(c.per_expert_scale), None, idx, w, counts, offsets, ss, ws)
    y = torch.empty(T, K, c.H, dtype=torch.float32, device="cuda")
    out = torch.empty(T, c.H, dtype=torch.bfloat16, device="cuda")
    lib.moe_expert_ffn(d, T, x, dev_tensor(c.gate_up, True), dev_tensor(c.down, True), w,
                       offsets, ss, y, ws)
    lib.moe_combine(d, T, y, None, out)
    torch.cuda.synchronize()
    oi, ow = oracle.router(c.x.f32, c.router_w, c.router_scale, c.per_expert_scale, K, c.eps)
    assert np.array_equal(host(idx), oi)
    np.testing.assert_allclose(host(w), ow, rtol=1e-6, atol=0)
    oc, oo, os_ = oracle.dispatch(oi, E)
    assert np.array_equal(host(counts), oc)
    assert np.array_equal(host(offsets), oo)
    assert np.array_equal(host(ss), os_)
    assert oc.max() > 1000 and (oc == 0).sum() > 0
    yh = host(y)
    refs = _per_slot_refs(c, oi, ow)
    for k in range(K):
        bk, ek = bf16_path_bound(c.x.f32, c.gate_up.f32, c.down.f32, oi[:, k:k + 1],
                                 ow[:, k:k + 1], out_rounded=False)
        np.testing.assert_allclose(ek, refs[:, k], rtol=1e-9, atol=1e-12)
        err = np.abs(yh[:, k] - refs[:, k])
        assert np.all(err <= bk), (k, float(np.max(err / bk)))
    acc = np.zeros((T, c.H), np.float32)
    for k in range(K):
        acc = acc + yh[:, k]                        # fp32, slot order, from +0
    ref = refs.sum(1)
    assert rel_max_err(acc, ref) <= BF16_TOL
    got = host(out)
    assert np.array_equal(got, torch.from_numpy(acc).to(torch.bfloat16).float().numpy())
    bound, exact = bf16_path_bound(c.x.f32, c.gate_up.f32, c.down.f32, oi, ow)
    np.testing.assert_allclose(exact, ref, rtol=1e-9, atol=1e-12)
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) / bound))


# ---------------------------------------------------------------------------
# whole experts-only path and the dual-path layer
# ---------------------------------------------------------------------------
def test_forward_tiny_fp32_and_determinism():
    c = synth.tiny_case()
    note("forward tiny fp32")
    d = _dims(c)
    ws = lib.workspace(d, c.T)
    x = dev_tensor(c.x, False)
    args = (dev_f32(c.router_w), dev_f32(c.router_scale), dev_f32(c.per_expert_scale),
            dev_tensor(c.gate_up, False), dev_tensor(c.down, False))
    outs = []
    for _ in range(2):
        out = torch.empty(c.T, c.H, device="cuda")
        lib.moe_forward(d, c.T, x, *args, out, None, None, ws)
        torch.cuda.synchronize()
        outs.append(host(out))
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    idx, w = oracle.router(c.x.f32, c.router_w, c.router_scale, c.per_expert_scale, c.K, c.eps)
    ref = oracle.experts(c.x.f32, c.gate_up.f32, c.down.f32, idx, w)
    assert rel_max_err(outs[0], ref) <= F32_TOL


def _run_block(b, bf16, slot_bf16=None):
    m = b.moe
    act = lib.MOE_BF16 if bf16 else lib.MOE_F32
    slot = lib.MOE_F32 if slot_bf16 is None else (lib.MOE_BF16 if slot_bf16 else lib.MOE_F32)
    d = lib.dims(m.H, m.E, m.K, m.I, b.D, m.eps, act, slot)
    ws = lib.workspace(d, m.T)
    dt = lambda t: dev_tensor(t, bf16)  # noqa: E731
    keep = [dev_f32(b.g_pre), dev_f32(b.g_pre2), dev_f32(b.g_post1), dev_f32(b.g_post2),
            dev_f32(b.g_post), dt(b.dense_gate), dt(b.dense_up), dt(b.dense_down),
            dev_f32(m.router_w), dev_f32(m.router_scale), dev_f32(m.per_expert_scale),
            dt(m.gate_up), dt(m.down)]
    wts = lib.ffn_weights(*keep, b.layer_scalar)
    x = dt(m.x)
    out = torch.empty(m.T, m.H, dtype=torch.bfloat16 if bf16 else torch.float32, device="cuda")
    ffn = torch.empty(m.T, m.H, dtype=torch.float32, device="cuda")
    idx = torch.empty(m.T, m.K, dtype=torch.int32, device="cuda")
    w = torch.empty(m.T, m.K, dtype=torch.float32, device="cuda")
    lib.gemma4_ffn_block(d, m.T, x, wts, out, ffn, idx, w, ws)
    torch.cuda.synchronize()
    return host(out), host(ffn), host(idx), host(w)


def _oracle_block(b, rows=None):
    m = b.moe
    sel = slice(None) if rows is None else rows
    return oracle.block(m.x.f32[sel], b.g_pre, b.g_pre2, b.g_post1, b.g_post2, b.g_post,
                        b.dense_gate.f32, b.dense_up.f32, b.dense_down.f32, m.router_w,
                        m.router_scale, m.per_expert_scale, m.gate_up.f32, m.down.f32,
                        b.layer_scalar, m.K)


@pytest.mark.parametrize("bf16", [False, True])
def test_block_small(bf16):
    b = synth.block_case(45, seed=3, H=128, E=16, K=4, I=64, D=96, weight_std=0.1, bf16=bf16)
    note(f"block small bf16={bf16}")
    out, ffn, idx, w = _run_block(b, bf16)
    r = _oracle_block(b)
    assert np.array_equal(idx, r["idx"])
    np.testing.assert_allclose(w, r["w"], rtol=1e-6)
    tol = BF16_TOL if bf16 else F32_TOL
    assert rel_max_err(ffn, r["o"]) <= tol
    assert rel_max_err(out, r["out"]) <= tol


@pytest.mark.parametrize("T", [64, 128, 256])
def test_block_26b_decode(T):
    """The full-size layer at decode batches, every row checked: at 64 tokens
    the dense branch and the experts take the weight-streaming kernels, at 128
    and 256 the dense branch takes the tiled GEMMs and the experts still
    stream."""
    b = synth.block_case(T, seed=4)
    note(f"block 26B T={T}")
    out, ffn, idx, w = _run_block(b, True)
    r = _oracle_block(b)
    assert np.array_equal(idx, r["idx"])
    np.testing.assert_allclose(w, r["w"], rtol=1e-6)
    assert rel_max_err(ffn, r["o"]) <= BF16_TOL
    assert rel_max_err(out, r["out"]) <= BF16_TOL


def test_block_26b_2048_all_rows():
    """The full-size layer at 2048 tokens (about 128 slots per expert, the
    tiled GEMMs for the experts and the dense branch), every row: routing
    exact, the pre-residual output o and the layer output within 2e-2 x RMS of
    the oracle."""
    b = synth.block_case(2048, seed=0)
    note("block 26B T=2048, all rows")
    out, ffn, idx, w = _run_block(b, True)
    r = _oracle_block(b)
    assert np.array_equal(idx, r["idx"])
    np.testing.assert_allclose(w, r["w"], rtol=1e-6)
    assert rel_max_err(ffn, r["o"]) <= BF16_TOL
    assert rel_max_err(out, r["out"]) <= BF16_TOL
