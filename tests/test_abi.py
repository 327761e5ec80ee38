"""The C-ABI library on the CPU: it loads, exports every function that
include/moe.h declares, and rejects bad arguments on the host before any HIP
call (so these tests need no GPU).  No test here launches a kernel."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

lib_mod = pytest.importorskip("sparse_moe_transformer_router_amd.lib",
                              reason="libmoe.so not built")
L = lib_mod.raw()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_expected_calls():
    fns = declared_functions()
    for name in ("moe_router", "moe_dispatch", "moe_expert_ffn", "moe_combine",
                 "gemma4_ffn_block", "gemma4_ffn_block_q", "moe_forward", "moe_workspace_size",
                 "moe_last_error"):
        assert name in fns


def test_every_declared_symbol_is_exported():
    out = subprocess.run(["nm", "-D", "--defined-only", lib_mod.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(L, name) is not None


FAKE = ctypes.c_void_p(0x10000)        # never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x10004)


def D(**kw):
    base = dict(hidden=2816, num_experts=128, top_k=8, expert_inter=704, dense_inter=2112,
                eps=1e-6, act=lib_mod.MOE_BF16)
    base.update(kw)
    return lib_mod.dims(**base)


def router(d, T, x=FAKE, ws=FAKE, ws_bytes=1 << 40, pre=None, idx=FAKE):
    return L.moe_router(ctypes.byref(d), T, x, FAKE, FAKE, FAKE, pre, idx, FAKE, ws, ws_bytes,
                        None)


def test_workspace_size_is_monotone_and_rejects_bad_dims():
    d = D()
    sizes = [L.moe_workspace_size(ctypes.byref(d), t) for t in (1, 8, 64, 4096)]
    assert all(s > 0 for s in sizes) and sizes == sorted(sizes)
    assert L.moe_workspace_size(ctypes.byref(D(hidden=100)), 8) == 0
    assert "hidden" in lib_mod.last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=100), lib_mod.MOE_ERR_UNSUPPORTED),
    (dict(hidden=0), lib_mod.MOE_ERR_UNSUPPORTED),
    (dict(num_experts=0), lib_mod.MOE_ERR_UNSUPPORTED),
    (dict(num_experts=300), lib_mod.MOE_ERR_UNSUPPORTED),
    (dict(top_k=0), lib_mod.MOE_ERR_UNSUPPORTED),
    (dict(top_k=129), lib_mod.MOE_ERR_UNSUPPORTED),
    (dict(num_experts=4, top_k=5), lib_mod.MOE_ERR_UNSUPPORTED),
    (dict(expert_inter=700), lib_mod.MOE_ERR_UNSUPPORTED),
    (dict(eps=0.0), lib_mod.MOE_ERR_ARG),
    (dict(act=7), lib_mod.MOE_ERR_ARG),
    (dict(act=lib_mod.MOE_F32, slot=lib_mod.MOE_BF16), lib_mod.MOE_ERR_UNSUPPORTED),
])
def test_bad_dims_are_rejected(kw, code):
    assert router(D(**kw), 4) == code
    assert lib_mod.last_error()


def test_bad_tokens_pointers_and_workspace():
    d = D()
    assert router(d, -1) == lib_mod.MOE_ERR_ARG
    assert router(d, 70000) == lib_mod.MOE_ERR_ARG
    assert router(d, 4, x=None) == lib_mod.MOE_ERR_ARG and "x" in lib_mod.last_error()
    assert router(d, 4, x=MISALIGNED) == lib_mod.MOE_ERR_ARG
    assert router(d, 4, pre=MISALIGNED) == lib_mod.MOE_ERR_ARG
    assert router(d, 4, idx=None) == lib_mod.MOE_ERR_ARG
    assert router(d, 4, ws=None) == lib_mod.MOE_ERR_WORKSPACE
    assert router(d, 4, ws=ctypes.c_void_p(0x10010)) == lib_mod.MOE_ERR_WORKSPACE
    need = L.moe_workspace_size(ctypes.byref(d), 4)
    assert router(d, 4, ws_bytes=need - 1) == lib_mod.MOE_ERR_WORKSPACE
    assert str(need) in lib_mod.last_error()


def test_zero_tokens_is_a_no_op_everywhere():
    d = D()
    dp = ctypes.byref(d)
    assert router(d, 0, x=None, ws=None, ws_bytes=0) == lib_mod.MOE_OK
    assert L.moe_dispatch(dp, 0, None, None, None, None, None, 0, None) == lib_mod.MOE_OK
    assert L.moe_expert_ffn(dp, 0, *([None] * 8), 0, None) == lib_mod.MOE_OK
    assert L.moe_combine(dp, 0, None, None, None, None) == lib_mod.MOE_OK
    assert L.moe_forward(dp, 0, *([None] * 10), 0, None) == lib_mod.MOE_OK
    assert L.gemma4_ffn_block(dp, 0, None, None, None, None, None, None, None, 0,
                              None) == lib_mod.MOE_OK


def test_block_requires_dense_branch_and_weights():
    d = D(dense_inter=0)
    assert L.gemma4_ffn_block(ctypes.byref(d), 4, FAKE, None, FAKE, None, None, None, FAKE,
                              1 << 40, None) == lib_mod.MOE_ERR_UNSUPPORTED
    d = D()
    assert L.gemma4_ffn_block(ctypes.byref(d), 4, FAKE, None, FAKE, None, None, None, FAKE,
                              1 << 40, None) == lib_mod.MOE_ERR_ARG
    w = lib_mod.Gemma4FfnWeights()
    for f, _ in w._fields_[:-1]:
        setattr(w, f, 0x10000)
    w.dense_up = None
    assert L.gemma4_ffn_block(ctypes.byref(d), 4, FAKE, ctypes.byref(w), FAKE, None, None, None,
                              FAKE, 1 << 40, None) == lib_mod.MOE_ERR_ARG
    assert "dense_up" in lib_mod.last_error()


def test_quantized_block_validates():
    """gemma4_ffn_block_q: a no-op at 0 tokens, and every refusal before any
    launch (format, dtype, token limit, dense branch, pointers, workspace)."""
    Lq = L.gemma4_ffn_block_q
    Lq.argtypes = [ctypes.POINTER(lib_mod.MoeDims), ctypes.c_int32, ctypes.c_void_p,
                   ctypes.POINTER(lib_mod.Gemma4FfnWeightsQ)] + [ctypes.c_void_p] * 5 + \
        [ctypes.c_size_t, ctypes.c_void_p]
    d = D()
    dp = ctypes.byref(d)
    assert Lq(dp, 0, None, None, None, None, None, None, None, 0, None) == lib_mod.MOE_OK
    w = lib_mod.Gemma4FfnWeightsQ()
    for f, _ in w._fields_[1:-1]:
        setattr(w, f, 0x10000)
    w.fmt = lib_mod.MOE_W_INT8
    wp = ctypes.byref(w)
    args = (FAKE, wp, FAKE, None, None, None, FAKE, 1 << 40, None)
    # past 256 tokens the tiled kernels take over: validation goes on to the
    # workspace check
    assert Lq(dp, 257, FAKE, wp, FAKE, None, None, None, FAKE, 0,
              None) == lib_mod.MOE_ERR_WORKSPACE
    d32 = D(act=lib_mod.MOE_F32)
    assert Lq(ctypes.byref(d32), 4, *args) == lib_mod.MOE_ERR_UNSUPPORTED
    d0 = D(dense_inter=0)
    assert Lq(ctypes.byref(d0), 4, *args) == lib_mod.MOE_ERR_UNSUPPORTED
    assert Lq(dp, 4, FAKE, None, FAKE, None, None, None, FAKE, 1 << 40,
              None) == lib_mod.MOE_ERR_ARG
    w.fmt = 9
    assert Lq(dp, 4, *args) == lib_mod.MOE_ERR_ARG and "format" in lib_mod.last_error()
    w.fmt = lib_mod.MOE_W_MXFP4
    w.dense_down_scale = None
    assert Lq(dp, 4, *args) == lib_mod.MOE_ERR_ARG
    assert "dense_down_scale" in lib_mod.last_error()
    w.dense_down_scale = 0x10000
    w.gate_up_q = 0x10004
    assert Lq(dp, 4, *args) == lib_mod.MOE_ERR_ARG and "aligned" in lib_mod.last_error()
    w.gate_up_q = 0x10000
    assert Lq(dp, 4, FAKE, wp, FAKE, None, None, None, FAKE, 0,
              None) == lib_mod.MOE_ERR_WORKSPACE
    # MXFP4 stages a contraction of at most 8192 weights' block scales
    dwide = D(dense_inter=8224)
    assert Lq(ctypes.byref(dwide), 4, *args) == lib_mod.MOE_ERR_UNSUPPORTED
    assert "dense_inter" in lib_mod.last_error()
    w.fmt = lib_mod.MOE_W_INT8
    assert Lq(ctypes.byref(dwide), 4, FAKE, wp, FAKE, None, None, None, FAKE, 0,
              None) == lib_mod.MOE_ERR_WORKSPACE


def test_other_calls_validate():
    d = D()
    dp = ctypes.byref(d)
    assert L.moe_dispatch(dp, 4, FAKE, FAKE, None, FAKE, FAKE, 1 << 40,
                          None) == lib_mod.MOE_ERR_ARG
    assert L.moe_expert_ffn(dp, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10,
                            None) == lib_mod.MOE_ERR_WORKSPACE
    assert L.moe_combine(dp, 4, FAKE, MISALIGNED, FAKE, None) == lib_mod.MOE_ERR_ARG
    assert L.moe_forward(dp, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, FAKE,
                         1 << 40, None) == lib_mod.MOE_ERR_ARG


def test_int8_entry_points_validate_on_the_host():
    q = L.moe_quantize_int8
    assert q(0, 64, None, None, None, None) == lib_mod.MOE_OK
    assert q(-1, 64, FAKE, FAKE, FAKE, None) == lib_mod.MOE_ERR_ARG
    assert q(4, 60, FAKE, FAKE, FAKE, None) == lib_mod.MOE_ERR_ARG and "cols" in lib_mod.last_error()
    assert q(4, 64, None, FAKE, FAKE, None) == lib_mod.MOE_ERR_ARG
    assert q(4, 64, FAKE, MISALIGNED, FAKE, None) == lib_mod.MOE_ERR_ARG
    f = L.moe_expert_ffn_int8
    d = D()
    args = [FAKE] * 10
    assert f(ctypes.byref(d), 0, *([None] * 10), 0, None) == lib_mod.MOE_OK
    assert f(ctypes.byref(d), 4097, *args, 0, None) == lib_mod.MOE_ERR_WORKSPACE
    d32 = D(act=lib_mod.MOE_F32)
    assert f(ctypes.byref(d32), 4, *args, 1 << 40, None) == lib_mod.MOE_ERR_UNSUPPORTED
    bad = list(args)
    bad[2] = None  # gate_up scales
    assert f(ctypes.byref(d), 4, *bad, 1 << 40, None) == lib_mod.MOE_ERR_ARG
    assert f(ctypes.byref(d), 4, *args, 0, None) == lib_mod.MOE_ERR_WORKSPACE


def test_dense_mask_entry_point_and_any_top_k_on_slot_calls():
    """The all-experts layout call validates on the host; the calls that only
    see token-slots take top_k up to num_experts, routing keeps top_k <= 32."""
    f = L.moe_dense_mask_dispatch
    d = D()
    dp = ctypes.byref(d)
    assert f(dp, 0, None, None, None, None, None, None) == lib_mod.MOE_OK
    assert f(dp, 4, FAKE, None, FAKE, FAKE, FAKE, None) == lib_mod.MOE_ERR_ARG
    assert f(dp, 4, FAKE, FAKE, FAKE, MISALIGNED, FAKE, None) == lib_mod.MOE_ERR_ARG
    assert f(dp, 8193, FAKE, FAKE, FAKE, FAKE, FAKE, None) == lib_mod.MOE_ERR_UNSUPPORTED
    assert "2^20" in lib_mod.last_error()
    dall = D(top_k=128)
    pa = ctypes.byref(dall)
    assert L.moe_workspace_size(pa, 64) > L.moe_workspace_size(dp, 64)
    assert L.moe_combine(pa, 4, FAKE, MISALIGNED, FAKE, None) == lib_mod.MOE_ERR_ARG
    assert L.moe_expert_ffn(pa, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10,
                            None) == lib_mod.MOE_ERR_WORKSPACE
    assert router(dall, 4) == lib_mod.MOE_ERR_UNSUPPORTED
    assert L.moe_workspace_size(ctypes.byref(D(top_k=129)), 64) == 0


def test_probe_library_exports_and_validates():
    """The measurement probes: every symbol include/moe_probe.h declares is
    exported, and bad arguments are refused before any launch."""
    probe = pytest.importorskip("sparse_moe_transformer_router_amd.probe",
                                reason="libmoe_probe.so not built")
    header = os.path.join(ROOT, "include", "moe_probe.h")
    text = re.sub(r"/\*.*?\*/", "", open(header).read(), flags=re.S)
    names = set(re.findall(r"^\s*(?:long long|int)\s+(\w+)\s*\(", text, flags=re.M))
    assert {"moe_probe_stream_read", "moe_probe_mfma", "moe_probe_read_blocks",
            "moe_probe_mfma_flops"} <= names
    out = subprocess.run(["nm", "-D", "--defined-only", probe.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    assert names <= exported
    P = probe.raw()
    assert P.moe_probe_read_blocks() > 0
    assert P.moe_probe_mfma_flops(2, 3) == 2 * 4 * 3 * 8 * 2 * 32 * 32 * 16
    assert P.moe_probe_stream_read(None, 1024, FAKE, None) == -1
    assert P.moe_probe_stream_read(FAKE, 1000, FAKE, None) == -1
    assert P.moe_probe_stream_read(MISALIGNED, 1024, FAKE, None) == -1
    assert P.moe_probe_mfma(0, 10, FAKE, None) == -1
    assert P.moe_probe_mfma(4, 0, FAKE, None) == -1
    assert P.moe_probe_mfma(4, 10, None, None) == -1


def test_quantized_format_entry_points_validate_on_the_host():
    """moe_quantize / moe_dequantize / moe_expert_ffn_q refuse unknown formats,
    bad sizes and pointers before any launch."""
    qz, dq, ffn = L.moe_quantize, L.moe_dequantize, L.moe_expert_ffn_q
    W8, F8, MX = lib_mod.MOE_W_INT8, lib_mod.MOE_W_FP8, lib_mod.MOE_W_MXFP4
    for f in (W8, F8, MX):
        assert qz(f, 0, 64, None, None, None, None) == lib_mod.MOE_OK
        assert dq(f, 0, 64, None, None, None, None) == lib_mod.MOE_OK
    assert qz(7, 4, 64, FAKE, FAKE, FAKE, None) == lib_mod.MOE_ERR_ARG
    assert "format" in lib_mod.last_error()
    assert qz(F8, 4, 60, FAKE, FAKE, FAKE, None) == lib_mod.MOE_ERR_ARG
    assert qz(MX, 4, 48, FAKE, FAKE, FAKE, None) == lib_mod.MOE_ERR_ARG
    assert "32" in lib_mod.last_error()
    assert qz(MX, 4, 64, FAKE, MISALIGNED, FAKE, None) == lib_mod.MOE_ERR_ARG
    assert dq(F8, 4, 24, FAKE, FAKE, FAKE, None) == lib_mod.MOE_ERR_ARG
    assert dq(MX, 4, 64, FAKE, None, FAKE, None) == lib_mod.MOE_ERR_ARG
    d = D()
    args = [FAKE] * 10
    assert ffn(ctypes.byref(d), F8, 0, *([None] * 10), 0, None) == lib_mod.MOE_OK
    assert ffn(ctypes.byref(d), 0, 4, *args, 1 << 40, None) == lib_mod.MOE_ERR_ARG
    assert ffn(ctypes.byref(d), MX, 4097, *args, 0, None) == lib_mod.MOE_ERR_WORKSPACE
    d32 = D(act=lib_mod.MOE_F32)
    assert ffn(ctypes.byref(d32), F8, 4, *args, 1 << 40, None) == lib_mod.MOE_ERR_UNSUPPORTED
    assert ffn(ctypes.byref(d), MX, 4, *args, 0, None) == lib_mod.MOE_ERR_WORKSPACE


def test_timed_gate_up_requires_both_events():
    d = D()
    for ev in ((None, FAKE), (FAKE, None), (None, None)):
        assert L.moe_expert_gate_up_timed(ctypes.byref(d), 4, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                          *ev) == lib_mod.MOE_ERR_ARG
        assert "event" in lib_mod.last_error()
    # argument checks of moe_expert_gate_up come first
    assert L.moe_expert_gate_up_timed(ctypes.byref(D(hidden=100)), 4, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, None, FAKE, FAKE) == lib_mod.MOE_ERR_UNSUPPORTED
    assert L.moe_expert_gate_up_timed(ctypes.byref(d), 4, MISALIGNED, FAKE, FAKE, FAKE, FAKE,
                                      None, FAKE, FAKE) == lib_mod.MOE_ERR_ARG


def test_noalloc_forward_validates_on_the_host():
    """moe_forward_noalloc: a no-op at 0 tokens, and the refusals (pointers,
    a workspace larger than the library's device array) come before any HIP
    call."""
    d = D(dense_inter=0)
    dp = ctypes.byref(d)
    f = L.moe_forward_noalloc
    assert f(dp, 0, None, None, None, None, None, None, None, None, None, None) == lib_mod.MOE_OK
    assert f(dp, 4, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
             None) == lib_mod.MOE_ERR_ARG
    assert f(dp, 4, MISALIGNED, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
             None) == lib_mod.MOE_ERR_ARG
    assert f(dp, 539, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
             None) == lib_mod.MOE_ERR_WORKSPACE
    assert "scratch" in lib_mod.last_error()
