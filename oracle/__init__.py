"""ctypes binding of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the package's smoke check and
the benchmark's CPU-baseline leg, never by the product path.

All functions take numpy arrays on the host.  bf16 tensors are passed as their
exactly widened fp32 values.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_P = ctypes.c_void_p
_I = ctypes.c_int


def build(verbose: bool = False) -> str:
    """Compile oracle.c with gcc: -O2, no fast-math, no FMA contraction, OpenMP.

    x86-64-v3 (AVX2 + FMA) keeps fmaf a single instruction and runs on any
    recent x86 server."""
    cmd = ["gcc", "-O2", "-march=x86-64-v3", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-o", _LIB + ".tmp", _SRC,
           "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        L.oracle_router.argtypes = [_I, _I, _I, _I, ctypes.c_float] + [_P] * 8
        L.oracle_router.restype = None
        L.oracle_dispatch.argtypes = [_I, _I, _I, _P, _P, _P, _P]
        L.oracle_dispatch.restype = None
        L.oracle_gelu_tanh.argtypes = [ctypes.c_double]
        L.oracle_gelu_tanh.restype = ctypes.c_double
        L.oracle_rmsnorm.argtypes = [_I, _I, ctypes.c_double, _P, _P, _P]
        L.oracle_rmsnorm.restype = None
        L.oracle_experts.argtypes = [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]
        L.oracle_experts.restype = None
        L.oracle_dense_mlp.argtypes = [_I, _I, _I, _P, _P, _P, _P, _P]
        L.oracle_dense_mlp.restype = None
        L.oracle_block.argtypes = ([_I] * 6 + [ctypes.c_float] + [_P] * 15 +
                                   [ctypes.c_double] + [_P] * 5)
        L.oracle_block.restype = None
        L.oracle_quantize_rows.argtypes = [ctypes.c_longlong, _I, _P, _P, _P]
        L.oracle_quantize_rows.restype = None
        L.oracle_dequantize_rows.argtypes = [ctypes.c_longlong, _I, _P, _P, _P]
        L.oracle_dequantize_rows.restype = None
        for name in ("oracle_quantize_fp8_rows", "oracle_dequantize_fp8_rows",
                     "oracle_quantize_mxfp4_rows", "oracle_dequantize_mxfp4_rows"):
            getattr(L, name).argtypes = [ctypes.c_longlong, _I, _P, _P, _P]
            getattr(L, name).restype = None
        L.oracle_quantize_mx8_rows.argtypes = [ctypes.c_longlong, _I, _P, _P, _P]
        L.oracle_quantize_mx8_rows.restype = None
        L.oracle_dequantize_mx8_rows.argtypes = [ctypes.c_longlong, _I, _P, _P, _P]
        L.oracle_dequantize_mx8_rows.restype = None
        L.oracle_experts_mx8.argtypes = [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]
        L.oracle_experts_mx8.restype = None
        L.oracle_e4m3_value.argtypes = [_I]
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_e2m1_value.argtypes = [_I]
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = _I
        L.oracle_set_num_threads.argtypes = [_I]
        L.oracle_set_num_threads.restype = None
        _lib = L
    return _lib


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of later oracle calls (timing only: results do not depend on it)."""
    lib().oracle_set_num_threads(int(n))


def router(x, router_w, router_scale, per_expert_scale, K, eps=1e-6, pre_gain=None,
           want_logits=False):
    """fp32 router: returns (idx [T,K] int32, w [T,K] fp32[, logits [T,E] fp32])."""
    x = _f32(x)
    T, H = x.shape
    rw = _f32(router_w)
    E = rw.shape[0]
    rs, pes = _f32(router_scale), _f32(per_expert_scale)
    pg = None if pre_gain is None else _f32(pre_gain)
    idx = np.zeros((T, K), np.int32)
    w = np.zeros((T, K), np.float32)
    logits = np.zeros((T, E), np.float32) if want_logits else None
    lib().oracle_router(T, H, E, K, eps, _p(x), _p(pg), _p(rw), _p(rs), _p(pes), _p(idx),
                        _p(w), _p(logits))
    return (idx, w, logits) if want_logits else (idx, w)


def dispatch(idx, E):
    """Returns (counts [E], offsets [E+1], sorted_slots [T*K]) as int32."""
    idx = _i32(idx)
    T, K = idx.shape
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    ss = np.zeros(T * K, np.int32)
    lib().oracle_dispatch(T, E, K, _p(idx), _p(counts), _p(offsets), _p(ss))
    return counts, offsets, ss


def gelu_tanh(z: float) -> float:
    return lib().oracle_gelu_tanh(float(z))


def rmsnorm(x, gain=None, eps=1e-6):
    x = _f64(x)
    T, H = x.shape
    g = None if gain is None else _f32(gain)
    out = np.zeros((T, H), np.float64)
    lib().oracle_rmsnorm(T, H, eps, _p(x), _p(g), _p(out))
    return out


def experts(xin, gate_up, down, idx, w):
    """Sparse expert loop in fp64: returns out [T,H] fp64."""
    xin = _f64(xin)
    T, H = xin.shape
    gu, dn = _f32(gate_up), _f32(down)
    E, I2, _ = gu.shape
    idx, w = _i32(idx), _f32(w)
    K = idx.shape[1]
    out = np.zeros((T, H), np.float64)
    lib().oracle_experts(T, H, E, K, I2 // 2, _p(xin), _p(gu), _p(dn), _p(idx), _p(w),
                         _p(out))
    return out


def dense_mlp(xin, wg, wu, wd):
    xin = _f64(xin)
    T, H = xin.shape
    wg, wu, wd = _f32(wg), _f32(wu), _f32(wd)
    D = wg.shape[0]
    out = np.zeros((T, H), np.float64)
    lib().oracle_dense_mlp(T, H, D, _p(xin), _p(wg), _p(wu), _p(wd), _p(out))
    return out


def block(x, g_pre, g_pre2, g_post1, g_post2, g_post, dense_gate, dense_up, dense_down,
          router_w, router_scale, per_expert_scale, gate_up, down, layer_scalar, K,
          eps=1e-6):
    """One dual-path layer; returns dict(out, o, moe, idx, w)."""
    x32 = _f32(x)
    x64 = _f64(x32)
    T, H = x32.shape
    gu, dn = _f32(gate_up), _f32(down)
    E, I2, _ = gu.shape
    D = np.asarray(dense_gate).shape[0]
    idx = np.zeros((T, K), np.int32)
    w = np.zeros((T, K), np.float32)
    out = np.zeros((T, H), np.float64)
    o = np.zeros((T, H), np.float64)
    moe = np.zeros((T, H), np.float64)
    args = [_f32(a) for a in (g_pre, g_pre2, g_post1, g_post2, g_post, dense_gate, dense_up,
                              dense_down, router_w, router_scale, per_expert_scale)]
    lib().oracle_block(T, H, E, K, I2 // 2, D, eps, _p(x32), _p(x64), *[_p(a) for a in args],
                       _p(gu), _p(dn), float(layer_scalar), _p(idx), _p(w), _p(out), _p(o),
                       _p(moe))
    return {"out": out, "o": o, "moe": moe, "idx": idx, "w": w}


def quantize_int8(w):
    """Per-row symmetric int8: returns (q int8 same shape, s fp32 [rows...]).
    The last axis is the channel's input dimension."""
    w = _f32(w)
    shape = w.shape
    rows = int(np.prod(shape[:-1]))
    q = np.zeros(shape, np.int8)
    s = np.zeros(shape[:-1], np.float32)
    lib().oracle_quantize_rows(rows, shape[-1], _p(w), _p(q), _p(s))
    return q, s


def dequantize_int8(q, s):
    """q * s rounded once to fp32, shape of q."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = _f32(s)
    out = np.zeros(q.shape, np.float32)
    lib().oracle_dequantize_rows(int(np.prod(q.shape[:-1])), q.shape[-1], _p(q), _p(s), _p(out))
    return out


def experts_int8(xin, gate_up_q, gate_up_s, down_q, down_s, idx, w):
    """The sparse expert loop (fp64) on the dequantized int8 weights."""
    return experts(xin, dequantize_int8(gate_up_q, gate_up_s), dequantize_int8(down_q, down_s),
                   idx, w)


def e4m3_value(code: int) -> float:
    """Value of an E4M3 code (OCP 8-bit floating point; NaN for S.1111.111)."""
    return lib().oracle_e4m3_value(int(code))


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code."""
    return lib().oracle_e2m1_value(int(code))


def quantize_fp8(w):
    """Per-row symmetric E4M3: returns (codes uint8 same shape, s fp32 [rows...])."""
    w = _f32(w)
    shape = w.shape
    q = np.zeros(shape, np.uint8)
    s = np.zeros(shape[:-1], np.float32)
    lib().oracle_quantize_fp8_rows(int(np.prod(shape[:-1])), shape[-1], _p(w), _p(q), _p(s))
    return q, s


def dequantize_fp8(q, s):
    """value(code) * s rounded once to fp32, shape of q."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = _f32(s)
    out = np.zeros(q.shape, np.float32)
    lib().oracle_dequantize_fp8_rows(int(np.prod(q.shape[:-1])), q.shape[-1], _p(q), _p(s),
                                     _p(out))
    return out


def quantize_mxfp4(w):
    """MXFP4 along the last axis (a multiple of 32): returns (codes uint8 [..., n/2],
    two E2M1 codes per byte, the even column in the low nibble; E8M0 scale codes
    uint8 [..., n/32])."""
    w = _f32(w)
    shape = w.shape
    n = shape[-1]
    assert n % 32 == 0
    q = np.zeros(shape[:-1] + (n // 2,), np.uint8)
    e8 = np.zeros(shape[:-1] + (n // 32,), np.uint8)
    lib().oracle_quantize_mxfp4_rows(int(np.prod(shape[:-1])), n, _p(w), _p(q), _p(e8))
    return q, e8


def dequantize_mxfp4(q, e8):
    """value(code) * 2^(e8 - 127), exact; shape [..., 2 * q.shape[-1]]."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    e8 = np.ascontiguousarray(e8, dtype=np.uint8)
    n = 2 * q.shape[-1]
    out = np.zeros(q.shape[:-1] + (n,), np.float32)
    lib().oracle_dequantize_mxfp4_rows(int(np.prod(q.shape[:-1])), n, _p(q), _p(e8), _p(out))
    return out


def experts_fp8(xin, gate_up_q, gate_up_s, down_q, down_s, idx, w):
    """The sparse expert loop (fp64) on the dequantized E4M3 weights."""
    return experts(xin, dequantize_fp8(gate_up_q, gate_up_s), dequantize_fp8(down_q, down_s),
                   idx, w)


def experts_mxfp4(xin, gate_up_q, gate_up_e8, down_q, down_e8, idx, w):
    """The sparse expert loop (fp64) on the dequantized MXFP4 weights."""
    return experts(xin, dequantize_mxfp4(gate_up_q, gate_up_e8),
                   dequantize_mxfp4(down_q, down_e8), idx, w)


def quantize_mx8(v):
    """MXFP8 along the last axis (a multiple of 32): returns (E4M3 codes uint8,
    same shape; E8M0 scale codes uint8 [..., n/32])."""
    v = _f64(v)
    shape = v.shape
    n = shape[-1]
    assert n % 32 == 0
    q = np.zeros(shape, np.uint8)
    e8 = np.zeros(shape[:-1] + (n // 32,), np.uint8)
    lib().oracle_quantize_mx8_rows(int(np.prod(shape[:-1])), n, _p(v), _p(q), _p(e8))
    return q, e8


def dequantize_mx8(q, e8):
    """value(code) * 2^(e8 - 127), exact (fp64)."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    e8 = np.ascontiguousarray(e8, dtype=np.uint8)
    out = np.zeros(q.shape, np.float64)
    lib().oracle_dequantize_mx8_rows(int(np.prod(q.shape[:-1])), q.shape[-1], _p(q), _p(e8),
                                     _p(out))
    return out


def experts_mx8(xin, gate_up, down, idx, w):
    """The sparse expert loop (fp64) with MXFP8 activations: the input row and
    the gated product are each replaced by their MXFP8 value before their
    projections; gate_up / down are weight values.  Returns [T,H] fp64."""
    x = _f64(xin)
    T, H = x.shape
    gu, dn = _f32(gate_up), _f32(down)
    E, I2, _ = gu.shape
    idx = _i32(idx)
    K = idx.shape[1]
    w = _f32(w)
    out = np.zeros((T, H), np.float64)
    lib().oracle_experts_mx8(T, H, E, K, I2 // 2, _p(x), _p(gu), _p(dn), _p(idx), _p(w), _p(out))
    return out


def experts_fp8_mx8(xin, gate_up_q, gate_up_s, down_q, down_s, idx, w):
    """E4M3 per-channel weights with MXFP8 activations (fp64 loop)."""
    return experts_mx8(xin, dequantize_fp8(gate_up_q, gate_up_s),
                       dequantize_fp8(down_q, down_s), idx, w)


def experts_mxfp4_mx8(xin, gate_up_q, gate_up_e8, down_q, down_e8, idx, w):
    """MXFP4 weights with MXFP8 activations (fp64 loop)."""
    return experts_mx8(xin, dequantize_mxfp4(gate_up_q, gate_up_e8),
                       dequantize_mxfp4(down_q, down_e8), idx, w)
