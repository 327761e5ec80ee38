"""Python binding of libmoe (include/moe.h): argument marshalling only.

Every function takes torch tensors that live on the GPU and passes their
device pointers and sizes to the C ABI; all arithmetic runs in the library's
HIP kernels.  torch supplies the memory and the stream (the current stream
unless one is given).  If libmoe.so has not been built, importing this module
raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16 = 0, 1
MOE_W_INT8, MOE_W_FP8, MOE_W_MXFP4, MOE_W_MXFP8 = 1, 2, 3, 4
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20   # the no-allocation entry point's device array


class MoeDims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("expert_inter", ctypes.c_int32),
                ("dense_inter", ctypes.c_int32), ("eps", ctypes.c_float),
                ("act_dtype", ctypes.c_int32), ("slot_dtype", ctypes.c_int32)]


class Gemma4FfnWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "g_pre", "g_pre2", "g_post1", "g_post2", "g_post", "dense_gate", "dense_up",
        "dense_down", "router_w", "router_scale", "per_expert_scale", "w_gate_up", "w_down")] + \
        [("layer_scalar", ctypes.c_float)]


class Gemma4FfnWeightsQ(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32)] + [(n, ctypes.c_void_p) for n in (
        "g_pre", "g_pre2", "g_post1", "g_post2", "g_post", "dense_gate_q", "dense_gate_scale",
        "dense_up_q", "dense_up_scale", "dense_down_q", "dense_down_scale", "router_w",
        "router_scale", "per_expert_scale", "gate_up_q", "gate_up_scale", "down_q",
        "down_scale")] + [("layer_scalar", ctypes.c_float)]


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libmoe error {code}: {msg}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m sparse_moe_transformer_router_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    D = ctypes.POINTER(MoeDims)
    L.moe_workspace_size.argtypes = [D, I32]
    L.moe_workspace_size.restype = SZ
    L.moe_last_error.argtypes = []
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_router.argtypes = [D, I32] + [P] * 8 + [SZ, P]
    L.moe_route.argtypes = [D, I32] + [P] * 11 + [SZ, P]
    L.moe_dispatch.argtypes = [D, I32] + [P] * 5 + [SZ, P]
    L.moe_expert_ffn.argtypes = [D, I32] + [P] * 8 + [SZ, P]
    L.moe_dense_mask_dispatch.argtypes = [D, I32] + [P] * 6
    L.moe_expert_gate_up.argtypes = [D, I32] + [P] * 6
    L.moe_expert_gate_up_timed.argtypes = [D, I32] + [P] * 8
    L.moe_expert_down.argtypes = [D, I32] + [P] * 7
    L.moe_combine.argtypes = [D, I32, P, P, P, P]
    L.moe_forward.argtypes = [D, I32] + [P] * 10 + [SZ, P]
    L.moe_forward_noalloc.argtypes = [D, I32] + [P] * 10
    L.moe_expert_ffn_mx.argtypes = [D, I32, I32] + [P] * 10 + [SZ, P]
    L.moe_quantize_int8.argtypes = [ctypes.c_int64, I32, P, P, P, P]
    L.moe_expert_ffn_int8.argtypes = [D, I32] + [P] * 10 + [SZ, P]
    L.moe_quantize.argtypes = [I32, ctypes.c_int64, I32, P, P, P, P]
    L.moe_dequantize.argtypes = [I32, ctypes.c_int64, I32, P, P, P, P]
    L.moe_expert_ffn_q.argtypes = [D, I32, I32] + [P] * 10 + [SZ, P]
    L.gemma4_ffn_block.argtypes = [D, I32, P, ctypes.POINTER(Gemma4FfnWeights)] + [P] * 5 + \
        [SZ, P]
    L.gemma4_ffn_block_q.argtypes = [D, I32, P, ctypes.POINTER(Gemma4FfnWeightsQ)] + [P] * 5 + \
        [SZ, P]
    for f in ("moe_router", "moe_route", "moe_dispatch", "moe_expert_ffn", "moe_expert_gate_up",
              "moe_expert_down", "moe_combine", "moe_forward", "gemma4_ffn_block",
              "moe_quantize_int8", "moe_expert_ffn_int8", "moe_dense_mask_dispatch",
              "moe_quantize", "moe_dequantize", "moe_expert_ffn_q", "moe_expert_gate_up_timed",
              "gemma4_ffn_block_q", "moe_forward_noalloc", "moe_expert_ffn_mx"):
        getattr(L, f).restype = ctypes.c_int
    return L


_lib = _load()


def raw():
    """The ctypes library object (for tests of the exported symbols)."""
    return _lib


def dims(hidden, num_experts, top_k, expert_inter, dense_inter=0, eps=1e-6, act=MOE_BF16,
         slot=MOE_F32) -> MoeDims:
    """Layer dimensions.  The per-slot expert outputs default to fp32: rounding
    them to bf16 adds a third rounding stage to the bf16 path."""
    return MoeDims(hidden, num_experts, top_k, expert_inter, dense_inter, eps, act, slot)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(rc: int):
    if rc != MOE_OK:
        raise MoeError(rc, _lib.moe_last_error().decode())


def last_error() -> str:
    return _lib.moe_last_error().decode()


def workspace_size(d: MoeDims, max_tokens: int) -> int:
    n = _lib.moe_workspace_size(ctypes.byref(d), max_tokens)
    if n == 0:
        raise MoeError(MOE_ERR_UNSUPPORTED, last_error())
    return n


def workspace(d: MoeDims, max_tokens: int, device="cuda") -> torch.Tensor:
    """A uint8 device buffer of moe_workspace_size bytes (256-byte aligned)."""
    return torch.empty(workspace_size(d, max_tokens), dtype=torch.uint8, device=device)


def moe_router(d, T, x, router_w, router_scale, per_expert_scale, pre_norm_gain, topk_idx,
               topk_w, ws, stream=None):
    _check(_lib.moe_router(ctypes.byref(d), T, _ptr(x), _ptr(router_w), _ptr(router_scale),
                           _ptr(per_expert_scale), _ptr(pre_norm_gain), _ptr(topk_idx),
                           _ptr(topk_w), _ptr(ws), ws.numel() if ws is not None else 0,
                           _stream(stream)))


def moe_route(d, T, x, router_w, router_scale, per_expert_scale, pre_norm_gain, topk_idx, topk_w,
              counts, offsets, sorted_slots, ws, stream=None):
    _check(_lib.moe_route(ctypes.byref(d), T, _ptr(x), _ptr(router_w), _ptr(router_scale),
                          _ptr(per_expert_scale), _ptr(pre_norm_gain), _ptr(topk_idx),
                          _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(sorted_slots), _ptr(ws),
                          ws.numel() if ws is not None else 0, _stream(stream)))


def moe_dispatch(d, T, topk_idx, counts, offsets, sorted_slots, ws, stream=None):
    _check(_lib.moe_dispatch(ctypes.byref(d), T, _ptr(topk_idx), _ptr(counts), _ptr(offsets),
                             _ptr(sorted_slots), _ptr(ws), ws.numel() if ws is not None else 0,
                             _stream(stream)))


def moe_dense_mask_dispatch(d, T, topk_idx, topk_w, offsets, sorted_slots, w_dense, stream=None):
    _check(_lib.moe_dense_mask_dispatch(ctypes.byref(d), T, _ptr(topk_idx), _ptr(topk_w),
                                        _ptr(offsets), _ptr(sorted_slots), _ptr(w_dense),
                                        _stream(stream)))


def moe_expert_ffn(d, T, x, w_gate_up, w_down, topk_w, offsets, sorted_slots, y_slots, ws,
                   stream=None):
    _check(_lib.moe_expert_ffn(ctypes.byref(d), T, _ptr(x), _ptr(w_gate_up), _ptr(w_down),
                               _ptr(topk_w), _ptr(offsets), _ptr(sorted_slots), _ptr(y_slots),
                               _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))


def moe_quantize_int8(w, q, scale, stream=None):
    """Per-row symmetric int8 codes and scales of a bf16 weight whose last axis
    is the row (input) dimension."""
    cols = w.shape[-1]
    rows = w.numel() // cols if cols else 0
    _check(_lib.moe_quantize_int8(rows, cols, _ptr(w), _ptr(q), _ptr(scale), _stream(stream)))


def moe_expert_ffn_int8(d, T, x, w_gate_up_q, w_gate_up_scale, w_down_q, w_down_scale, topk_w,
                        offsets, sorted_slots, y_slots, ws, stream=None):
    _check(_lib.moe_expert_ffn_int8(ctypes.byref(d), T, _ptr(x), _ptr(w_gate_up_q),
                                    _ptr(w_gate_up_scale), _ptr(w_down_q), _ptr(w_down_scale),
                                    _ptr(topk_w), _ptr(offsets), _ptr(sorted_slots),
                                    _ptr(y_slots), _ptr(ws), ws.numel() if ws is not None else 0,
                                    _stream(stream)))


def moe_quantize(fmt, w, q, scale, stream=None):
    """Codes and scales of a bf16 weight whose last axis is the row (input)
    dimension, in format fmt (MOE_W_INT8, MOE_W_FP8 or MOE_W_MXFP4)."""
    cols = w.shape[-1]
    rows = w.numel() // cols if cols else 0
    _check(_lib.moe_quantize(fmt, rows, cols, _ptr(w), _ptr(q), _ptr(scale), _stream(stream)))


def moe_dequantize(fmt, rows, cols, q, scale, out, stream=None):
    _check(_lib.moe_dequantize(fmt, rows, cols, _ptr(q), _ptr(scale), _ptr(out),
                               _stream(stream)))


def moe_expert_ffn_q(d, fmt, T, x, w_gate_up_q, w_gate_up_scale, w_down_q, w_down_scale, topk_w,
                     offsets, sorted_slots, y_slots, ws, stream=None):
    _check(_lib.moe_expert_ffn_q(ctypes.byref(d), fmt, T, _ptr(x), _ptr(w_gate_up_q),
                                 _ptr(w_gate_up_scale), _ptr(w_down_q), _ptr(w_down_scale),
                                 _ptr(topk_w), _ptr(offsets), _ptr(sorted_slots),
                                 _ptr(y_slots), _ptr(ws), ws.numel() if ws is not None else 0,
                                 _stream(stream)))


def moe_expert_ffn_mx(d, fmt, T, x, w_gate_up_q, w_gate_up_scale, w_down_q, w_down_scale,
                      topk_w, offsets, sorted_slots, y_slots, ws, stream=None):
    """E4M3 / MXFP4 experts on the 8-bit / 4-bit matrix instructions, MXFP8
    activations."""
    _check(_lib.moe_expert_ffn_mx(ctypes.byref(d), fmt, T, _ptr(x), _ptr(w_gate_up_q),
                                  _ptr(w_gate_up_scale), _ptr(w_down_q), _ptr(w_down_scale),
                                  _ptr(topk_w), _ptr(offsets), _ptr(sorted_slots),
                                  _ptr(y_slots), _ptr(ws), ws.numel() if ws is not None else 0,
                                  _stream(stream)))


def moe_expert_gate_up(d, T, x, w_gate_up, offsets, sorted_slots, h, stream=None):
    _check(_lib.moe_expert_gate_up(ctypes.byref(d), T, _ptr(x), _ptr(w_gate_up), _ptr(offsets),
                                   _ptr(sorted_slots), _ptr(h), _stream(stream)))


def moe_expert_gate_up_timed(d, T, x, w_gate_up, offsets, sorted_slots, h, start, stop,
                             stream=None):
    """moe_expert_gate_up recording torch.cuda.Event start / stop on the
    kernel's own dispatch; both events must have been recorded once before
    (torch creates its events at their first record)."""
    hs, he = start.cuda_event, stop.cuda_event
    if not hs or not he:
        raise RuntimeError("moe_expert_gate_up_timed: record both events once before use")
    _check(_lib.moe_expert_gate_up_timed(ctypes.byref(d), T, _ptr(x), _ptr(w_gate_up),
                                         _ptr(offsets), _ptr(sorted_slots), _ptr(h),
                                         _stream(stream), ctypes.c_void_p(hs),
                                         ctypes.c_void_p(he)))


def moe_expert_down(d, T, h, w_down, topk_w, offsets, sorted_slots, y_slots, stream=None):
    _check(_lib.moe_expert_down(ctypes.byref(d), T, _ptr(h), _ptr(w_down), _ptr(topk_w),
                                _ptr(offsets), _ptr(sorted_slots), _ptr(y_slots),
                                _stream(stream)))


def moe_combine(d, T, y_slots, addend, out, stream=None):
    _check(_lib.moe_combine(ctypes.byref(d), T, _ptr(y_slots), _ptr(addend), _ptr(out),
                            _stream(stream)))


def moe_forward(d, T, x, router_w, router_scale, per_expert_scale, w_gate_up, w_down, out,
                topk_idx, topk_w, ws, stream=None):
    _check(_lib.moe_forward(ctypes.byref(d), T, _ptr(x), _ptr(router_w), _ptr(router_scale),
                            _ptr(per_expert_scale), _ptr(w_gate_up), _ptr(w_down), _ptr(out),
                            _ptr(topk_idx), _ptr(topk_w), _ptr(ws),
                            ws.numel() if ws is not None else 0, _stream(stream)))


def moe_forward_noalloc(d, T, x, router_w, router_scale, per_expert_scale, w_gate_up, w_down,
                        out, topk_idx, topk_w, stream=None):
    """moe_forward with the library's own device scratch array as workspace."""
    _check(_lib.moe_forward_noalloc(ctypes.byref(d), T, _ptr(x), _ptr(router_w),
                                    _ptr(router_scale), _ptr(per_expert_scale), _ptr(w_gate_up),
                                    _ptr(w_down), _ptr(out), _ptr(topk_idx), _ptr(topk_w),
                                    _stream(stream)))


def ffn_weights(g_pre, g_pre2, g_post1, g_post2, g_post, dense_gate, dense_up, dense_down,
                router_w, router_scale, per_expert_scale, w_gate_up, w_down,
                layer_scalar) -> Gemma4FfnWeights:
    ts = (g_pre, g_pre2, g_post1, g_post2, g_post, dense_gate, dense_up, dense_down, router_w,
          router_scale, per_expert_scale, w_gate_up, w_down)
    return Gemma4FfnWeights(*[_ptr(t) for t in ts], float(layer_scalar))


def ffn_weights_q(fmt, g_pre, g_pre2, g_post1, g_post2, g_post, dense_gate_q, dense_gate_scale,
                  dense_up_q, dense_up_scale, dense_down_q, dense_down_scale, router_w,
                  router_scale, per_expert_scale, gate_up_q, gate_up_scale, down_q, down_scale,
                  layer_scalar) -> Gemma4FfnWeightsQ:
    ts = (g_pre, g_pre2, g_post1, g_post2, g_post, dense_gate_q, dense_gate_scale, dense_up_q,
          dense_up_scale, dense_down_q, dense_down_scale, router_w, router_scale,
          per_expert_scale, gate_up_q, gate_up_scale, down_q, down_scale)
    return Gemma4FfnWeightsQ(int(fmt), *[_ptr(t) for t in ts], float(layer_scalar))


def gemma4_ffn_block_q(d, T, residual, weights: Gemma4FfnWeightsQ, out, ffn_out, topk_idx,
                       topk_w, ws, stream=None):
    _check(_lib.gemma4_ffn_block_q(ctypes.byref(d), T, _ptr(residual), ctypes.byref(weights),
                                   _ptr(out), _ptr(ffn_out), _ptr(topk_idx), _ptr(topk_w),
                                   _ptr(ws), ws.numel() if ws is not None else 0,
                                   _stream(stream)))


def gemma4_ffn_block(d, T, residual, weights: Gemma4FfnWeights, out, ffn_out, topk_idx, topk_w,
                     ws, stream=None):
    _check(_lib.gemma4_ffn_block(ctypes.byref(d), T, _ptr(residual), ctypes.byref(weights),
                                 _ptr(out), _ptr(ffn_out), _ptr(topk_idx), _ptr(topk_w),
                                 _ptr(ws), ws.numel() if ws is not None else 0,
                                 _stream(stream)))
