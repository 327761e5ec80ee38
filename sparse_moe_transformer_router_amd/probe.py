"""Python binding of the measurement probes (include/moe_probe.h): argument
marshalling only.  Importing it raises if libmoe_probe.so is missing."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_probe.so")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m sparse_moe_transformer_router_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    L.moe_probe_read_blocks.argtypes = []
    L.moe_probe_read_blocks.restype = ctypes.c_int
    L.moe_probe_stream_read.argtypes = [P, ctypes.c_longlong, P, P]
    L.moe_probe_stream_read.restype = ctypes.c_int
    L.moe_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    L.moe_probe_mfma_flops.restype = ctypes.c_longlong
    L.moe_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, P, P]
    L.moe_probe_mfma.restype = ctypes.c_int
    return L


_lib = _load()


def raw():
    return _lib


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def read_blocks() -> int:
    return _lib.moe_probe_read_blocks()


def stream_read(buf, block_xor, stream=None) -> None:
    """buf: a contiguous device tensor; block_xor: int32 device tensor of
    read_blocks() entries."""
    rc = _lib.moe_probe_stream_read(ctypes.c_void_p(buf.data_ptr()),
                                    buf.numel() * buf.element_size(),
                                    ctypes.c_void_p(block_xor.data_ptr()), _stream(stream))
    if rc != 0:
        raise RuntimeError(f"moe_probe_stream_read failed ({rc})")


def mfma_flops(blocks: int, iters: int) -> int:
    return _lib.moe_probe_mfma_flops(blocks, iters)


def mfma(blocks: int, iters: int, out, stream=None) -> None:
    """out: fp32 device tensor of blocks * 4 entries."""
    rc = _lib.moe_probe_mfma(blocks, iters, ctypes.c_void_p(out.data_ptr()), _stream(stream))
    if rc != 0:
        raise RuntimeError(f"moe_probe_mfma failed ({rc})")
