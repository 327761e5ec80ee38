"""Helpers for the GPU parity tests: moving synthetic tensors to the device and
comparing against the oracle.  Imported only by tests marked `gpu`."""
from __future__ import annotations

import sys

import numpy as np
import torch

from sparse_moe_transformer_router_amd import synth


def note(msg: str):
    """Print what the next GPU step is about to run (visible even if the run dies)."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def dev_tensor(t: synth.Tensor, bf16: bool, device="cuda") -> torch.Tensor:
    if bf16:
        assert t.bf16 is not None
        return torch.from_numpy(np.ascontiguousarray(t.bf16).view(np.int16)).to(device).view(
            torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(t.f32)).to(device)


def dev_f32(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def rel_max_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / RMS(ref) over the whole tensor."""
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref))) / max(rms, 1e-30)


BF16_TOL = 2e-2     # max|err| <= 2e-2 * RMS(ref) for the bf16 path
F32_TOL = 1e-4      # max|err| <= 1e-4 * RMS(ref) for the fp32 path


def ws_logits_view(ws: torch.Tensor, T: int, E: int) -> torch.Tensor:
    """The router's fp32 logits inside the workspace (third region: after two
    256-byte-aligned [T] fp32 arrays)."""
    a = lambda n: (n + 255) // 256 * 256  # noqa: E731
    off = 2 * a(4 * T)
    return ws[off: off + 4 * T * E].view(torch.float32).view(T, E)


def bf16_path_bound(x, gate_up, down, idx, w, bf16_slots=False, out_rounded=True):
    """Per-element error bound of the bf16 expert path against the exact result.

    The bf16 path rounds twice: h = gelu(gate) * up is rounded to bf16 before
    the down projection, and the combined output is rounded to bf16.  A bf16
    round-to-nearest moves a value v by at most 2^-8 |v| (8 significant bits),
    so |gpu - exact| <= 2^-8 |out| + sum_k |w_k| (|W_d[e_k]| @ |h_k|) 2^-8, plus
    fp32 accumulation error (taken as 1e-5 of the summed magnitudes).  Inputs
    are the exactly widened bf16 values.  With bf16_slots the K per-slot
    outputs are also rounded to bf16 before their sum, which adds at most
    2^-8 |w_k y_k| <= 2^-8 |w_k| (|W_d[e_k]| @ |h_k|) per slot.  With
    out_rounded=False the result is taken before its final rounding (an fp32
    slot output or an fp32 sum of slots), which drops the 2^-8 |out| term.
    Returns (bound [T,H], exact [T,H])."""
    x = np.asarray(x, np.float64)
    T, H = x.shape
    E, I2, _ = gate_up.shape
    I = I2 // 2
    idx = np.asarray(idx)
    w = np.asarray(w, np.float64)
    exact = np.zeros((T, H))
    hterm = np.zeros((T, H))
    # the (token, slot) pairs of each expert at once; a token picks an expert
    # at most once, so the rows of tt are distinct
    for e in range(E):
        tt, kk = np.nonzero(idx == e)
        if len(tt) == 0:
            continue
        gu = x[tt] @ gate_up[e].astype(np.float64).T
        g, u = gu[:, :I], gu[:, I:]
        hh = 0.5 * g * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (g + 0.044715 * g ** 3))) * u
        wd = down[e].astype(np.float64)
        wk = w[tt, kk][:, None]
        exact[tt] += wk * (hh @ wd.T)
        hterm[tt] += np.abs(wk) * (np.abs(hh) @ np.abs(wd).T)
    mag = hterm
    bound = (2.0 ** -8 * np.abs(exact) * 1.001 if out_rounded else 0.0) + \
        2.0 ** -8 * hterm + 1e-5 * mag
    if bf16_slots:
        bound += 2.0 ** -8 * hterm * 1.001
    return bound, exact


# Accumulation error of gfx950's scaled 8-bit / 4-bit matrix instruction,
# relative to the sum of the magnitudes of the products it adds: an
# in-bounds check of the instruction on random E4M3 / E2M1 operands with
# random block scales, against an exact host evaluation, found at most
# 1.5e-4 (median 2e-5) with an 8-bit operand; 2^-12 = 2.4e-4 covers it.
MX_ACC_REL = 2.0 ** -12


def _mx8_on_scale(v, shared):
    """E4M3 value (torch float8_e4m3fn rounding, +-448 saturation) of v on
    the grid 2^shared (shared broadcast per element), times 2^shared."""
    s = np.clip(v / 2.0 ** shared, -448, 448)
    r = torch.tensor(s, dtype=torch.float32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    return r * 2.0 ** shared


def mx_path_bound(x, gate_up, down, idx, w, acc_rel=MX_ACC_REL):
    """Per-element bound of the 8-bit / 4-bit expert path against the
    oracle's expert loop with MXFP8 activations (oracle.experts_mx8), on the
    weights' values gate_up / down.

    The input's MXFP8 codes are the same on both sides (bit-exact quantizer),
    so the path differs from the oracle only by (i) the matrix instruction's
    accumulation, at most acc_rel of the summed product magnitudes, in the
    gate / up sums, in the down sums and (ii) through (i), the MXFP8 codes of
    h: an element within its error interval of an E4M3 decision point may
    take the neighbouring code, and a block whose maximum lies within its
    interval of a power of two may take the neighbouring scale.  Each
    element of h may so move by d = the largest distance, over both ends of
    its interval and the candidate scales, between its MXFP8 value and the
    oracle's; y then moves by at most |w| (|W_d| @ d).  Plus the output's
    bf16 rounding (2^-8 |out|) and fp32 rounding.  Returns (bound, exact)."""
    import oracle
    x = np.asarray(x, np.float64)
    T, H = x.shape
    E, I2, _ = gate_up.shape
    I = I2 // 2
    xq = oracle.dequantize_mx8(*oracle.quantize_mx8(x))
    idx = np.asarray(idx)
    w = np.asarray(w, np.float64)
    exact = np.zeros((T, H))
    err = np.zeros((T, H))
    c0 = np.sqrt(2.0 / np.pi)
    for e in range(E):
        tt, kk = np.nonzero(idx == e)
        if len(tt) == 0:
            continue
        wg = gate_up[e, :I].astype(np.float64)
        wu = gate_up[e, I:].astype(np.float64)
        wd = down[e].astype(np.float64)
        a = xq[tt]
        g, u = a @ wg.T, a @ wu.T
        gerr = acc_rel * (np.abs(a) @ np.abs(wg).T) + 2.0 ** -23 * np.abs(g)
        uerr = acc_rel * (np.abs(a) @ np.abs(wu).T) + 2.0 ** -23 * np.abs(u)
        th = np.tanh(c0 * (g + 0.044715 * g ** 3))
        gel = 0.5 * g * (1.0 + th)
        h = gel * u
        # |gelu'| <= 1.13 everywhere; fp32 evaluation of gelu and the product
        herr = 1.13 * gerr * (np.abs(u) + uerr) + np.abs(gel) * uerr + 1e-6 * np.abs(h)
        hq, he8 = oracle.quantize_mx8(h)
        q = oracle.dequantize_mx8(hq, he8)
        shared = np.repeat(he8.astype(np.int64) - 127, 32, axis=1)
        d = np.zeros_like(h)
        for s_shift in (0, -1, 1):
            if s_shift != 0:
                # blocks whose maximum's interval reaches across a power of two
                bmax = np.abs(h).reshape(len(tt), -1, 32)
                berr = herr.reshape(len(tt), -1, 32)
                lo = np.max(np.maximum(bmax - berr, 0.0), -1)
                hi = np.max(bmax + berr, -1)
                sh = he8.astype(np.int64) - 127 - 8
                if s_shift > 0:
                    cand = hi >= 2.0 ** (sh + 9)
                else:
                    cand = lo < 2.0 ** (sh + 8)
                mask = np.repeat(cand & (he8 > 0), 32, axis=1)
                if not mask.any():
                    continue
            else:
                mask = np.ones_like(h, dtype=bool)
            for v in (h - herr, h + herr):
                qv = _mx8_on_scale(v, shared + s_shift)
                d = np.maximum(d, np.where(mask, np.abs(qv - q), 0.0))
        wk = w[tt, kk][:, None]
        exact[tt] += wk * (q @ wd.T)
        err[tt] += np.abs(wk) * (d @ np.abs(wd).T + acc_rel * (np.abs(q) @ np.abs(wd).T))
    bound = 2.0 ** -8 * np.abs(exact) * 1.001 + err * 1.001 + 1e-6 * np.abs(exact)
    return bound, exact
