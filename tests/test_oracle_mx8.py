"""Pins of the oracle's MXFP8 activation reading (E4M3 elements, one E8M0
scale per 32 consecutive values along the contraction, shared exponent
floor(log2 max|v|) - 8) and of the expert loop that feeds MXFP8 activations
to the 8-bit / 4-bit matrix products: hand-worked blocks with exact ties,
subnormals, saturation and exact powers of two; torch's float8_e4m3fn
rounding; the error bound; symmetry, power-of-two scaling and the lossless
case; the expert loop against a composition of torch routines."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _block(vals):
    v = np.zeros(32)
    v[:len(vals)] = vals
    return v


def test_hand_block_codes():
    """amax 1.0 -> shared -8 (E8M0 code 119); elements x 256 on the E4M3 grid."""
    v = _block([1.0, -1.0, 0.5, 136 / 256, 152 / 256, 2.0 ** -9 / 256, 1.5 * 2.0 ** -9 / 256,
                2.5 * 2.0 ** -9 / 256, 0.0, -0.75])
    q, e8 = oracle.quantize_mx8(v[None])
    assert e8.tolist() == [[119]]
    want = [0x78, 0xF8, 0x70,
            0x70,   # 136 is half-way between 128 (m=0) and 144 (m=1): even -> 128
            0x72,   # 152 is half-way between 144 (m=1) and 160 (m=2): even -> 160
            0x01,   # 2^-9, the smallest subnormal
            0x02,   # 1.5 * 2^-9: half-way between codes 1 and 2 -> even (2)
            0x02,   # 2.5 * 2^-9: half-way between codes 2 and 3 -> even (2)
            0x00, 0xF0 | 0x04]  # -0.75 * 256 = -192 = -1.5 * 2^7 -> exponent 14, m = 4
    assert q[0, :10].tolist() == want
    assert np.all(q[0, 10:] == 0)


def test_saturation_powers_of_two_and_zero_block():
    # amax 1.9: shared -8, 1.9 * 256 = 486.4 lies past 448 and saturates
    q, e8 = oracle.quantize_mx8(_block([1.9, -1.9, 1.0])[None])
    assert e8[0, 0] == 119 and q[0, :3].tolist() == [0x7E, 0xFE, 0x78]
    # amax exactly 2: log2 is exactly 1, shared -7; 2 * 128 = 256
    q, e8 = oracle.quantize_mx8(_block([2.0, 1.0])[None])
    assert e8[0, 0] == 120 and q[0, :2].tolist() == [0x78, 0x70]
    # just below 2: shared -8
    q, e8 = oracle.quantize_mx8(_block([np.nextafter(2.0, 0.0)])[None])
    assert e8[0, 0] == 119 and q[0, 0] == 0x7E
    q, e8 = oracle.quantize_mx8(np.zeros((1, 64)))
    assert np.all(q == 0) and np.all(e8 == 0)
    np.testing.assert_array_equal(oracle.dequantize_mx8(q, e8), 0.0)


def _torch_mx8(v):
    """Reference MXFP8 value with torch's float8_e4m3fn rounding (round to
    nearest even) of the scaled block, clamped to +-448 first."""
    v = np.asarray(v, np.float64).reshape(-1, 32)
    out = np.zeros_like(v)
    for i, blk in enumerate(v):
        amax = np.max(np.abs(blk))
        if amax == 0:
            continue
        _, ex = math.frexp(amax)        # amax = f * 2^ex, f in [0.5, 1)
        shared = ex - 1 - 8
        s = np.clip(blk / 2.0 ** shared, -448, 448)
        r = torch.tensor(s, dtype=torch.float32).to(torch.float8_e4m3fn).to(torch.float64)
        out[i] = r.numpy() * 2.0 ** shared
    return out


@pytest.mark.parametrize("scale", [1e-3, 1.0, 37.0])
def test_matches_torch_float8_rounding(scale):
    rng = np.random.default_rng(int(scale * 1000))
    v = rng.standard_normal((40, 96)) * scale
    v[3] *= 1e-4                                   # a block of tiny values
    v[5, :32] = 0.0                                # a zero block
    # values exactly on E4M3 half-way points of their block's grid
    v[7, :32] = (np.arange(32) + 0.5) / 64.0
    q, e8 = oracle.quantize_mx8(v)
    got = oracle.dequantize_mx8(q, e8)
    np.testing.assert_array_equal(got, _torch_mx8(v).reshape(v.shape))


def test_error_bound_symmetry_scaling_lossless():
    rng = np.random.default_rng(7)
    v = rng.standard_normal((64, 128)) * np.exp(rng.uniform(-5, 5, (64, 1)))
    q, e8 = oracle.quantize_mx8(v)
    d = oracle.dequantize_mx8(q, e8)
    sc = np.repeat(2.0 ** (e8.astype(np.int64) - 127), 32, axis=1)
    a = np.abs(v) / sc                                   # element magnitude on the grid
    normal = (a >= 2.0 ** -6) & (a <= 448)
    sat = a > 448
    assert np.all(np.abs(d - v)[normal] <= 2.0 ** -4 * np.abs(v)[normal])
    assert np.all(np.abs(d - v)[a < 2.0 ** -6] <= 2.0 ** -10 * sc[a < 2.0 ** -6])
    assert np.all(np.abs(d)[sat] == 448 * sc[sat]) and sat.any()
    assert np.all(a < 512) and np.all(np.max(a.reshape(64, 4, 32), -1) >= 256)
    # symmetry
    qn, e8n = oracle.quantize_mx8(-v)
    assert np.array_equal(e8n, e8) and np.array_equal(qn, q ^ 0x80)
    # scaling by a power of two moves only the scale codes
    q2, e82 = oracle.quantize_mx8(v * 2.0 ** 5)
    assert np.array_equal(q2, q) and np.array_equal(e82.astype(int), e8.astype(int) + 5)
    # values already on the grid come back exactly
    q3, e83 = oracle.quantize_mx8(d)
    assert np.array_equal(oracle.dequantize_mx8(q3, e83), d)


def test_expert_loop_against_torch_composition():
    """oracle.experts_mx8 equals: MXFP8 of the input row (torch float8
    rounding), torch F.linear gate / up, torch GELU-tanh, MXFP8 of the gated
    product, torch F.linear down, weighted sum over the slots (all fp64)."""
    rng = np.random.default_rng(3)
    T, H, E, K, I = 7, 96, 4, 2, 64
    x = rng.standard_normal((T, H))
    gu = (rng.standard_normal((E, 2 * I, H)) / np.sqrt(H)).astype(np.float32)
    dn = (rng.standard_normal((E, H, I)) / np.sqrt(I)).astype(np.float32)
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.2, 1.0, (T, K)).astype(np.float32)
    got = oracle.experts_mx8(x, gu, dn, idx, w)
    t = lambda a: torch.tensor(np.asarray(a, np.float64))  # noqa: E731
    xq = t(_torch_mx8(x).reshape(T, H))
    ref = torch.zeros(T, H, dtype=torch.float64)
    for tt in range(T):
        for k in range(K):
            e = idx[tt, k]
            g = F.linear(xq[tt], t(gu[e, :I]))
            u = F.linear(xq[tt], t(gu[e, I:]))
            a = F.gelu(g, approximate="tanh") * u
            aq = t(_torch_mx8(a.numpy()).reshape(I))
            ref[tt] += float(w[tt, k]) * F.linear(aq, t(dn[e]))
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-13)
    # and it is the plain loop up to the 3-bit activation rounding
    plain = oracle.experts(x, gu, dn, idx, w)
    assert np.max(np.abs(got - plain)) / np.sqrt(np.mean(plain ** 2)) < 0.35
