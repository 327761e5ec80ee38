"""Pins of the oracle's int8 per-channel symmetric weights (the int8-expert
variant of "Porting a 128-expert MoE (Gemma-4 26B-A4B) to AWS Inferentia2",
section "Can it run on a smaller box?"): hand-computed codes with exact
ties, the rounding error bound, symmetry and exact power-of-two scaling,
zero rows, and the lossless case where the int8 expert FFN must equal the
plain one bit for bit."""
import numpy as np

import oracle
from sparse_moe_transformer_router_amd import synth


def test_hand_codes_round_half_to_even():
    # max |w| = 127 * 2^-4, so s = 2^-4 exactly and w / s is exact
    row = np.array([127, 63.5, -62.5, 0.5, -0.5, 1.5, 2.5, 0, -127], np.float32) / 16
    q, s = oracle.quantize_int8(row[None, :])
    assert s[0] == np.float32(1 / 16)
    assert q[0].tolist() == [127, 64, -62, 0, 0, 2, 2, 0, -127]


def test_zero_row():
    q, s = oracle.quantize_int8(np.zeros((2, 64), np.float32))
    assert np.all(q == 0) and np.all(s == 0)
    assert np.all(oracle.dequantize_int8(q, s) == 0)


def test_error_bound_and_extreme_code():
    rng = np.random.default_rng(0)
    w = (rng.standard_normal((37, 300)) * rng.uniform(0.01, 3, (37, 1))).astype(np.float32)
    q, s = oracle.quantize_int8(w)
    err = np.abs(w.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None] * 0.5 * (1 + 1e-5))
    assert np.all(np.abs(q).max(axis=1) == 127)
    assert np.all(np.abs(q) <= 127)
    # the channel's largest magnitude maps to +-127 with its own sign
    j = np.abs(w).argmax(axis=1)
    assert np.all(q[np.arange(37), j] == np.sign(w[np.arange(37), j]) * 127)


def test_symmetry_and_power_of_two_scaling():
    rng = np.random.default_rng(1)
    w = rng.standard_normal((9, 128)).astype(np.float32)
    q, s = oracle.quantize_int8(w)
    qn, sn = oracle.quantize_int8(-w)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    for j in (-3, 5):
        qs, ss = oracle.quantize_int8(w * np.float32(2.0 ** j))
        assert np.array_equal(qs, q)
        assert np.array_equal(ss, s * np.float32(2.0 ** j))


def test_lossless_weights_give_the_plain_expert_ffn():
    """Weights of the form q * 2^-k with a +-127 code in every channel survive
    quantization unchanged, so the int8 expert FFN equals the plain one."""
    c = synth.tiny_case(seed=5, T=12, H=64, E=6, K=2, I=32)
    rng = np.random.default_rng(2)

    def exact(shape, k):
        codes = rng.integers(-127, 128, size=shape).astype(np.float32)
        codes[..., 0] = 127
        return codes * np.float32(2.0 ** -k)

    gu, dn = exact(c.gate_up.f32.shape, 9), exact(c.down.f32.shape, 8)
    guq, gus = oracle.quantize_int8(gu)
    dnq, dns = oracle.quantize_int8(dn)
    assert np.array_equal(oracle.dequantize_int8(guq, gus), gu)
    assert np.array_equal(oracle.dequantize_int8(dnq, dns), dn)
    idx, w = oracle.router(c.x.f32, c.router_w, c.router_scale, c.per_expert_scale, c.K)
    a = oracle.experts(c.x.f32, gu, dn, idx, w)
    b = oracle.experts_int8(c.x.f32, guq, gus, dnq, dns, idx, w)
    assert np.array_equal(a, b)
