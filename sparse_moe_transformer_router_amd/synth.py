"""Seeded synthetic inputs for the Gemma-4 26B-A4B feed-forward block.

This module draws random numbers and converts number formats; it holds none of
the block's arithmetic (no norm, no routing, no expert math).  Both the CPU
oracle tests and the GPU path take their inputs from here, so that the two
sides see identical bits.

Shapes follow the 26B-A4B layer described on the page "Porting a 128-expert
MoE (Gemma-4 26B-A4B) to AWS Inferentia2" (section "The architecture: a
dual-path FFN nobody warned me about": gate_up_proj [128,1408,2816],
down_proj [128,2816,704], dense MLP 2112) and the model config quoted on
"Lab 008 - Raw lab detail" (section "The model under test": 128 experts,
moe_intermediate_size 704, hidden 2816, 30 layers, gelu_pytorch_tanh).

Every tensor is drawn from numpy's PCG64 seeded by
SeedSequence([seed, tensor_id, layer]), in fp32, then rounded to bf16
(round to nearest even) where the tensor is stored in bf16.  A bf16 tensor is
handed around as its uint16 bit pattern plus the exactly widened fp32 copy.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# Hidden sizes of the 26B-A4B layer.
H_26B = 2816
E_26B = 128
K_26B = 8
I_26B = 704
D_26B = 2112

TENSOR_IDS = {
    "x": 1,
    "router_w": 2,
    "router_scale": 3,
    "per_expert_scale": 4,
    "gate_up": 5,
    "down": 6,
    "router_bias": 7,
    "g_pre": 8,
    "g_pre2": 9,
    "g_post1": 10,
    "g_post2": 11,
    "g_post": 12,
    "dense_gate": 13,
    "dense_up": 14,
    "dense_down": 15,
}


def rng_for(seed: int, name: str, layer: int = 0) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([seed, TENSOR_IDS[name], layer])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> fp32, exact."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Tensor:
    """A synthetic tensor: fp32 values plus, for bf16 storage, the bit pattern.

    ``f32`` always holds the exact values the kernels see (bf16 widened)."""
    f32: np.ndarray
    bf16: Optional[np.ndarray] = None

    @property
    def shape(self):
        return self.f32.shape


def _normal(seed, name, shape, std, layer=0, bf16=True) -> Tensor:
    v = rng_for(seed, name, layer).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    if not bf16:
        return Tensor(np.ascontiguousarray(v))
    bits = f32_to_bf16_bits(v)
    return Tensor(bf16_bits_to_f32(bits).reshape(shape), bits.reshape(shape))


def _uniform(seed, name, shape, lo, hi, layer=0) -> np.ndarray:
    return rng_for(seed, name, layer).uniform(lo, hi, size=shape).astype(np.float32)


@dataclasses.dataclass
class MoECase:
    """Inputs of the experts-only path (router, dispatch, experts, combine)."""
    T: int
    H: int
    E: int
    K: int
    I: int
    bf16: bool          # activations and expert weights stored as bf16
    eps: float
    x: Tensor           # [T,H]
    router_w: np.ndarray        # [E,H] fp32
    router_scale: np.ndarray    # [H] fp32
    per_expert_scale: np.ndarray  # [E] fp32
    gate_up: Tensor     # [E,2I,H]
    down: Tensor        # [E,H,I]


@dataclasses.dataclass
class BlockCase:
    """Inputs of one dual-path feed-forward layer."""
    moe: MoECase        # x is the residual input; router/experts weights
    D: int
    g_pre: np.ndarray
    g_pre2: np.ndarray
    g_post1: np.ndarray
    g_post2: np.ndarray
    g_post: np.ndarray
    dense_gate: Tensor  # [D,H]
    dense_up: Tensor    # [D,H]
    dense_down: Tensor  # [H,D]
    layer_scalar: float


def tiny_case(seed: int = 0, T: int = 16, H: int = 64, E: int = 8, K: int = 2,
              I: int = 32, bf16: bool = False) -> MoECase:
    """Tiny experts-only case: fp32, weights N(0,1)/sqrt(fan_in), activations N(0,1),
    router norm eps 1e-6 with scale 1, per_expert_scale ~ U(0.5, 1.5)."""
    x = _normal(seed, "x", (T, H), 1.0, bf16=bf16)
    rw = _normal(seed, "router_w", (E, H), 1.0 / np.sqrt(H), bf16=False).f32
    gu = _normal(seed, "gate_up", (E, 2 * I, H), 1.0 / np.sqrt(H), bf16=bf16)
    dn = _normal(seed, "down", (E, H, I), 1.0 / np.sqrt(I), bf16=bf16)
    return MoECase(T, H, E, K, I, bf16, 1e-6, x, rw,
                   np.ones(H, np.float32), _uniform(seed, "per_expert_scale", (E,), 0.5, 1.5),
                   gu, dn)


def moe_x(T: int, seed: int = 0, skew: bool = False, H: int = H_26B, bf16: bool = True,
          layer: int = 0) -> Tensor:
    """The experts-only case's input x [T, H] ~ N(0,1) (channel 0 set to 1
    when skew), exactly as moe_case draws it.  The first rows of a larger
    draw equal a smaller draw of the same seed."""
    x = _normal(seed, "x", (T, H), 1.0, layer=layer, bf16=False).f32
    if skew:
        x[:, 0] = 1.0
    if bf16:
        bits = f32_to_bf16_bits(x)
        return Tensor(bf16_bits_to_f32(bits).reshape(T, H), bits.reshape(T, H))
    return Tensor(x)


def moe_router_weights(seed: int = 0, skew: bool = False, H: int = H_26B, E: int = E_26B,
                       weight_std: float = 0.02, router_scale_std: float = 0.0,
                       layer: int = 0):
    """(router_w [E,H] fp32, router_scale [H], per_expert_scale [E]) as
    moe_case draws them."""
    rw = _normal(seed, "router_w", (E, H), weight_std, layer=layer, bf16=False).f32
    if skew:
        rw[:, 0] = _normal(seed, "router_bias", (E,), 1.0, layer=layer, bf16=False).f32
    if router_scale_std > 0:
        rs = (1.0 + _normal(seed, "router_scale", (H,), router_scale_std, layer=layer,
                            bf16=False).f32).astype(np.float32)
    else:
        rs = np.ones(H, np.float32)
    pes = _uniform(seed, "per_expert_scale", (E,), 0.5, 1.5, layer=layer)
    return rw, rs, pes


def moe_expert_weights(seed: int = 0, H: int = H_26B, E: int = E_26B, I: int = I_26B,
                       weight_std: float = 0.02, bf16: bool = True, layer: int = 0):
    """(gate_up [E,2I,H], down [E,H,I]) as moe_case draws them."""
    gu = _normal(seed, "gate_up", (E, 2 * I, H), weight_std, layer=layer, bf16=bf16)
    dn = _normal(seed, "down", (E, H, I), weight_std, layer=layer, bf16=bf16)
    return gu, dn


def moe_case(T: int, seed: int = 0, skew: bool = False, H: int = H_26B, E: int = E_26B,
             K: int = K_26B, I: int = I_26B, weight_std: float = 0.02,
             bf16: bool = True, router_scale_std: float = 0.0, layer: int = 0) -> MoECase:
    """26B-A4B-shaped experts-only case.  x ~ N(0,1); gate_up, down ~ N(0, 0.02)
    bf16; router weight N(0, 0.02) fp32 (near-uniform expert load).

    skew=True realises an imbalanced (Zipf-like) expert load through the data:
    channel 0 of every token is set to 1 and router_w[:,0] = b ~ N(0,1), so
    that after the router's RMSNorm each expert's logit is shifted by about b_e.
    """
    xt = moe_x(T, seed, skew, H, bf16, layer)
    rw, rs, pes = moe_router_weights(seed, skew, H, E, weight_std, router_scale_std, layer)
    gu, dn = moe_expert_weights(seed, H, E, I, weight_std, bf16, layer)
    return MoECase(T, H, E, K, I, bf16, 1e-6, xt, rw, rs, pes, gu, dn)


def block_case(T: int, seed: int = 0, H: int = H_26B, E: int = E_26B, K: int = K_26B,
               I: int = I_26B, D: int = D_26B, weight_std: float = 0.02, bf16: bool = True,
               layer: int = 0, layer_scalar: float = 0.06) -> BlockCase:
    """One dual-path layer: residual x ~ N(0,1), GEMM weights N(0, 0.02), norm
    gains 1 + N(0, 0.02), layer_scalar 0.06 (the order of the real per-layer
    value quoted on "Porting Gemma-4 (2B / 4B / 12B) to AWS Inferentia2",
    section 4.6)."""
    m = moe_case(T, seed=seed, H=H, E=E, K=K, I=I, weight_std=weight_std, bf16=bf16,
                 router_scale_std=0.02, layer=layer)

    def gain(name):
        return (1.0 + _normal(seed, name, (H,), 0.02, layer=layer, bf16=False).f32
                ).astype(np.float32)

    return BlockCase(
        m, D, gain("g_pre"), gain("g_pre2"), gain("g_post1"), gain("g_post2"), gain("g_post"),
        _normal(seed, "dense_gate", (D, H), weight_std, layer=layer, bf16=bf16),
        _normal(seed, "dense_up", (D, H), weight_std, layer=layer, bf16=bf16),
        _normal(seed, "dense_down", (H, D), weight_std, layer=layer, bf16=bf16),
        float(layer_scalar))



def toy_case() -> MoECase:
    """Hand-checkable 2-token, 4-expert case (H=64, K=2, I=1, fp32).

    Router rows are constant: expert 0 = 1/32, expert 1 = 1/64, expert 2 = 0,
    expert 3 = -1/64, so a token of all ones has logits (2r, r, 0, -r) with
    r = 1/sqrt(1 + eps), and the alternating token (2, -2, 2, ...) has four
    logits that are exactly zero (a four-way tie).  Expert 0: gate row 1/64,
    up row = unit vector at channel 0, down column = unit vector at channel 0.
    Expert 1: gate row 0.5 at channel 1, up row 1 at channel 2, down column =
    unit vector at channel 1.  Experts 2 and 3 hold 10 everywhere, so any
    misrouted slot shows up as a large error.
    """
    H, E, K, I = 64, 4, 2, 1
    x = np.ones((2, H), np.float32)
    x[1] = np.where(np.arange(H) % 2 == 0, 2.0, -2.0)
    rw = np.zeros((E, H), np.float32)
    rw[0], rw[1], rw[2], rw[3] = 1.0 / 32, 1.0 / 64, 0.0, -1.0 / 64
    gu = np.full((E, 2 * I, H), 10.0, np.float32)
    dn = np.full((E, H, I), 10.0, np.float32)
    gu[0, 0, :] = 1.0 / 64
    gu[0, 1, :] = 0.0
    gu[0, 1, 0] = 1.0
    dn[0, :, 0] = 0.0
    dn[0, 0, 0] = 1.0
    gu[1, :, :] = 0.0
    gu[1, 0, 1] = 0.5
    gu[1, 1, 2] = 1.0
    dn[1, :, 0] = 0.0
    dn[1, 1, 0] = 1.0
    pes = np.array([1.0, 2.0, 0.5, 1.5], np.float32)
    return MoECase(2, H, E, K, I, False, 1e-6, Tensor(x), rw, np.ones(H, np.float32), pes,
                   Tensor(gu), Tensor(dn))
