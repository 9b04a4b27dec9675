"""Seeded synthetic inputs for the routed-expert MoE layer.

This module only draws random numbers and stores them in the layer's interchange
layout. It contains none of the layer's arithmetic (no routing, no dequantisation,
no matrix products), so both the HIP path and the CPU oracle can be fed from it.

Interchange layout of one layer (E routed experts, S in {0,1} shared experts stacked
after them as expert index E, hidden H, expert intermediate I, group size 64):

  router_w  float32 [E, H]              router_b  float32 [E] or None
  int4 format (``fmt == "int4"``):
    w13_q  uint8  [E+S, 2I, H/2]   codes; byte j holds element 2j in its low nibble
                                   and element 2j+1 in its high nibble
    w13_s  uint16 [E+S, 2I, H/64]  bf16 bit patterns of the per-group scale
    w13_b  uint16 [E+S, 2I, H/64]  bf16 bit patterns of the per-group bias
    w2_q   uint8  [E+S, H, I/2]    w2_s / w2_b uint16 [E+S, H, I/64]
  fp32 format (``fmt == "f32"``):
    w13    float32 [E+S, 2I, H]    w2 float32 [E+S, H, I]

Rows 0..I-1 of w13 are the gate projection, rows I..2I-1 the up projection.
Activations are returned as bf16 bit patterns (uint16) for the bf16 configurations and
float32 for the fp32 configuration.

Workload shapes follow the Qwen3.6-35B-A3B MoE layer described in "Optimizing
On-Device Inference for Apple Silicon" (section "Qwen creates three distinct workload
shapes": 256 routed experts, eight selected, one shared) with the int4 group-64 format
of its section "Dequantize weights during matrix multiplication".
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

GROUP = 64
# standard deviation of a uniform 4-bit code in 0..15: sqrt((16**2 - 1) / 12)
NIBBLE_STD = math.sqrt(21.25)


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Layer:
    """One MoE layer in interchange layout (host numpy arrays)."""

    hidden: int
    inter: int
    n_experts: int
    top_k: int
    n_shared: int
    fmt: str  # "int4" or "f32"
    router_w: np.ndarray
    router_b: np.ndarray | None = None
    w13_q: np.ndarray | None = None
    w13_s: np.ndarray | None = None
    w13_b: np.ndarray | None = None
    w2_q: np.ndarray | None = None
    w2_s: np.ndarray | None = None
    w2_b: np.ndarray | None = None
    w13: np.ndarray | None = None
    w2: np.ndarray | None = None

    @property
    def n_total(self) -> int:
        return self.n_experts + self.n_shared

    def expert_bytes(self) -> int:
        """Stored bytes of one expert (codes + scales + biases, or fp32 values)."""
        H, I = self.hidden, self.inter
        if self.fmt == "f32":
            return 3 * H * I * 4
        codes = 2 * I * H // 2 + H * I // 2
        groups = 2 * I * H // GROUP + H * I // GROUP
        return codes + 2 * 2 * groups


def _int4_block(rng, rows_shape, K, scale_mag):
    codes = rng.integers(0, 256, size=(*rows_shape, K // 2), dtype=np.uint8)
    s = (rng.uniform(0.5, 1.5, size=(*rows_shape, K // GROUP)) * scale_mag).astype(np.float32)
    s_bits = f32_to_bf16_bits(s)
    s_val = bf16_bits_to_f32(s_bits)
    b = (-s_val * rng.uniform(6.5, 8.5, size=s_val.shape)).astype(np.float32)
    return codes, s_bits, f32_to_bf16_bits(b)


def make_int4_layer(seed: int, hidden=2048, inter=512, n_experts=256, top_k=8,
                    n_shared=1, router_std=0.02, weight_std=0.02,
                    router_bias: np.ndarray | None = None) -> Layer:
    """Int4 group-64 layer. Draw order per seed: router, W13 codes/scales/biases,
    W2 codes/scales/biases (expert index n_experts is the shared expert)."""
    assert hidden % GROUP == 0 and inter % GROUP == 0
    rng = np.random.default_rng(seed)
    E, H, I, n = n_experts, hidden, inter, n_experts + n_shared
    router_w = rng.normal(0.0, router_std, size=(E, H)).astype(np.float32)
    mag = weight_std / NIBBLE_STD
    w13_q, w13_s, w13_b = _int4_block(rng, (n, 2 * I), H, mag)
    w2_q, w2_s, w2_b = _int4_block(rng, (n, H), I, mag)
    rb = None if router_bias is None else np.ascontiguousarray(router_bias, dtype=np.float32)
    return Layer(H, I, E, top_k, n_shared, "int4", router_w, rb,
                 w13_q=w13_q, w13_s=w13_s, w13_b=w13_b, w2_q=w2_q, w2_s=w2_s, w2_b=w2_b)


def make_f32_layer(seed: int, hidden=128, inter=64, n_experts=256, top_k=8, n_shared=1,
                   std=0.05) -> tuple[Layer, np.random.Generator]:
    """Unquantised fp32 layer; returns the generator so activations continue the stream."""
    rng = np.random.default_rng(seed)
    E, H, I, n = n_experts, hidden, inter, n_experts + n_shared
    router_w = rng.normal(0.0, std, size=(E, H)).astype(np.float32)
    w13 = rng.normal(0.0, std, size=(n, 2 * I, H)).astype(np.float32)
    w2 = rng.normal(0.0, std, size=(n, H, I)).astype(np.float32)
    return Layer(H, I, E, top_k, n_shared, "f32", router_w, None, w13=w13, w2=w2), rng


def zipf_router_bias(n_experts=256, hidden=2048, router_std=0.02, gamma=0.7, s=1.1,
                     seed=1) -> np.ndarray:
    """Per-expert router bias whose induced popularity decays like rank**-s.

    b_e = -gamma * sigma_z * s * ln(rank_e), sigma_z = router_std * sqrt(hidden), with
    rank a seeded permutation of 1..n_experts."""
    rank = np.random.default_rng(seed).permutation(n_experts) + 1
    sigma_z = router_std * math.sqrt(hidden)
    return (-gamma * sigma_z * s * np.log(rank)).astype(np.float32)


def bf16_activations(seed: int, shape) -> np.ndarray:
    """bf16 bit patterns of standard normal draws."""
    return f32_to_bf16_bits(np.random.default_rng(seed).standard_normal(shape).astype(np.float32))


# ---- named workloads -----------------------------------------------------------------

def tiny_config(seed: int = 0):
    """fp32 layer T=64, H=128, I=64, E=256, k=8, one shared expert; weights ~N(0,0.05),
    x ~ N(0,1), all from one generator seeded with ``seed``."""
    layer, rng = make_f32_layer(seed)
    x = rng.standard_normal((64, layer.hidden)).astype(np.float32)
    return layer, x


def decode_layer(seed: int = 0) -> Layer:
    """Decode-shaped layer: H=2048, I=512, E=256, k=8, S=1, int4 g64, router ~N(0,0.02)."""
    return make_int4_layer(seed)


def decode_token(t: int, hidden: int = 2048) -> np.ndarray:
    """bf16 bits of decode token t (1 x H)."""
    return bf16_activations(1_000_000 + t, (1, hidden))


def prefill_x(T: int = 4096, hidden: int = 2048, seed: int = 2) -> np.ndarray:
    return bf16_activations(seed, (T, hidden))


def skewed_layer(seed: int = 0, gamma: float = 0.7) -> Layer:
    return make_int4_layer(seed, router_bias=zipf_router_bias(gamma=gamma))


# ---- decode attention inputs ---------------------------------------------------------------
# Grouped-query attention of the model's full-attention layers: 16 query heads, two key-value
# heads (eight query heads per KV head), 256 values per head, bf16 cache.
ATTN_Q_HEADS, ATTN_KV_HEADS, ATTN_HEAD_DIM = 16, 2, 256


def attn_inputs(ctx: int, seed: int = 0, n_q: int = ATTN_Q_HEADS, n_kv: int = ATTN_KV_HEADS,
                D: int = ATTN_HEAD_DIM, n_hot: int = 16, hot_score: float = 8.0):
    """One decode token's query and a KV cache of ctx positions, as bf16 bit patterns:
    q [n_q, D], k and v [n_kv, ctx, D]. Draw order per seed: q, k, v ~ N(0, 1), then the
    n_hot "hot" positions per KV head (without replacement). A hot key is the mean of its
    group's queries scaled so that that mean query scores hot_score against it at scale
    1/sqrt(D), so the softmax has a few dominant positions over a flat background, as
    attention over a long context does."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n_q, D), dtype=np.float32)
    k = rng.standard_normal((n_kv, ctx, D), dtype=np.float32)
    v = rng.standard_normal((n_kv, ctx, D), dtype=np.float32)
    qb = f32_to_bf16_bits(q)
    qf = bf16_bits_to_f32(qb).astype(np.float64)
    G = n_q // n_kv
    scale = 1.0 / np.sqrt(D)
    for g in range(n_kv):
        hot = rng.choice(ctx, size=min(n_hot, ctx), replace=False)
        qbar = qf[g * G:(g + 1) * G].mean(axis=0)
        k[g, hot] = (hot_score / (scale * float(qbar @ qbar)) * qbar).astype(np.float32)
    return qb, f32_to_bf16_bits(k), f32_to_bf16_bits(v)


# ---- Gated DeltaNet inputs ------------------------------------------------------------------
# Dimensions: 32 value heads and 16 key heads of 128 values each, so that one layer's fp32
# state is 32 x 128 x 128 x 4 B = 2 MiB (a blockwise scan over 2K tokens in 32-token blocks
# then reads and writes 256 MiB of state, the figure the page gives for its ablation).
GDN_K_HEADS, GDN_V_HEADS, GDN_DK, GDN_DV = 16, 32, 128, 128


def gdn_inputs(T: int, seed: int = 0, n_k: int = GDN_K_HEADS, n_v: int = GDN_V_HEADS,
               d_k: int = GDN_DK, d_v: int = GDN_DV):
    """Inputs of a Gated DeltaNet scan over T tokens. Draw order per seed: q, k, v ~ N(0, 1),
    then the gate and write-strength logits ~ N(3, 1) and N(0, 1). q and k are L2-normalised
    per (token, head) in fp32 (q further scaled by 1/sqrt(d_k)) and rounded to bf16; v is
    bf16; alpha = sigmoid(N(3, 1)) (the state keeps about 95 % per token) and
    beta = sigmoid(N(0, 1)) stay fp32. Returns (q, k [T, n_k, d_k], v [T, n_v, d_v] as bf16
    bits; alpha, beta [T, n_v] float32)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, n_k, d_k), dtype=np.float32)
    k = rng.standard_normal((T, n_k, d_k), dtype=np.float32)
    v = rng.standard_normal((T, n_v, d_v), dtype=np.float32)
    ga = rng.standard_normal((T, n_v), dtype=np.float32) + 3.0
    gb = rng.standard_normal((T, n_v), dtype=np.float32)
    q /= np.linalg.norm(q, axis=-1, keepdims=True) * np.float32(np.sqrt(d_k))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    alpha = (1.0 / (1.0 + np.exp(-ga))).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-gb))).astype(np.float32)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v), alpha, beta
