"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Every check here is a closed form, an invariant, a library routine (torch fp64
``linear``/``silu``/``rms_norm``, scipy ``softmax``, numpy sort and matmul) or brute
force on tiny inputs, chosen so that a plausible slip in the oracle (a dropped term,
a wrong sign or index, a swapped nibble, a transposed operand, a weight attached to
the wrong expert) fails at least one of them.

Source of what the layer computes: "Optimizing On-Device Inference for Apple Silicon",
sections "Qwen creates three distinct workload shapes" (256 experts, eight selected,
one shared), "Dequantize weights during matrix multiplication" (int4 codes, one bf16
scale and bias per 64 weights), "Keep expert routing on the GPU" (histogram, prefix
scan, grouping) and "Reduce intermediate and state traffic" (gated input projections,
output projection combined with the routing score and the shared expert).
"""
import itertools
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from routed_expert_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_int4(seed, H=128, I=64, E=16, k=4, S=1, router_bias=None):
    return synth.make_int4_layer(seed, hidden=H, inter=I, n_experts=E, top_k=k, n_shared=S,
                                 router_std=0.05, weight_std=0.05, router_bias=router_bias)


def small_f32(seed, H=32, I=16, E=8, k=2, S=1):
    layer, _ = synth.make_f32_layer(seed, hidden=H, inter=I, n_experts=E, top_k=k,
                                    n_shared=S, std=0.2)
    return layer


def dense_swiglu_torch(w13, w2, x):
    """Textbook SwiGLU MLP with torch fp64 library ops: W2 (silu(W1 x) * (W3 x))."""
    w13 = torch.as_tensor(np.asarray(w13, dtype=np.float64))
    w2 = torch.as_tensor(np.asarray(w2, dtype=np.float64))
    x = torch.as_tensor(np.asarray(x, dtype=np.float64))
    inter = w13.shape[0] // 2
    g = torch.nn.functional.linear(x, w13[:inter])
    u = torch.nn.functional.linear(x, w13[inter:])
    return torch.nn.functional.linear(torch.nn.functional.silu(g) * u, w2).numpy()


def bf16(v):
    return synth.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def rng_x(seed, T, H):
    return np.random.default_rng(seed).standard_normal((T, H)).astype(np.float32)


# ---- dequantisation --------------------------------------------------------------------

def test_dequant_nibble_order_golden(oracle_lib):
    # byte 0x21: element 0 is the low nibble (1), element 1 the high nibble (2)
    codes = np.zeros((1, 32), dtype=np.uint8)
    codes[0, 0] = 0x21
    codes[0, 1] = 0xF0
    s = bf16([[1.0]])
    b = bf16([[0.0]])
    w = oracle.dequant(codes, s, b)
    assert w[0, 0] == 1.0 and w[0, 1] == 2.0 and w[0, 2] == 0.0 and w[0, 3] == 15.0
    assert np.all(w[0, 4:] == 0.0)


def test_dequant_closed_form_pattern(oracle_lib):
    # code of element c is c mod 16; group g has scale 2^-(g+1) and bias g/4 - 1, so
    # w[r, c] = 2^-(g+1) * (c mod 16) + g/4 - 1 exactly (all values are dyadic).
    rows, K = 3, 256
    c = np.arange(K)
    q = c % 16
    byte = (q[0::2] | (q[1::2] << 4)).astype(np.uint8)
    codes = np.tile(byte, (rows, 1))
    g = np.arange(K // 64)
    s = np.tile(bf16(2.0 ** -(g + 1.0)), (rows, 1))
    b = np.tile(bf16(g / 4.0 - 1.0), (rows, 1))
    w = oracle.dequant(codes, s, b)
    expect = 2.0 ** -(c // 64 + 1.0) * q + (c // 64) / 4.0 - 1.0
    assert np.array_equal(w, np.tile(expect, (rows, 1)))


def test_dequant_extremes(oracle_lib):
    rng = np.random.default_rng(3)
    s = bf16(rng.uniform(0.01, 0.1, (4, 2)))
    b = bf16(rng.uniform(-1, 1, (4, 2)))
    sf, bfv = synth.bf16_bits_to_f32(s).astype(np.float64), synth.bf16_bits_to_f32(b).astype(np.float64)
    w0 = oracle.dequant(np.zeros((4, 64), np.uint8), s, b)
    assert np.array_equal(w0, np.repeat(bfv, 64, axis=1))          # q = 0 -> bias
    w15 = oracle.dequant(np.full((4, 64), 0xFF, np.uint8), s, b)
    assert np.array_equal(w15, np.repeat(15 * sf + bfv, 64, axis=1))  # q = 15 -> 15 s + b
    wz = oracle.dequant(rng.integers(0, 256, (4, 64), dtype=np.uint8), bf16(np.zeros((4, 2))), b)
    assert np.array_equal(wz, np.repeat(bfv, 64, axis=1))          # s = 0 -> bias


# ---- router, top-k, renormalisation -----------------------------------------------------

def test_logits_one_hot_rows(oracle_lib):
    H, E = 64, 16
    layer = small_f32(0, H=H, E=E, k=2)
    pick = np.random.default_rng(1).integers(0, H, E)
    layer.router_w = np.zeros((E, H), np.float32)
    layer.router_w[np.arange(E), pick] = 1.0
    x = rng_x(2, 5, H)
    z = oracle.logits(layer, x)
    assert np.array_equal(z, x[:, pick].astype(np.float64))


def test_logits_match_numpy_matmul_with_bias(oracle_lib):
    layer = small_f32(4, H=48, E=12, k=3)
    layer.router_b = np.random.default_rng(5).normal(0, 1, 12).astype(np.float32)
    x = rng_x(6, 7, 48)
    z = oracle.logits(layer, x)
    ref = x.astype(np.float64) @ layer.router_w.astype(np.float64).T + layer.router_b
    np.testing.assert_allclose(z, ref, rtol=0, atol=1e-12)


def test_all_ties_pick_lowest_ids_uniform_weights(oracle_lib):
    layer = small_int4(0, E=32, k=8)
    layer.router_w = np.zeros_like(layer.router_w)
    ids, w, margin = oracle.route(layer, synth.bf16_activations(1, (5, layer.hidden)))
    assert np.array_equal(ids, np.tile(np.arange(8, dtype=np.int32), (5, 1)))
    assert np.all(w == 1.0 / 8) and np.all(margin == 0.0)


def test_decreasing_bias_gives_softmax_of_bias(oracle_lib):
    E, k = 32, 8
    bias = np.linspace(1.0, -2.0, E).astype(np.float32)
    layer = small_int4(0, E=E, k=k, router_bias=bias)
    layer.router_w = np.zeros_like(layer.router_w)
    ids, w, _ = oracle.route(layer, synth.bf16_activations(1, (3, layer.hidden)))
    assert np.array_equal(ids, np.tile(np.arange(k, dtype=np.int32), (3, 1)))
    ref = scipy.special.softmax(bias[:k].astype(np.float64))
    np.testing.assert_allclose(w, np.tile(ref, (3, 1)), rtol=1e-14, atol=0)


def test_partial_ties_go_to_lower_id(oracle_lib):
    E, k = 8, 3
    layer = small_f32(0, H=16, E=E, k=k)
    layer.router_w = np.zeros_like(layer.router_w)
    layer.router_b = np.array([0, 1, 0, 1, 2, 0, 1, 0], np.float32)
    ids, w, margin = oracle.route(layer, np.zeros((1, 16), np.float32))
    assert ids.tolist() == [[1, 3, 4]]          # 2, then the two lowest ids tied at 1
    assert margin[0] == 0.0                     # expert 6 ties with the third pick


def test_topk_brute_force_over_subsets(oracle_lib):
    E, k, T = 10, 3, 25
    layer = small_f32(7, H=16, E=E, k=k)
    x = rng_x(8, T, 16)
    ids, w, margin = oracle.route(layer, x)
    z = x.astype(np.float64) @ layer.router_w.astype(np.float64).T
    for t in range(T):
        best = max(itertools.combinations(range(E), k), key=lambda c: sum(z[t, list(c)]))
        assert ids[t].tolist() == list(best)
        p = scipy.special.softmax(z[t])
        np.testing.assert_allclose(w[t], p[list(best)] / p[list(best)].sum(), rtol=1e-13)
        zs = np.sort(z[t])[::-1]
        np.testing.assert_allclose(margin[t], zs[k - 1] - zs[k], rtol=0, atol=1e-15)


def test_weights_sum_to_one_and_follow_logits(oracle_lib):
    layer, x = synth.tiny_config()
    ids, w, _ = oracle.route(layer, x)
    z = oracle.logits(layer, x)
    assert np.all(np.abs(w.sum(1) - 1.0) <= 1e-15) and np.all(w > 0)
    for t in range(x.shape[0]):
        order_w = np.argsort(-w[t], kind="stable")
        order_z = np.argsort(-z[t, ids[t]], kind="stable")
        assert np.array_equal(order_w, order_z)
        assert np.all(np.diff(ids[t]) > 0)


# ---- grouping --------------------------------------------------------------------------

def _check_grouping(ids, counts, offsets, sorted_tok, slot_of, E, k):
    T = ids.shape[0]
    assert counts.sum() == k * T
    assert np.array_equal(counts, np.bincount(ids.reshape(-1), minlength=E))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts) and offsets[-1] == k * T
    for t in range(T):
        assert len(set(ids[t].tolist())) == k
        for j in range(k):
            s = slot_of[t, j]
            assert sorted_tok[s] == t and offsets[ids[t, j]] <= s < offsets[ids[t, j] + 1]
    for e in range(E):
        grp = sorted_tok[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(grp) > 0)  # stable: tokens ascending inside a group
        assert set(grp.tolist()) == set(np.nonzero((ids == e).any(1))[0].tolist())


def test_grouping_invariants_tiny(oracle_lib):
    layer, x = synth.tiny_config()
    ids, _, _ = oracle.route(layer, x)
    counts, offsets, sorted_tok, slot_of = oracle.group(layer, ids)
    _check_grouping(ids, counts, offsets, sorted_tok, slot_of, 256, 8)


def test_grouping_page_example_2k_prompt(oracle_lib):
    with open(os.path.join(GOLDEN, "assignments_2k.json")) as f:
        g = json.load(f)
    T, E, k = g["tokens"], g["experts"], g["top_k"]
    layer = synth.make_f32_layer(0, hidden=64, inter=64, n_experts=E, top_k=k)[0]
    x = rng_x(9, T, 64)
    ids, _, _ = oracle.route(layer, x)
    counts, offsets, sorted_tok, slot_of = oracle.group(layer, ids)
    assert counts.sum() == g["assignments"] and offsets[-1] == g["assignments"]
    assert counts.mean() == g["mean_rows_per_expert"]
    _check_grouping(ids, counts, offsets, sorted_tok, slot_of, E, k)


# ---- experts and the full layer ---------------------------------------------------------

def test_single_expert_is_dense_swiglu_f32(oracle_lib):
    layer = small_f32(11, H=32, I=16, E=1, k=1, S=0)
    x = rng_x(12, 6, 32)
    y = oracle.moe(layer, x)
    ref = dense_swiglu_torch(layer.w13[0], layer.w2[0], x)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)


def test_single_expert_is_dense_swiglu_int4(oracle_lib):
    layer = small_int4(13, H=128, I=64, E=1, k=1, S=0)
    x = synth.bf16_activations(14, (4, 128))
    y = oracle.moe(layer, x)
    w13 = oracle.dequant(layer.w13_q[0], layer.w13_s[0], layer.w13_b[0])
    w2 = oracle.dequant(layer.w2_q[0], layer.w2_s[0], layer.w2_b[0])
    ref = dense_swiglu_torch(w13, w2, synth.bf16_bits_to_f32(x))
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)


def test_zero_input_gives_zero_output(oracle_lib):
    layer = small_int4(15)
    y = oracle.moe(layer, np.zeros((3, layer.hidden), np.float32))
    assert np.all(y == 0.0)


def test_identical_experts_collapse(oracle_lib):
    # every routed expert equal => y = shared(x) + expert(x) for any routing (sum w = 1)
    layer = small_f32(16, H=32, I=16, E=8, k=3, S=1)
    layer.w13[:8] = layer.w13[0]
    layer.w2[:8] = layer.w2[0]
    x = rng_x(17, 9, 32)
    y = oracle.moe(layer, x)
    ref = dense_swiglu_torch(layer.w13[8], layer.w2[8], x) + dense_swiglu_torch(layer.w13[0], layer.w2[0], x)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_weights_attach_to_their_experts(oracle_lib):
    # zero router + decreasing bias: ids 0..k-1 with weights softmax(bias[:k]); expert e's
    # output projection is 2^e * W2_base (exact in fp32), so y = shared + sum_j w_j 2^j base(x).
    E, k = 8, 3
    layer = small_f32(18, H=32, I=16, E=E, k=k, S=1)
    layer.router_w = np.zeros_like(layer.router_w)
    layer.router_b = np.linspace(0.5, -1.5, E).astype(np.float32)
    layer.w13[:E] = layer.w13[0]
    for e in range(E):
        layer.w2[e] = layer.w2[0] * np.float32(2.0 ** e) if e else layer.w2[0]
    x = rng_x(19, 5, 32)
    y = oracle.moe(layer, x)
    p = scipy.special.softmax(layer.router_b[:k].astype(np.float64))
    base = dense_swiglu_torch(layer.w13[0], layer.w2[0], x)
    ref = dense_swiglu_torch(layer.w13[E], layer.w2[E], x) + sum(p[j] * 2.0 ** j * base for j in range(k))
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_shared_expert_adds_exactly_its_output(oracle_lib):
    layer = small_f32(20, H=32, I=16, E=8, k=2, S=1)
    x = rng_x(21, 6, 32)
    y1 = oracle.moe(layer, x)
    layer0 = small_f32(20, H=32, I=16, E=8, k=2, S=1)
    layer0.n_shared = 0
    layer0.w13 = layer0.w13[:8].copy()
    layer0.w2 = layer0.w2[:8].copy()
    y0 = oracle.moe(layer0, x)
    np.testing.assert_allclose(y1 - y0, dense_swiglu_torch(layer.w13[8], layer.w2[8], x),
                               rtol=1e-10, atol=1e-13)


def test_output_projection_scaling(oracle_lib):
    layer = small_f32(22)
    x = rng_x(23, 4, layer.hidden)
    y = oracle.moe(layer, x)
    layer.w2 = layer.w2 * np.float32(4.0)
    assert np.array_equal(oracle.moe(layer, x), 4.0 * y)


def test_tiny_layer_brute_force(oracle_lib):
    # full brute force on a small layer: full sort for top-k, scipy softmax, torch SwiGLU
    E, k, H, I, T = 12, 3, 32, 16, 10
    layer = small_f32(24, H=H, I=I, E=E, k=k, S=1)
    x = rng_x(25, T, H)
    y = oracle.moe(layer, x)
    z = x.astype(np.float64) @ layer.router_w.astype(np.float64).T
    for t in range(T):
        sel = sorted(np.argsort(-z[t], kind="stable")[:k].tolist())
        p = scipy.special.softmax(z[t])[sel]
        p = p / p.sum()
        ref = dense_swiglu_torch(layer.w13[E], layer.w2[E], x[t])
        for j, e in enumerate(sel):
            ref = ref + p[j] * dense_swiglu_torch(layer.w13[e], layer.w2[e], x[t])
        np.testing.assert_allclose(y[t], ref, rtol=1e-11, atol=1e-13)


def test_token_independence(oracle_lib):
    layer = small_int4(26)
    x = synth.bf16_activations(27, (6, layer.hidden))
    y = oracle.moe(layer, x)
    for t in (0, 3, 5):
        assert np.array_equal(oracle.moe(layer, x[t:t + 1])[0], y[t])


# ---- RMSNorm (layer stack glue) ---------------------------------------------------------

def test_rmsnorm_constant_row_and_torch(oracle_lib):
    c = 0.75
    out = oracle.rmsnorm(np.full((1, 64), c, np.float32), 1e-6)
    np.testing.assert_allclose(out, c / np.sqrt(c * c + 1e-6), rtol=1e-15)
    h = rng_x(28, 5, 96).astype(np.float64)
    ref = torch.nn.functional.rms_norm(torch.as_tensor(h), (96,), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.rmsnorm(h, 1e-6), ref, rtol=1e-13)


# ---- decode attention ------------------------------------------------------------------
# What it computes: per query head, the softmax-weighted average of its key-value head's
# cached values, weights from the scaled query-key scores; eight query heads share one KV
# head ("Qwen creates three distinct workload shapes", "Read the attention cache
# efficiently"). Readings: consecutive query heads share a KV head; scale 1/sqrt(D).

def _attn_rand(seed, n_kv, ctx, D, n_q):
    rng = np.random.default_rng(seed)
    q = bf16(rng.standard_normal((n_q, D)))
    k = bf16(rng.standard_normal((n_kv, ctx, D)))
    v = bf16(rng.standard_normal((n_kv, ctx, D)))
    return q, k, v


def _bf16_neighbours(v):
    """The two bf16 values bracketing float64 v (brute force over the bit patterns of the
    float32 truncation and its successor), as float64."""
    f = np.float32(v)
    if abs(float(f)) > abs(v):  # float32 rounding went away from zero: step back
        f = np.nextafter(f, np.float32(0.0))
    lo_bits = (np.array([f], np.float32).view(np.uint32)[0] >> 16).astype(np.uint32)
    lo = float((np.array([lo_bits << 16], np.uint32)).view(np.float32)[0])
    hi = float((np.array([(lo_bits + 1) << 16], np.uint32)).view(np.float32)[0])
    return (lo, int(lo_bits)), (hi, int(lo_bits) + 1)


def test_round_bf16_matches_torch_on_float32_values(oracle_lib):
    # torch rounds float32 to bf16 to nearest, ties to even: for values that are exact in
    # float32 that is the single rounding the oracle must reproduce (normal, subnormal,
    # both signs, exact bf16 values and exact midpoints included)
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(4000),
                        rng.standard_normal(500) * 1e-39,          # bf16 subnormals
                        rng.standard_normal(500) * 1e30,
                        [0.0, -0.0, 1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 3.0e38]])
    x = x.astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)
    # the two exact midpoints above round to the even neighbour
    assert got[-3] == 0x3F80 and got[-2] == 0x3F82


def test_round_bf16_brute_force_nearest_on_float64(oracle_lib):
    # values that are not float32: the result is the nearer of the two bracketing bf16
    # values, the even one on an exact tie (no detour through float32)
    rng = np.random.default_rng(12)
    vals = rng.standard_normal(3000) * np.exp(rng.uniform(-20, 20, 3000))
    got = oracle.round_bf16(vals)
    for v, g in zip(vals, got):
        (lo, lb), (hi, hb) = _bf16_neighbours(abs(v))
        d_lo, d_hi = abs(v) - lo, hi - abs(v)
        assert d_lo >= 0 and d_hi >= 0
        want = lb if (d_lo < d_hi or (d_lo == d_hi and lb % 2 == 0)) else hb
        assert (int(g) & 0x7FFF) == want and (int(g) >> 15) == (v < 0)
    # a value just above a midpoint whose float32 rounding lands exactly on the midpoint:
    # rounding through float32 would tie to the even (lower) neighbour, the exact value
    # rounds up
    mid = 1.0 + 2.0 ** -8                     # between 1.0 (0x3F80) and 1 + 2^-7 (0x3F81)
    v = mid + 2.0 ** -40
    assert float(np.float32(v)) == mid
    assert oracle.round_bf16(np.array([v]))[0] == 0x3F81
    assert oracle.round_bf16(np.array([mid]))[0] == 0x3F80


def test_stack_layer_input_constant_row(oracle_lib):
    # RMSNorm of a constant row c is c / sqrt(c^2 + eps) in every element, then one
    # rounding to bf16
    c, eps = 0.75, 1e-6
    h = synth.f32_to_bf16_bits(np.full((2, 64), c, np.float32))
    want = oracle.round_bf16(np.full((2, 64), c / np.sqrt(c * c + eps)))
    assert np.array_equal(oracle.stack_layer_input(h, eps), want)
    assert np.all(want == 0x3F80)              # 0.99999911 rounds to 1.0


def test_attn_single_position_returns_its_value():
    q, k, v = _attn_rand(1, 2, 1, 16, 4)
    out = oracle.attn_decode(q, k, v, 4, 2, 0.25)
    vf = synth.bf16_bits_to_f32(v).astype(np.float64)
    for h in range(4):
        assert np.array_equal(out[h], vf[h // 2, 0])


def test_attn_equal_keys_give_the_mean_value():
    # identical keys: every score equal, softmax uniform, output = plain mean of the values
    q, k, v = _attn_rand(2, 2, 37, 16, 8)
    k[:] = k[:, :1]
    out = oracle.attn_decode(q, k, v, 8, 2, 0.25)
    vf = synth.bf16_bits_to_f32(v).astype(np.float64)
    for h in range(8):
        np.testing.assert_allclose(out[h], vf[h // 4].mean(axis=0), rtol=0, atol=1e-13)


def test_attn_dominant_key_selects_its_value():
    q, k, v = _attn_rand(3, 1, 50, 16, 2)
    qf = synth.bf16_bits_to_f32(q).astype(np.float64)
    k[0, 17] = bf16(40.0 * qf.mean(axis=0))   # score tens of units above every other
    out = oracle.attn_decode(q, k, v, 2, 1, 1.0)
    vf = synth.bf16_bits_to_f32(v).astype(np.float64)
    for h in range(2):
        np.testing.assert_allclose(out[h], vf[0, 17], rtol=0, atol=1e-9)


def test_attn_matches_torch_sdpa_with_grouped_heads():
    # the library's scaled-dot-product attention on the CPU in fp64, KV heads expanded so
    # that query head h reads KV head h // G
    n_q, n_kv, D, ctx = 8, 2, 32, 53
    q, k, v = _attn_rand(4, n_kv, ctx, D, n_q)
    scale = 0.37
    out = oracle.attn_decode(q, k, v, n_q, n_kv, scale)
    f = lambda a: torch.as_tensor(synth.bf16_bits_to_f32(a).astype(np.float64))
    G = n_q // n_kv
    kk = f(k).repeat_interleave(G, dim=0)[None]           # [1, n_q, ctx, D]
    vv = f(v).repeat_interleave(G, dim=0)[None]
    qq = f(q)[None, :, None, :]                           # [1, n_q, 1, D]
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)
    np.testing.assert_allclose(out, ref[0, :, 0].numpy(), rtol=1e-12, atol=1e-13)


def test_attn_heads_read_only_their_kv_head():
    n_q, n_kv, D, ctx = 6, 3, 16, 20
    q, k, v = _attn_rand(5, n_kv, ctx, D, n_q)
    base = oracle.attn_decode(q, k, v, n_q, n_kv, 0.25)
    v2 = v.copy()
    v2[1] = bf16(np.full((ctx, D), 3.0))                  # change KV head 1 only
    out = oracle.attn_decode(q, k, v2, n_q, n_kv, 0.25)
    assert np.array_equal(out[[0, 1, 4, 5]], base[[0, 1, 4, 5]])
    np.testing.assert_allclose(out[[2, 3]], 3.0, rtol=0, atol=1e-12)


def test_attn_is_invariant_to_reordering_positions():
    q, k, v = _attn_rand(6, 2, 41, 16, 4)
    perm = np.random.default_rng(7).permutation(41)
    a = oracle.attn_decode(q, k, v, 4, 2, 0.3)
    b = oracle.attn_decode(q, k[:, perm], v[:, perm], 4, 2, 0.3)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


def test_attn_brute_force_two_positions():
    # closed form for two positions: w1 = 1 / (1 + exp(s0 - s1)), out = (1 - w1) v0 + w1 v1
    q, k, v = _attn_rand(8, 1, 2, 8, 1)
    scale = 0.5
    qf, kf, vf = (synth.bf16_bits_to_f32(a).astype(np.float64) for a in (q, k, v))
    s0, s1 = scale * qf[0] @ kf[0, 0], scale * qf[0] @ kf[0, 1]
    w1 = 1.0 / (1.0 + np.exp(s0 - s1))
    out = oracle.attn_decode(q, k, v, 1, 1, scale)
    np.testing.assert_allclose(out[0], (1 - w1) * vf[0, 0] + w1 * vf[0, 1], rtol=1e-13)


def test_attn_inputs_recipe_has_hot_positions():
    q, k, v = synth.attn_inputs(300, seed=1)
    assert q.shape == (16, 256) and k.shape == (2, 300, 256) and v.shape == k.shape
    qf = synth.bf16_bits_to_f32(q).astype(np.float64)
    kf = synth.bf16_bits_to_f32(k).astype(np.float64)
    s = np.einsum("hd,htd->ht", qf.reshape(2, 8, 256).mean(axis=1), kf) / 16.0
    assert (s > 6).sum(axis=1).tolist() == [16, 16] and np.abs(s[s < 6]).max() < 6


# ---- Gated DeltaNet recurrence ---------------------------------------------------------
# What it computes: a fixed-size matrix state per head, kept in part by a learned gate and
# written by a delta update from the current token ("Qwen creates three distinct workload
# shapes", "Keep recurrent state on chip"). Reading: the gated delta rule
# S_t = alpha S_{t-1} + beta (v - alpha S_{t-1} k) k^T, o_t = S_t q_t.

def _gdn_rand(seed, T, n_k, n_v, d_k, d_v):
    rng = np.random.default_rng(seed)
    q = bf16(rng.standard_normal((T, n_k, d_k)) * 0.3)
    k = bf16(rng.standard_normal((T, n_k, d_k)) * 0.3)
    v = bf16(rng.standard_normal((T, n_v, d_v)))
    a = rng.uniform(0.5, 1.0, (T, n_v)).astype(np.float32)
    b = rng.uniform(0.0, 1.0, (T, n_v)).astype(np.float32)
    s0 = rng.standard_normal((n_v, d_v, d_k))
    return q, k, v, a, b, s0


def _f(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def test_gdn_keep_all_write_nothing_reads_the_initial_state():
    q, k, v, a, b, s0 = _gdn_rand(1, 9, 2, 4, 8, 6)
    out, st = oracle.gdn_scan(q, k, v, np.ones_like(a), np.zeros_like(b), 2, 4, s0)
    qf = np.repeat(_f(q), 2, axis=1)                       # value head j reads key head j // 2
    np.testing.assert_allclose(out, np.einsum("jde,tje->tjd", s0, qf), rtol=1e-13, atol=1e-13)
    assert np.array_equal(st, s0)


def test_gdn_zero_gate_forgets_the_past():
    # alpha = 0: S_t = beta v_t k_t^T, so o_t = beta (k_t . q_t) v_t whatever came before
    q, k, v, a, b, s0 = _gdn_rand(2, 7, 1, 2, 8, 5)
    out, _ = oracle.gdn_scan(q, k, v, np.zeros_like(a), b, 1, 2, s0)
    kq = np.einsum("te,te->t", _f(k)[:, 0], _f(q)[:, 0])
    ref = b[:, :, None] * kq[:, None, None] * _f(v)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-14)


def test_gdn_full_write_recalls_the_value_under_its_key():
    # beta = 1 with a unit key: S_t k_t = v_t exactly, whatever the state and gate were
    T, d_k, d_v = 12, 8, 6
    rng = np.random.default_rng(3)
    k = np.zeros((T, 1, d_k), dtype=np.float32)
    k[np.arange(T), 0, rng.integers(0, d_k, T)] = 1.0        # one-hot keys, exact in bf16
    kb = bf16(k)
    v = bf16(rng.standard_normal((T, 1, d_v)))
    a = rng.uniform(0.3, 1.0, (T, 1)).astype(np.float32)
    out, _ = oracle.gdn_scan(kb, kb, v, a, np.ones((T, 1), np.float32), 1, 1,
                             rng.standard_normal((1, d_v, d_k)))
    np.testing.assert_allclose(out, _f(v), rtol=0, atol=1e-14)


def test_gdn_matches_the_literal_matrix_form():
    # S_t = S_{t-1} (alpha (I - beta k k^T)) + beta v k^T, o = S q, with numpy matrices
    T, n_k, n_v, d_k, d_v = 6, 1, 2, 5, 4
    q, k, v, a, b, s0 = _gdn_rand(4, T, n_k, n_v, d_k, d_v)
    out, st = oracle.gdn_scan(q, k, v, a, b, n_k, n_v, s0)
    S = s0.copy()
    for t in range(T):
        kk, qq = _f(k)[t, 0], _f(q)[t, 0]
        for j in range(n_v):
            S[j] = S[j] @ (float(a[t, j]) * (np.eye(d_k) - float(b[t, j]) * np.outer(kk, kk))) \
                + float(b[t, j]) * np.outer(_f(v)[t, j], kk)
            np.testing.assert_allclose(out[t, j], S[j] @ qq, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st, S, rtol=1e-12, atol=1e-13)


def test_gdn_value_heads_read_their_key_head():
    q, k, v, a, b, s0 = _gdn_rand(5, 5, 2, 4, 8, 3)
    base, _ = oracle.gdn_scan(q, k, v, a, b, 2, 4, s0)
    k2 = k.copy()
    k2[:, 1] = bf16(np.full((5, 8), 0.25))                   # change key head 1 only
    out, _ = oracle.gdn_scan(q, k2, v, a, b, 2, 4, s0)
    assert np.array_equal(out[:, :2], base[:, :2])
    assert not np.allclose(out[:, 2:], base[:, 2:])


def test_gdn_scan_continues_from_its_final_state():
    q, k, v, a, b, s0 = _gdn_rand(6, 20, 2, 4, 8, 6)
    full, st_full = oracle.gdn_scan(q, k, v, a, b, 2, 4, s0)
    o1, st1 = oracle.gdn_scan(q[:13], k[:13], v[:13], a[:13], b[:13], 2, 4, s0)
    o2, st2 = oracle.gdn_scan(q[13:], k[13:], v[13:], a[13:], b[13:], 2, 4, st1)
    assert np.array_equal(np.concatenate([o1, o2]), full) and np.array_equal(st2, st_full)


def test_gdn_inputs_recipe():
    q, k, v, a, b = synth.gdn_inputs(40, seed=1)
    assert q.shape == (40, 16, 128) and v.shape == (40, 32, 128) and a.shape == (40, 32)
    kn = np.linalg.norm(_f(k), axis=-1)
    qn = np.linalg.norm(_f(q), axis=-1) * np.sqrt(128)
    assert np.all(np.abs(kn - 1) < 1e-2) and np.all(np.abs(qn - 1) < 1e-2)
    assert 0.85 < a.mean() < 0.99 and np.all((a > 0) & (a < 1)) and np.all((b > 0) & (b < 1))
