"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Workloads (seeded, synthetic; shapes of the Qwen3.6-35B-A3B MoE layer described in
"Optimizing On-Device Inference for Apple Silicon", sections "Qwen creates three
distinct workload shapes" and "Dequantize weights during matrix multiplication"):
  - fp32 layer, T=64, H=128, I=64, E=256, k=8, one shared expert;
  - int4 g64 layer, H=2048, I=512, E=256, k=8, one shared expert: batch-1 decode
    tokens, ragged prefill sizes, T=4096 with near-uniform routing and with Zipf-skewed
    routing;
  - small int4 layers for edge cases (T=1, ragged tails, no shared expert).
Bar: routing ids/weights exact off the tie window, grouping bit-exact, outputs within
1e-4 (fp32) or 2e-2 (bf16) of the output RMS.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from parity_util import (BF16_TOL, F32_TOL, check_grouping, check_routing, delta_for,
                         rel_err, to_np)
from routed_expert_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def M():
    from routed_expert_amd import moe
    moe.lib()
    return moe


@pytest.fixture(scope="module")
def tiny(M):
    layer, x = synth.tiny_config(0)
    return layer, x, M.DeviceLayer.from_host(layer, DEV)


@pytest.fixture(scope="module")
def big(M):
    layer = synth.decode_layer(0)
    return layer, M.DeviceLayer.from_host(layer, DEV)


@pytest.fixture(scope="module")
def skewed(M):
    layer = synth.skewed_layer(0)
    return layer, M.DeviceLayer.from_host(layer, DEV)


def bf16_dev(M, bits):
    return M.bf16_from_bits(bits, DEV)


def y_np(y):
    return y.float().cpu().numpy()


def announce(msg):
    print(f"\n[case] {msg}", flush=True)


# ---- fp32 tiny layer ------------------------------------------------------------------------

def test_tiny_prefill_fp32(M, tiny):
    layer, x, dl = tiny
    announce("moe_prefill fp32 T=64 H=128 I=64 E=256 k=8 S=1 seed 0")
    buf = M.route_buffers(dl, 64, DEV)
    y = M.moe_prefill(dl, torch.from_numpy(x).to(DEV), route_out=buf)
    torch.cuda.synchronize()
    g = to_np(buf)
    assert check_routing(layer, x, g["topk_ids"], g["topk_w"], delta_for(128)) == 0
    check_grouping(layer, g)
    assert rel_err(y.cpu().numpy(), oracle.moe(layer, x)) <= F32_TOL


def test_tiny_decode_fp32(M, tiny):
    layer, x, dl = tiny
    announce("moe_decode fp32 tokens 0..15 of the T=64 fp32 layer")
    ws = M.workspace(dl, 1)
    ref = oracle.moe(layer, x[:16])
    for t in range(16):
        y = M.moe_decode(dl, torch.from_numpy(x[t:t + 1]).to(DEV), ws=ws)
        assert rel_err(y.cpu().numpy()[0], ref[t]) <= F32_TOL, t


def test_tiny_route_api(M, tiny):
    layer, x, dl = tiny
    announce("moe_route fp32 T=64")
    g = to_np(M.moe_route(dl, torch.from_numpy(x).to(DEV)))
    assert check_routing(layer, x, g["topk_ids"], g["topk_w"], delta_for(128)) == 0
    check_grouping(layer, g)


# ---- int4 decode ----------------------------------------------------------------------------

def test_decode_int4_tokens(M, big):
    # every one of the decode workload's 1000 tokens, each compared in full
    layer, dl = big
    n = 1000
    announce(f"moe_decode int4 H=2048 I=512 E=256 k=8 S=1 layer seed 0, tokens 0..{n - 1}")
    xs = np.concatenate([synth.decode_token(t) for t in range(n)])
    _, _, margin = oracle.route(layer, xs)
    ref = oracle.moe(layer, xs)
    ws = M.workspace(dl, 1)
    ys = torch.empty((n, 2048), dtype=torch.bfloat16, device=DEV)
    xd = bf16_dev(M, xs)
    for t in range(n):
        M.moe_decode(dl, xd[t:t + 1], y=ys[t:t + 1], ws=ws)
    got = y_np(ys)
    sure = margin >= delta_for(2048)
    errs = [rel_err(got[t], ref[t]) for t in np.flatnonzero(sure)]
    assert sure.sum() >= n - 5
    assert max(errs) <= BF16_TOL, max(errs)


def test_decode_residual_alias_and_determinism(M, big):
    layer, dl = big
    announce("moe_decode int4 residual (aliasing y) and repeat determinism, token 3")
    xb = synth.decode_token(3)
    x = bf16_dev(M, xb)
    ws = M.workspace(dl, 1)
    y1 = M.moe_decode(dl, x, ws=ws)
    y2 = M.moe_decode(dl, x, ws=ws)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    r = bf16_dev(M, synth.bf16_activations(77, (1, 2048)))
    yr = r.clone()
    M.moe_decode(dl, x, y=yr, residual=yr, ws=ws)
    ref = oracle.moe(layer, xb)[0] + synth.bf16_bits_to_f32(
        synth.bf16_activations(77, (1, 2048)))[0]
    assert rel_err(y_np(yr)[0], ref) <= BF16_TOL


# ---- int4 prefill ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 5, 300])
def test_prefill_int4_full_compare(M, big, T):
    layer, dl = big
    announce(f"moe_prefill int4 full-shape layer T={T}")
    xb = synth.prefill_x(T, seed=11)
    buf = M.route_buffers(dl, T, DEV)
    y = M.moe_prefill(dl, bf16_dev(M, xb), route_out=buf)
    torch.cuda.synchronize()
    g = to_np(buf)
    unsure = check_routing(layer, xb, g["topk_ids"], g["topk_w"], delta_for(2048))
    check_grouping(layer, g)
    ref = oracle.moe(layer, xb)
    _, _, margin = oracle.route(layer, xb)
    sure = margin >= delta_for(2048)
    assert unsure <= max(2, T // 100)
    assert rel_err(y_np(y)[sure], ref[sure]) <= BF16_TOL


def _prefill_big(M, layer, dl, seed, T=4096, n_sample=None):
    """One prefill call at size T; every row whose routing is off the tie window is compared
    with the oracle (n_sample: only that many seeded rows plus the edges instead)."""
    xb = synth.prefill_x(T, seed=seed)
    buf = M.route_buffers(dl, T, DEV)
    y = M.moe_prefill(dl, bf16_dev(M, xb), route_out=buf)
    torch.cuda.synchronize()
    g = to_np(buf)
    unsure = check_routing(layer, xb, g["topk_ids"], g["topk_w"], delta_for(2048))
    check_grouping(layer, g)
    _, _, margin = oracle.route(layer, xb)
    if n_sample is None:
        sample = np.arange(T)
    else:
        rng = np.random.default_rng(seed + 1)
        sample = np.unique(np.concatenate([[0, 1, 127, 128, T - 33, T - 1],
                                           rng.choice(T, n_sample, replace=False)]))
    sample = sample[margin[sample] >= delta_for(2048)]
    ref = oracle.moe(layer, xb[sample])
    got = y_np(y)[sample]
    return g, unsure, rel_err(got, ref), y


def tile_cases(c):
    """Group sizes by the tile shapes they take at 128-row tiles: a remainder of 1..32 rows
    joined to the last full tile (a 160-row tile), the same behind further full tiles, a
    partial last tile above 32 rows, groups of one partial tile, exact multiples of 128."""
    r = c % 128
    merged = (c > 128) & (r > 0) & (r <= 32)
    return {"merged": int(merged.sum()), "merged_multi": int((merged & (c > 256)).sum()),
            "partial": int(((c > 128) & (r > 32)).sum()), "single": int(((c > 0) & (c < 128)).sum()),
            "multiple": int(((c > 0) & (r == 0)).sum())}


def test_prefill_uniform_4096(M, big):
    layer, dl = big
    announce("moe_prefill int4 T=4096 near-uniform routing, x seed 2")
    g, unsure, err, _ = _prefill_big(M, layer, dl, 2)
    c = g["counts"]
    assert c.sum() == 8 * 4096 and c.min() > 0
    # the call exercises merged 160-row tiles, partial and single tiles, and full tiles alone
    cases = tile_cases(c)
    assert cases["merged"] >= 50 and cases["partial"] >= 1 and cases["single"] >= 50, cases
    assert cases["multiple"] >= 1, cases
    assert unsure <= 20
    assert err <= BF16_TOL, err


def test_prefill_skewed_4096(M, skewed):
    layer, dl = skewed
    announce("moe_prefill int4 T=4096 Zipf(1.1)-skewed routing, x seed 2")
    g, unsure, err, _ = _prefill_big(M, layer, dl, 2)
    c = g["counts"]
    assert c.max() > 500 and (c <= 5).sum() >= 32   # very uneven groups, some empty-ish
    # merged tiles behind several full tiles, partial last tiles of large groups
    cases = tile_cases(c)
    assert cases["merged_multi"] >= 3 and cases["partial"] >= 10, cases
    assert unsure <= 20
    assert err <= BF16_TOL, err


@pytest.mark.timeout(600)
def test_prefill_uniform_8192(M, big):
    # twice the workload's prompt: most experts fill two or more 128-row tiles, so merged
    # remainders sit behind several full tiles; every row against the oracle
    layer, dl = big
    announce("moe_prefill int4 T=8192 near-uniform routing, x seed 13")
    g, unsure, err, _ = _prefill_big(M, layer, dl, 13, T=8192)
    c = g["counts"]
    assert c.sum() == 8 * 8192
    cases = tile_cases(c)
    assert cases["merged_multi"] >= 20 and cases["partial"] >= 20, cases
    assert unsure <= 40
    assert err <= BF16_TOL, err


def test_prefill_shared_expert_merged_tail(M, big):
    # T = 4100 = 32 x 128 + 4: the shared expert's last 4 rows join its last full tile (a
    # 132-row tile); every row against the oracle
    layer, dl = big
    announce("moe_prefill int4 T=4100 (shared expert's 4-row remainder merged), x seed 12")
    g, unsure, err, _ = _prefill_big(M, layer, dl, 12, T=4100)
    assert g["counts"].sum() == 8 * 4100
    assert unsure <= 20
    assert err <= BF16_TOL, err


def test_prefill_skewed_ragged_1000(M, skewed):
    # the router bias with a token count that is not a multiple of 64 (the last routing
    # block holds 40 tokens): every token's routing and output against the oracle
    layer, dl = skewed
    T = 1000
    announce(f"moe_prefill int4 T={T} Zipf(1.1)-skewed routing, x seed 5")
    g, unsure, err, _ = _prefill_big(M, layer, dl, 5, T=T)
    assert g["counts"].sum() == 8 * T
    assert unsure <= 10
    assert err <= BF16_TOL, err


def test_prefill_ragged_12000(M, big):
    # one call well past the benchmark size whose token count is not a multiple of 64:
    # 188 count blocks, the last one half full, and a tile map of about 860 tiles
    layer, dl = big
    T = 12000
    announce(f"moe_prefill int4 T={T} near-uniform routing, x seed 3")
    g, unsure, err, _ = _prefill_big(M, layer, dl, 3, T=T, n_sample=128)
    c = g["counts"]
    assert c.sum() == 8 * T and c.min() > 0
    assert unsure <= 60
    assert err <= BF16_TOL, err


def test_prefill_determinism_and_residual(M, big):
    layer, dl = big
    T = 700
    announce(f"moe_prefill int4 T={T} repeat determinism and residual")
    xb = synth.prefill_x(T, seed=21)
    x = bf16_dev(M, xb)
    ws = M.workspace(dl, T)
    y1 = M.moe_prefill(dl, x, ws=ws)
    y2 = M.moe_prefill(dl, x, ws=ws)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    rb = synth.bf16_activations(22, (T, 2048))
    yr = bf16_dev(M, rb)
    M.moe_prefill(dl, x, y=yr, residual=yr, ws=ws)
    # y + r evaluated in fp32 then rounded once: compare every row with the unrounded sum
    _, _, margin = oracle.route(layer, xb)
    sure = margin >= delta_for(2048)
    ref = oracle.moe(layer, xb) + synth.bf16_bits_to_f32(rb)
    assert rel_err(y_np(yr)[sure], ref[sure]) <= BF16_TOL


def test_prefill_residual_without_shared_expert(M):
    # no shared expert: the weighted routed rows are summed by the separate combine kernel,
    # which also adds the residual (here aliasing y); every row compared
    layer = synth.make_int4_layer(540, n_experts=64, top_k=4, n_shared=0)
    dl = M.DeviceLayer.from_host(layer, DEV)
    T = 300
    announce(f"moe_prefill int4 H=2048 E=64 k=4 S=0 T={T} with residual")
    xb = synth.prefill_x(T, seed=41)
    rb = synth.bf16_activations(42, (T, 2048))
    yr = bf16_dev(M, rb)
    M.moe_prefill(dl, bf16_dev(M, xb), y=yr, residual=yr)
    torch.cuda.synchronize()
    _, _, margin = oracle.route(layer, xb)
    sure = margin >= delta_for(2048)
    assert sure.sum() >= T - 3
    ref = oracle.moe(layer, xb) + synth.bf16_bits_to_f32(rb)
    assert rel_err(y_np(yr)[sure], ref[sure]) <= BF16_TOL


def test_prefill_rows_match_decode(M, big):
    layer, dl = big
    announce("prefill rows vs per-token decode, T=16")
    xb = synth.prefill_x(16, seed=31)
    yp = y_np(M.moe_prefill(dl, bf16_dev(M, xb)))
    ws = M.workspace(dl, 1)
    _, _, margin = oracle.route(layer, xb)
    for t in range(16):
        if margin[t] < delta_for(2048):
            continue
        yd = y_np(M.moe_decode(dl, bf16_dev(M, xb[t:t + 1]), ws=ws))[0]
        assert rel_err(yp[t], yd) <= BF16_TOL


# ---- small int4 layers: edge cases ----------------------------------------------------------

@pytest.mark.parametrize("T,E,k,S", [(1, 64, 4, 1), (63, 64, 4, 1), (65, 64, 4, 0),
                                     (129, 32, 8, 1), (257, 16, 1, 1)])
def test_small_int4_layers(M, T, E, k, S):
    announce(f"moe_prefill/moe_decode small int4 H=256 I=128 E={E} k={k} S={S} T={T}")
    layer = synth.make_int4_layer(100 + T, hidden=256, inter=128, n_experts=E, top_k=k,
                                  n_shared=S, router_std=0.1)
    dl = M.DeviceLayer.from_host(layer, DEV)
    xb = synth.bf16_activations(200 + T, (T, 256))
    buf = M.route_buffers(dl, T, DEV)
    y = M.moe_prefill(dl, bf16_dev(M, xb), route_out=buf)
    torch.cuda.synchronize()
    g = to_np(buf)
    check_routing(layer, xb, g["topk_ids"], g["topk_w"], delta_for(256))
    check_grouping(layer, g)
    ref = oracle.moe(layer, xb)
    _, _, margin = oracle.route(layer, xb)
    sure = margin >= delta_for(256)
    assert rel_err(y_np(y)[sure], ref[sure]) <= BF16_TOL
    t = int(np.argmax(margin))
    yd = M.moe_decode(dl, bf16_dev(M, xb[t:t + 1]))
    assert rel_err(y_np(yd)[0], ref[t]) <= BF16_TOL


def _tile_reference(q, sc, bi, rows, K, inter, gate_up):
    """Tiled layout of moe_pack_weights written out with numpy reshapes (layout only)."""
    n = q.shape[0]
    order = np.arange(rows)
    if gate_up:  # block j: gate rows 32j..32j+31, then up rows 32j..32j+31
        order = np.stack([order[:inter].reshape(-1, 32), order[inter:].reshape(-1, 32)],
                         1).reshape(-1)
    qb = q[:, order].reshape(n, rows // 64, 64, K // 64, 32).transpose(0, 1, 3, 2, 4)
    ng = K // 64
    ng4 = (ng + 3) // 4 * 4
    pairs = np.zeros((n, rows, ng4, 2), np.uint16)
    pairs[:, :, :ng, 0], pairs[:, :, :ng, 1] = sc, bi
    sb = pairs[:, order].reshape(n, rows // 64, 64, ng4 // 4, 4, 2).transpose(0, 1, 3, 2, 4, 5)
    return np.ascontiguousarray(qb).reshape(-1), np.ascontiguousarray(sb).reshape(-1)


@pytest.mark.parametrize("H,I", [(256, 128), (512, 384)])
def test_pack_weights_layout(M, H, I):
    announce(f"moe_pack_weights H={H} I={I} E=4 S=1")
    layer = synth.make_int4_layer(7, hidden=H, inter=I, n_experts=4, top_k=2, n_shared=1)
    dl = M.DeviceLayer.from_host(layer, DEV)
    torch.cuda.synchronize()
    buf = dl.t["tiled"].cpu().numpy()
    base = dl.t["tiled"].data_ptr()
    d = dl.desc
    for qa, sa, ba, rows, K, gu, tp, sp in (
            (layer.w13_q, layer.w13_s, layer.w13_b, 2 * I, H, True, d.w13_t, d.w13_tsb),
            (layer.w2_q, layer.w2_s, layer.w2_b, H, I, False, d.w2_t, d.w2_tsb)):
        want_q, want_sb = _tile_reference(qa, sa, ba, rows, K, I, gu)
        got_q = buf[tp - base: tp - base + want_q.size]
        got_sb = buf[sp - base: sp - base + 2 * want_sb.size].view(np.uint16)
        assert np.array_equal(got_q, want_q)
        assert np.array_equal(got_sb, want_sb)
    # router planes: hi = fp16(w), lo = fp16((w - hi) * 2048), so hi + lo / 2048 is w to
    # 2^-22 relative (2^-25 absolute where w is an fp16 subnormal), stored in operand order
    # [E_pad/32][H/16][plane][lane 64][8]: lane l of (c, s) holds expert 32c + l % 32 at
    # k = 16 s + 8 (l // 32) .. +7, experts past E zero
    E = layer.n_experts
    ep = -(-E // 128) * 128
    frag = buf[d.router_planes - base: d.router_planes - base + 2 * ep * H * 2].view(np.float16)
    frag = frag.reshape(ep // 32, H // 16, 2, 2, 32, 8)       # c, s, plane, l//32, l%32, j
    planes = frag.transpose(2, 0, 4, 1, 3, 5).reshape(2, ep, H)  # plane, expert, k
    hi, lo = planes[0], planes[1]
    assert np.all(hi[E:] == 0) and np.all(lo[E:] == 0)
    hi, lo = hi[:E], lo[:E]
    w = layer.router_w
    assert np.array_equal(hi, w.astype(np.float16))
    assert np.array_equal(lo, ((w - hi.astype(np.float32)) * 2048).astype(np.float16))
    err = np.abs(hi.astype(np.float64) + lo.astype(np.float64) / 2048 - w.astype(np.float64))
    assert np.all(err <= 2.0 ** -22 * np.abs(w) + 2.0 ** -25)


def test_prefill_small_layer_padded_scale_blocks(M):
    # I = 384: the down GEMM has 6 K steps, so its last scale block is half padding
    announce("moe_prefill int4 H=512 I=384 E=16 k=4 S=1 T=77")
    layer = synth.make_int4_layer(55, hidden=512, inter=384, n_experts=16, top_k=4,
                                  n_shared=1, router_std=0.1)
    dl = M.DeviceLayer.from_host(layer, DEV)
    xb = synth.bf16_activations(56, (77, 512))
    y = M.moe_prefill(dl, bf16_dev(M, xb))
    torch.cuda.synchronize()
    ref = oracle.moe(layer, xb)
    _, _, margin = oracle.route(layer, xb)
    sure = margin >= delta_for(512)
    assert sure.sum() >= 70
    assert rel_err(y_np(y)[sure], ref[sure]) <= BF16_TOL


@pytest.mark.parametrize("E,k,S", [(64, 4, 0), (32, 1, 1), (128, 8, 0)])
def test_model_width_layers_other_routing(M, E, k, S):
    # hidden 2048 / intermediate 512 takes the three-kernel decode path for any E <= 256,
    # k + S <= 9: idle top-k slots, no shared expert, fewer router workgroups
    announce(f"moe_decode/moe_prefill int4 H=2048 I=512 E={E} k={k} S={S}")
    layer = synth.make_int4_layer(500 + E + k, n_experts=E, top_k=k, n_shared=S)
    dl = M.DeviceLayer.from_host(layer, DEV)
    xb = synth.bf16_activations(600 + E, (70, 2048))
    ref = oracle.moe(layer, xb)
    _, _, margin = oracle.route(layer, xb)
    sure = margin >= delta_for(2048)
    for t in np.flatnonzero(sure)[:6]:
        yd = M.moe_decode(dl, bf16_dev(M, xb[t:t + 1]))
        torch.cuda.synchronize()
        assert rel_err(y_np(yd)[0], ref[t]) <= BF16_TOL, t
    buf = M.route_buffers(dl, 70, DEV)
    y = M.moe_prefill(dl, bf16_dev(M, xb), route_out=buf)
    torch.cuda.synchronize()
    g = to_np(buf)
    check_routing(layer, xb, g["topk_ids"], g["topk_w"], delta_for(2048))
    check_grouping(layer, g)
    assert rel_err(y_np(y)[sure], ref[sure]) <= BF16_TOL


@pytest.mark.parametrize("which,T", [("uniform", 4096), ("skewed", 4096), ("uniform", 777),
                                     ("skewed", 20000)])
def test_route_api_int4_full_width(M, big, skewed, which, T):
    # moe_route alone on the model-width layer (bf16 activations, the MFMA router): ids and
    # weights against the oracle off the tie window, the grouping bit for bit, and the same
    # routing as moe_prefill's route_out on the same input. T = 20,000 is 313 routing blocks:
    # the grouping counts per chunk of 64 blocks (five chunks, the last one partial)
    layer, dl = big if which == "uniform" else skewed
    announce(f"moe_route int4 H=2048 E=256 k=8 {which} T={T}")
    xb = synth.prefill_x(T, seed=31)
    xd = bf16_dev(M, xb)
    g = to_np(M.moe_route(dl, xd))
    buf = M.route_buffers(dl, T, DEV)
    M.moe_prefill(dl, xd, route_out=buf)
    torch.cuda.synchronize()
    gp = to_np(buf)
    unsure = check_routing(layer, xb, g["topk_ids"], g["topk_w"], delta_for(2048))
    assert unsure <= max(2, T // 200)
    check_grouping(layer, g)
    for key in g:
        assert np.array_equal(g[key], gp[key]), key


def test_bias_only_routing_fills_eight_experts(M, big):
    # Zero router weights and a strictly decreasing router bias: every logit is its bias
    # exactly, so every token selects experts 0..7 with the weights softmax(b_0..b_7) (the
    # top-k and its renormalisation pinned by the definition, no rounding in the logits).
    # At T = 4096 those eight experts hold all 32,768 routed rows (32 full tiles each) and
    # the other 248 none: the far end of uneven expert groups ("Qwen creates three distinct
    # workload shapes"). Rows of x = 0 are mixed in; with no biases inside the experts their
    # output is exactly zero. Every row of the prefill, the small-T path and decode tokens
    # are compared with the oracle.
    layer0, _ = big
    E = layer0.n_experts
    layer = dataclasses.replace(layer0, router_w=np.zeros_like(layer0.router_w),
                                router_b=(-0.25 * np.arange(E)).astype(np.float32))
    dl = M.DeviceLayer.from_host(layer, DEV)
    T = 4096
    announce(f"moe_prefill/moe_decode int4 bias-only routing, T={T}, all rows to experts 0..7")
    xb = synth.prefill_x(T, seed=23)
    zero_rows = np.array([0, 17, 2048, T - 1])
    xb[zero_rows] = 0
    buf = M.route_buffers(dl, T, DEV)
    y = M.moe_prefill(dl, bf16_dev(M, xb), route_out=buf)
    y5 = M.moe_prefill(dl, bf16_dev(M, xb[:5]))          # small-T kernels
    ws = M.workspace(dl, 1)
    dec = [M.moe_decode(dl, bf16_dev(M, xb[t:t + 1]), ws=ws) for t in (0, 1, 2)]
    torch.cuda.synchronize()
    g = to_np(buf)
    assert np.array_equal(g["topk_ids"], np.tile(np.arange(8, dtype=g["topk_ids"].dtype), (T, 1)))
    assert check_routing(layer, xb, g["topk_ids"], g["topk_w"], delta_for(2048)) == 0
    check_grouping(layer, g)
    assert np.array_equal(g["counts"], np.r_[np.full(8, T), np.zeros(E - 8)].astype(g["counts"].dtype))
    ref = oracle.moe(layer, xb)
    got = y_np(y)
    assert np.all(got[zero_rows] == 0) and np.all(ref[zero_rows] == 0)
    assert rel_err(got, ref) <= BF16_TOL
    assert rel_err(y_np(y5), ref[:5]) <= BF16_TOL
    assert np.all(y_np(y5)[0] == 0)
    assert np.all(y_np(dec[0]) == 0)
    for t in (1, 2):
        assert rel_err(y_np(dec[t])[0], ref[t]) <= BF16_TOL, t


@pytest.mark.timeout(600)
def test_prefill_beyond_32bit_offsets_runs_as_consecutive_calls(M, big):
    # x of more than 2^32 bytes: the library runs the call as consecutive calls of at most
    # t_max tokens (the GEMMs gather rows by 32-bit byte offsets). T = t_max + 200 with
    # t_max = 1,048,512 at hidden 2048 (about 62 GB on the device). x is drawn on the GPU from
    # a seeded generator; 40 rows (both sides of the split, the first and last rows, seeded
    # rows between) against the oracle, and the rows around the split bit for bit against a
    # separate 128-token call (a token's result does not depend on the rest of its call)
    layer, dl = big
    t_max = (0xFFFFFFFF // (2 * 2048)) & ~63
    T = t_max + 200
    announce(f"moe_prefill int4 T={T} (x beyond 2^32 bytes, split at {t_max})")
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    x = torch.randn((T, 2048), generator=g, device=DEV).to(torch.bfloat16)
    y = M.moe_prefill(dl, x)
    near = x[t_max - 64:t_max + 64].clone()
    y_near = M.moe_prefill(dl, near)
    torch.cuda.synchronize()
    rng = np.random.default_rng(78)
    rows = np.unique(np.concatenate([[0, t_max - 2, t_max - 1, t_max, t_max + 1, T - 1],
                                     rng.choice(T, 34, replace=False)]))
    rows_d = torch.from_numpy(rows).to(DEV)
    xb = x[rows_d].view(torch.int16).cpu().numpy().view(np.uint16)
    got = y_np(y[rows_d])
    _, _, margin = oracle.route(layer, xb)
    sure = margin >= delta_for(2048)
    assert sure.sum() >= len(rows) - 2
    ref = oracle.moe(layer, xb)
    assert rel_err(got[sure], ref[sure]) <= BF16_TOL
    assert torch.equal(y[t_max - 64:t_max + 64].view(torch.int16), y_near.view(torch.int16))
    del x, y
    torch.cuda.empty_cache()


def test_empty_prefill_is_noop(M, big):
    _, dl = big
    announce("moe_prefill T=0")
    x = torch.empty((0, 2048), dtype=torch.bfloat16, device=DEV)
    y = M.moe_prefill(dl, x, ws=M.workspace(dl, 1))
    assert y.shape == (0, 2048)


def test_rmsnorm(M):
    announce("moe_rmsnorm bf16 and fp32, T=33 H=2048, H=320 (a partial 2048 stretch), "
             "H=4096/6144/8192 T=9 in place and misaligned")
    eps = float(np.float32(1e-6))
    for H in (2048, 320):
        hb = synth.bf16_activations(41 + H, (33, H))
        out = M.moe_rmsnorm(bf16_dev(M, hb), eps)
        torch.cuda.synchronize()
        # fp64 arithmetic rounded once: the bits of the oracle's bf16 rounding
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, oracle.round_bf16(oracle.rmsnorm(hb, eps)))
    # the one-wave-per-row kernel at every width it takes (2048 * n up to 8192, a row count
    # that leaves a partial workgroup), in place, and the same rows at an address that is not
    # 8-byte aligned (the 512-thread kernel): all give the oracle's bits
    for H in (4096, 6144, 8192):
        hb = synth.bf16_activations(47 + H, (9, H))
        want = oracle.round_bf16(oracle.rmsnorm(hb, eps))
        hd = bf16_dev(M, hb)
        out = M.moe_rmsnorm(hd, eps)
        M.moe_rmsnorm(hd, eps, out=hd)
        flat = torch.zeros(9 * H + 1, dtype=torch.bfloat16, device=DEV)
        shifted = flat[1:].view(9, H)
        shifted.copy_(bf16_dev(M, hb))
        M.moe_rmsnorm(shifted, eps, out=shifted)
        torch.cuda.synchronize()
        for got in (out, hd, shifted):
            assert np.array_equal(got.contiguous().view(torch.int16).cpu().numpy().view(np.uint16),
                                  want), H
    # degenerate rows on both kernels (H = 2048: one wave per row; H = 320: the 512-thread
    # kernel): all zeros (the output is zero), one non-zero element, magnitudes near the bf16
    # maximum (their squares overflow fp32, not fp64), bf16 subnormal inputs, alternating
    # signs, and a row whose outputs land on the bf16 subnormal grid or round to a signed zero
    for H in (2048, 320):
        rows = np.zeros((6, H), np.float32)
        rows[1, H // 3] = -3.0
        rows[2] = np.where(np.arange(H) % 2, 3.0e38, -2.5e38)
        rows[3] = 1.0e-39 * (1 + np.arange(H) % 7)
        rows[4] = np.where(np.arange(H) % 3, 1.0, -1.0)
        rows[5, :9] = [1.0e30, 1.0e-30, -7.0, 0.0, 2.0, -1.0e-30, 1.0e-10, -2.0e-12, 3.0e-9]
        hb = synth.f32_to_bf16_bits(rows)
        want = oracle.round_bf16(oracle.rmsnorm(hb, eps))
        assert not np.any(want[0]) and np.any(want[3])
        assert want[5, 5] == 0x8000 and 0 < want[5, 6] < 0x80 and want[5, 7] >> 15
        got = M.moe_rmsnorm(bf16_dev(M, hb), eps)
        torch.cuda.synchronize()
        assert np.array_equal(got.view(torch.int16).cpu().numpy().view(np.uint16), want), H
    hf = np.random.default_rng(42).standard_normal((33, 2048)).astype(np.float32)
    outf = M.moe_rmsnorm(torch.from_numpy(hf).to(DEV), eps)
    ref = oracle.rmsnorm(hf, eps)
    # one rounding to fp32 of the fp64 result: within half an fp32 ulp (plus fp64 noise)
    assert np.all(np.abs(outf.cpu().numpy() - ref) <= 2.0 ** -24 * np.abs(ref) * 1.0001)
