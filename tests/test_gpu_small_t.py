"""GPU parity of the small-T path: moe_prefill with 2..8 tokens and no routing output runs
the decode-style kernels (router, top-k + union of the tokens' experts + gate/up, output),
reading each selected expert's weights once for all the tokens that chose it.

Workloads: the int4 layer of the model's width ("Optimizing On-Device Inference for Apple
Silicon", sections "Qwen creates three distinct workload shapes" and "Optimize the one-row
weight path"), the Zipf-skewed variant, and model-width layers with other E / k / S.
Bar: every token whose top-k boundary is at least the tie window wide matches the oracle
within 2e-2 of the output RMS; the path is deterministic.
"""
import numpy as np
import pytest
import torch

import oracle
from parity_util import BF16_TOL, delta_for, rel_err
from routed_expert_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def M():
    from routed_expert_amd import moe
    moe.lib()
    return moe


@pytest.fixture(scope="module")
def big(M):
    layer = synth.decode_layer(0)
    return layer, M.DeviceLayer.from_host(layer, DEV)


def announce(msg):
    print(f"\n[small-T] {msg}", flush=True)


def check(layer, xb, y, min_sure=None):
    ref = oracle.moe(layer, xb)
    _, _, margin = oracle.route(layer, xb)
    sure = margin >= delta_for(layer.hidden)
    assert sure.sum() >= (min_sure if min_sure is not None else max(1, len(xb) - 1))
    got = y.float().cpu().numpy()
    assert rel_err(got[sure], ref[sure]) <= BF16_TOL, rel_err(got[sure], ref[sure])


@pytest.mark.parametrize("T", [1, 2, 3, 5, 8])
def test_small_t_full_width(M, big, T):
    layer, dl = big
    announce(f"moe_prefill int4 H=2048 E=256 k=8 S=1 T={T}")
    xb = synth.prefill_x(T, seed=40 + T)
    y = M.moe_prefill(dl, M.bf16_from_bits(xb, DEV))
    torch.cuda.synchronize()
    check(layer, xb, y, min_sure=T if T == 1 else None)


def test_small_t_residual_alias_and_determinism(M, big):
    layer, dl = big
    T = 6
    announce(f"moe_prefill int4 T={T}: repeat determinism, residual aliasing y")
    xb = synth.prefill_x(T, seed=61)
    x = M.bf16_from_bits(xb, DEV)
    y1 = M.moe_prefill(dl, x)
    y2 = M.moe_prefill(dl, x)
    rb = synth.bf16_activations(62, (T, 2048))
    r = M.bf16_from_bits(rb, DEV)
    M.moe_prefill(dl, x, y=r, residual=r)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    ref = oracle.moe(layer, xb) + synth.bf16_bits_to_f32(rb)
    _, _, margin = oracle.route(layer, xb)
    sure = margin >= delta_for(2048)
    assert rel_err(r.float().cpu().numpy()[sure], ref[sure]) <= BF16_TOL


def test_small_t_shared_experts_across_tokens(M, big):
    # every token the same: the union is one token's 8 experts, each used by all 8 tokens
    layer, dl = big
    announce("moe_prefill int4 T=8, eight copies of one token")
    xb = np.repeat(synth.prefill_x(1, seed=71), 8, axis=0)
    y = M.moe_prefill(dl, M.bf16_from_bits(xb, DEV))
    torch.cuda.synchronize()
    yn = y.view(torch.int16).cpu().numpy()
    assert all(np.array_equal(yn[0], yn[i]) for i in range(8))
    check(layer, xb, y, min_sure=8)   # (this token's top-k boundary is 8.7e-3 wide)


def test_small_t_skewed(M):
    announce("moe_prefill int4 T=8 Zipf(1.1)-skewed routing")
    layer = synth.skewed_layer(0)
    dl = M.DeviceLayer.from_host(layer, DEV)
    xb = synth.prefill_x(8, seed=81)
    y = M.moe_prefill(dl, M.bf16_from_bits(xb, DEV))
    torch.cuda.synchronize()
    check(layer, xb, y)


@pytest.mark.parametrize("E,k,S", [(64, 4, 0), (32, 1, 1), (128, 8, 0)])
def test_small_t_other_routing(M, E, k, S):
    announce(f"moe_prefill int4 H=2048 I=512 E={E} k={k} S={S} T=7")
    layer = synth.make_int4_layer(90 + E + k, n_experts=E, top_k=k, n_shared=S)
    dl = M.DeviceLayer.from_host(layer, DEV)
    xb = synth.prefill_x(7, seed=91)
    y = M.moe_prefill(dl, M.bf16_from_bits(xb, DEV))
    torch.cuda.synchronize()
    check(layer, xb, y)


def test_small_t_matches_prefill_pipeline(M, big):
    # the same tokens through the routing + grouped-GEMM pipeline (asked for its routing
    # output, which the small-T path does not produce): both within the bar of each other
    layer, dl = big
    T = 8
    announce(f"small-T path vs prefill pipeline, T={T}")
    xb = synth.prefill_x(T, seed=101)
    x = M.bf16_from_bits(xb, DEV)
    ys = M.moe_prefill(dl, x)
    yp = M.moe_prefill(dl, x, route_out=M.route_buffers(dl, T, DEV))
    torch.cuda.synchronize()
    _, _, margin = oracle.route(layer, xb)
    sure = margin >= delta_for(2048)
    a, b = ys.float().cpu().numpy()[sure], yp.float().cpu().numpy()[sure]
    assert rel_err(a, b) <= BF16_TOL


def test_small_t_stack_chunk(M):
    # a 6-token prompt through two full-width layers: the chunk is a small-T call after the
    # RMSNorm kernel; each layer is checked teacher-forced against the oracle
    announce("moe_stack_forward 2 int4 layers H=2048, T=6")
    layers = [synth.decode_layer(l) for l in range(2)]
    dls = [M.DeviceLayer.from_host(L, DEV) for L in layers]
    hb = synth.bf16_activations(111, (6, 2048))
    h0 = M.bf16_from_bits(hb, DEV)
    h1 = h0.clone()
    M.moe_stack_forward(dls[:1], h1, chunk_tokens=40, eps=1e-6)
    h2 = h1.clone()
    M.moe_stack_forward(dls[1:], h2, chunk_tokens=40, eps=1e-6)
    torch.cuda.synchronize()
    for layer, hin, hout in ((layers[0], h0, h1), (layers[1], h1, h2)):
        xin = oracle.to_f64(hin.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
        xn = oracle.rmsnorm(xin, 1e-6)
        ref = xin + oracle.moe(layer, xn)
        sure = oracle.route(layer, xn)[2] >= delta_for(2048)
        assert sure.sum() >= 5
        got = oracle.to_f64(hout.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
        d = np.abs(got - ref)[sure]
        assert np.max(d) / np.sqrt(np.mean(ref[sure] ** 2)) <= BF16_TOL
