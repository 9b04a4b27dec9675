"""GPU checks of the prefill ablations (moe_prefill_ablation): the rejected designs of
"Optimizing On-Device Inference for Apple Silicon", section "Optimize sparse expert
computation" (separate dequantisation pass, host-inspected routing, smaller tiles) and a
fixed tile height without the load-adaptive tail, each rebuilt on the product kernels.

Every variant changes how the work is scheduled or where the weights are expanded, never
the arithmetic of an output row, so its y must equal moe_prefill's (grouped path, T > 8)
byte for byte; the control variant is also checked against the oracle at T <= 8, where
moe_prefill itself takes the small-T kernels.
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
    print(f"\n[ablation] {msg}", flush=True)


def same_bytes(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def variants(M):
    return [(n, v) for n, v in M.ABLATIONS.items()]


@pytest.mark.parametrize("T", [9, 1000])
def test_ablations_match_prefill_full_width(M, big, T):
    layer, dl = big
    xb = synth.prefill_x(T, seed=70 + T)
    x = M.bf16_from_bits(xb, DEV)
    rb = synth.bf16_activations(71, (T, 2048))
    r = M.bf16_from_bits(rb, DEV)
    y0 = M.moe_prefill(dl, x)
    yr0 = M.moe_prefill(dl, x, residual=r)
    for name, v in variants(M):
        announce(f"moe_prefill_ablation {name} int4 H=2048 E=256 k=8 S=1 T={T}")
        ws = M.ablation_workspace(dl, T, v, DEV)
        y = M.moe_prefill_ablation(dl, x, v, ws=ws)
        yr = M.moe_prefill_ablation(dl, x, v, residual=r, ws=ws)
        torch.cuda.synchronize()
        assert same_bytes(y, y0), name
        assert same_bytes(yr, yr0), name


def test_ablations_match_prefill_skewed_4096(M):
    # Zipf-skewed routing: experts with hundreds of rows (many full tiles) next to experts
    # with a handful (short partial tiles), the case the tile policy is about
    layer = synth.skewed_layer(0)
    dl = M.DeviceLayer.from_host(layer, DEV)
    T = 4096
    x = M.bf16_from_bits(synth.prefill_x(T, seed=2), DEV)
    y0 = M.moe_prefill(dl, x)
    for name, v in variants(M):
        announce(f"moe_prefill_ablation {name} skewed T={T}")
        y = M.moe_prefill_ablation(dl, x, v)
        torch.cuda.synchronize()
        assert same_bytes(y, y0), name


@pytest.mark.parametrize("T,E,k,S", [(77, 16, 4, 1), (300, 64, 4, 0), (129, 32, 1, 1)])
def test_ablations_small_layers(M, T, E, k, S):
    # H=512 I=384: the down GEMM's K is 6 steps (a half-padded scale block); other E, k, S
    announce(f"moe_prefill_ablation * int4 H=512 I=384 E={E} k={k} S={S} T={T}")
    layer = synth.make_int4_layer(300 + T, hidden=512, inter=384, n_experts=E, top_k=k,
                                  n_shared=S, router_std=0.1)
    dl = M.DeviceLayer.from_host(layer, DEV)
    xb = synth.bf16_activations(301 + T, (T, 512))
    x = M.bf16_from_bits(xb, DEV)
    y0 = M.moe_prefill(dl, x)
    for name, v in variants(M):
        y = M.moe_prefill_ablation(dl, x, v)
        torch.cuda.synchronize()
        assert same_bytes(y, y0), name
    ref = oracle.moe(layer, xb)
    _, _, margin = oracle.route(layer, xb)
    sure = margin >= delta_for(512)
    assert rel_err(y0.float().cpu().numpy()[sure], ref[sure]) <= BF16_TOL


@pytest.mark.parametrize("T", [1, 5])
def test_ablation_grouped_path_at_small_t(M, big, T):
    # below 9 tokens moe_prefill runs the small-T kernels; the ablations still run the
    # grouped GEMMs (one partial tile per selected expert), checked against the oracle
    layer, dl = big
    announce(f"moe_prefill_ablation * int4 full width T={T}")
    xb = synth.prefill_x(T, seed=80 + T)
    x = M.bf16_from_bits(xb, DEV)
    ys = {name: M.moe_prefill_ablation(dl, x, v) for name, v in variants(M)}
    torch.cuda.synchronize()
    for name in ys:
        assert same_bytes(ys[name], ys["none"]), name
    ref = oracle.moe(layer, xb)
    _, _, margin = oracle.route(layer, xb)
    sure = margin >= delta_for(2048)
    assert sure.sum() >= max(1, T - 1)
    assert rel_err(ys["none"].float().cpu().numpy()[sure], ref[sure]) <= BF16_TOL


def test_ablation_workspace_short_is_rejected(M, big):
    _, dl = big
    T = 64
    x = M.bf16_from_bits(synth.prefill_x(T, seed=90), DEV)
    ws = M.workspace(dl, T, DEV)  # the product workspace lacks the expanded weights
    with pytest.raises(M.MoeError) as ei:
        M.moe_prefill_ablation(dl, x, M.ABL_SEPARATE_DEQUANT, ws=ws)
    assert ei.value.code == M.E_WORKSPACE
