"""The layer's calls replayed from a HIP graph ("Optimizing On-Device Inference for Apple
Silicon", section "Keep expert routing on the GPU": routing, grouping and the expert work are
enqueued as one stream of GPU work with no CPU round trip in between).

moe_prefill, moe_decode and a two-layer moe_stack_forward step are captured once and replayed
several times, with other eager calls on the same workspaces and synchronisations between the
replays; every replay must reproduce the eager results bit for bit. A call that waited on the
host or copied to it could not be captured at all.
"""
import numpy as np
import pytest
import torch

from routed_expert_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def M():
    from routed_expert_amd import moe
    moe.lib()
    return moe


def test_layer_calls_replay_from_a_graph(M):
    print("\n[graph] capture moe_prefill T=300, 4 x moe_decode, a 2-layer stack decode step",
          flush=True)
    dls = [M.DeviceLayer.from_host(synth.decode_layer(l), DEV) for l in range(2)]
    dl = dls[0]
    T = 300
    x = M.bf16_from_bits(synth.prefill_x(T, seed=61), DEV)
    xo = M.bf16_from_bits(synth.prefill_x(T, seed=62), DEV)      # other eager work
    xt = M.bf16_from_bits(np.concatenate([synth.decode_token(t) for t in range(4)]), DEV)
    h0 = M.bf16_from_bits(synth.decode_token(9), DEV)
    ws, wsd = M.workspace(dl, T, DEV), M.workspace(dl, 1, DEV)
    wss = M.stack_workspace(dls, 1, DEV)
    # eager reference results
    y_ref = M.moe_prefill(dl, x, ws=ws)
    yd_ref = torch.stack([M.moe_decode(dl, xt[t:t + 1], ws=wsd)[0] for t in range(4)])
    hs_ref = M.moe_stack_forward(dls, h0.clone(), chunk_tokens=1, ws=wss)
    torch.cuda.synchronize()
    y = torch.empty_like(y_ref)
    yd = torch.empty_like(yd_ref)
    hs = torch.empty_like(h0)

    def work():
        M.moe_prefill(dl, x, y=y, ws=ws)
        for t in range(4):
            M.moe_decode(dl, xt[t:t + 1], y=yd[t:t + 1], ws=wsd)
        hs.copy_(h0)
        M.moe_stack_forward(dls, hs, chunk_tokens=1, ws=wss)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(5):
        y.zero_()
        yd.zero_()
        hs.zero_()
        M.moe_prefill(dl, xo, ws=ws)                # eager work on the same workspaces
        M.moe_decode(dl, xt[3:4], ws=wsd)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), rep
        assert torch.equal(yd.view(torch.int16), yd_ref.view(torch.int16)), rep
        assert torch.equal(hs.view(torch.int16), hs_ref.view(torch.int16)), rep
