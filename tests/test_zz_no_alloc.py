"""moe_decode_noalloc (the decode entry point for callers that cannot allocate: it runs on the
library's static per-GPU scratch array instead of a caller workspace) against moe_decode, called
through the C ABI: two calls in a row, the second on a smaller layer (the generic decode path
with a smaller hidden size), then the model-width layer again with a residual. The results
must be the bits moe_decode gives, since both run the same kernels."""
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


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_decode_noalloc_matches_decode(M):
    print("\n[noalloc] model-width layer, then H=256 E=16 k=4, then model width + residual",
          flush=True)
    big = M.DeviceLayer.from_host(synth.decode_layer(0), DEV)
    small = M.DeviceLayer.from_host(
        synth.make_int4_layer(81, hidden=256, inter=128, n_experts=16, top_k=4, n_shared=1,
                              router_std=0.1), DEV)
    x1 = M.bf16_from_bits(synth.decode_token(5), DEV)
    x2 = M.bf16_from_bits(synth.bf16_activations(82, (1, 256)), DEV)
    r = M.bf16_from_bits(synth.bf16_activations(83, (1, 2048)), DEV)
    ref1 = M.moe_decode(big, x1, ws=M.workspace(big, 1, DEV))
    ref2 = M.moe_decode(small, x2, ws=M.workspace(small, 1, DEV))
    ref3 = M.moe_decode(big, x1, residual=r, ws=M.workspace(big, 1, DEV))
    y1 = M.moe_decode_noalloc(big, x1)
    y2 = M.moe_decode_noalloc(small, x2)
    y3 = M.moe_decode_noalloc(big, x1, residual=r)
    torch.cuda.synchronize()
    assert _same(y1, ref1)
    assert _same(y2, ref2)
    assert _same(y3, ref3)
    assert not _same(y1, y3)
