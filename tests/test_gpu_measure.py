"""The measurement aids behind the bench's ceilings run on the GPU and compute nothing of the
layer ("Optimizing On-Device Inference for Apple Silicon", section "Limits of further
optimization": kernels are judged against the fastest rate measured for their own access
pattern): the dense MFMA loop on both kinds of operands, and the decode kernels' weight loads
without their arithmetic. Each must return MOE_OK, report the FLOP it runs, leave its sink
untouched (it is written only if a checksum equals one fixed word), and leave the layer's own
results unchanged.
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


def test_mfma_ceiling_both_operand_kinds(M):
    print("\n[measure] moe_mfma_ceiling, 10 iterations, both operand kinds", flush=True)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    for kind in (M.CEIL_FULL_MANTISSA, M.CEIL_LOW_ENTROPY):
        flops = M.mfma_ceiling(10, sink, kind)
        torch.cuda.synchronize()
        # 512 workgroups x 4 waves x 10 iterations x 8 MFMAs of 32x32x16 (32,768 FLOP)
        assert flops == 512 * 4 * 10 * 8 * 32768
        assert int(sink.item()) == 0


def test_decode_read_ceilings_leave_the_layer_alone(M):
    print("\n[measure] moe_decode_read_ceiling parts 0-2 on the decode layer", flush=True)
    layer = synth.decode_layer(0)
    dl = M.DeviceLayer.from_host(layer, DEV)
    x = M.bf16_from_bits(synth.decode_token(0), DEV)
    ws = M.workspace(dl, 1, DEV)
    y0 = M.moe_decode(dl, x, ws=ws)
    torch.cuda.synchronize()
    ids = torch.arange(0, 256, 32, dtype=torch.int32, device=DEV)   # 8 distinct experts
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    for part in (0, 1, 2):
        M.decode_read_ceiling(dl, ids, part, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    y1 = M.moe_decode(dl, x, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    assert np.isfinite(y1.float().cpu().numpy()).all()
