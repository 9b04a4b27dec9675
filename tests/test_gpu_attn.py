"""GPU parity of grouped-query decode attention (moe_attn_decode) against the oracle.

Workload: the model's full-attention layers ("Optimizing On-Device Inference for Apple
Silicon", section "Qwen creates three distinct workload shapes": 16 query heads, two KV
heads, eight query heads per KV head, 256 values per head; bf16 cache, section "Read the
attention cache efficiently"), one decode token over caches from 1 to 131,072 positions
(the page's sweep reaches 128K), with the seeded recipe of synth.attn_inputs.

Bar: per element |out - ref| <= 2^-8 |ref| + 1e-4 rms(ref). Scores, softmax and sums are
fp32 (bf16 products are exact in fp32), so the error is the final rounding to bf16 (at most
2^-9 relative) plus fp32 summation error orders of magnitude smaller. The unpacked
variant runs the same blocks and arithmetic per head and must match bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from routed_expert_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def M():
    from routed_expert_amd import moe
    moe.lib()
    return moe


def announce(msg):
    print(f"\n[attn] {msg}", flush=True)


def dev_bits(M, bits):
    return M.bf16_from_bits(bits, DEV)


def check(out, ref):
    got = out.float().cpu().numpy().astype(np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-4 * rms
    assert np.all(err <= bound), (float(err.max()), float((err / (np.abs(ref) + rms)).max()))


def run(M, ctx, seed, n_q=16, n_kv=2, packed=True):
    q, k, v = synth.attn_inputs(ctx, seed=seed, n_q=n_q, n_kv=n_kv)
    out = M.moe_attn_decode(dev_bits(M, q), dev_bits(M, k), dev_bits(M, v), packed=packed)
    torch.cuda.synchronize()
    return q, k, v, out


@pytest.mark.parametrize("ctx", [1, 2, 31, 32, 33, 127, 128, 129, 1000, 3840])
def test_attn_short_contexts(M, ctx):
    announce(f"moe_attn_decode 16/2/256 ctx={ctx}")
    q, k, v, out = run(M, ctx, seed=ctx)
    check(out, oracle.attn_decode(q, k, v, 16, 2, 1 / 16))


@pytest.mark.parametrize("ctx", [32768, 65536 + 777, 131072])
def test_attn_long_contexts(M, ctx):
    # block splitting at its full width (256 blocks per KV head) and a ragged last block
    announce(f"moe_attn_decode 16/2/256 ctx={ctx}")
    q, k, v, out = run(M, ctx, seed=7)
    check(out, oracle.attn_decode(q, k, v, 16, 2, 1 / 16))


@pytest.mark.parametrize("n_q,n_kv", [(8, 8), (8, 4), (8, 2), (4, 1)])
def test_attn_other_groupings(M, n_q, n_kv):
    ctx = 2000
    announce(f"moe_attn_decode {n_q}/{n_kv}/256 ctx={ctx}")
    q, k, v, out = run(M, ctx, seed=11, n_q=n_q, n_kv=n_kv)
    check(out, oracle.attn_decode(q, k, v, n_q, n_kv, 1 / 16))


@pytest.mark.parametrize("n_q,n_kv,ctx,blocks", [(16, 2, 12000, 94), (4, 1, 50000, 391),
                                                  (16, 2, 9000, 71)])
def test_attn_merge_widths(M, n_q, n_kv, ctx, blocks):
    # the merge takes ceil(blocks / 64) partials per lane: 2 at 94 and 71 blocks, 8 at 391
    # (one KV head may use up to 512 blocks)
    announce(f"moe_attn_decode {n_q}/{n_kv}/256 ctx={ctx} ({blocks} blocks)")
    q, k, v, out = run(M, ctx, seed=ctx, n_q=n_q, n_kv=n_kv)
    check(out, oracle.attn_decode(q, k, v, n_q, n_kv, 1 / 16))


@pytest.mark.parametrize("ctx", [500, 40000])
def test_attn_unpacked_is_bit_identical(M, ctx):
    announce(f"moe_attn_decode_unpacked vs packed ctx={ctx}")
    q, k, v = synth.attn_inputs(ctx, seed=21)
    qd, kd, vd = dev_bits(M, q), dev_bits(M, k), dev_bits(M, v)
    a = M.moe_attn_decode(qd, kd, vd)
    b = M.moe_attn_decode(qd, kd, vd, packed=False)
    c = M.moe_attn_decode(qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_attn_cache_capacity_and_scale(M):
    # a cache allocated for 6000 positions of which 4100 are filled; another scale
    ctx, cap = 4100, 6000
    announce(f"moe_attn_decode ctx={ctx} in a cache of {cap}, scale 0.11")
    q, k, v = synth.attn_inputs(ctx, seed=31)
    kc = np.zeros((2, cap, 256), dtype=np.uint16)
    vc = np.full((2, cap, 256), 0x7F80, dtype=np.uint16)   # +inf past ctx: must never be read
    kc[:, :ctx], vc[:, :ctx] = k, v
    out = M.moe_attn_decode(dev_bits(M, q), dev_bits(M, kc), dev_bits(M, vc), ctx=ctx,
                            scale=0.11)
    torch.cuda.synchronize()
    check(out, oracle.attn_decode(q, k, v, 16, 2, 0.11))


def test_attn_workspace_short_is_rejected(M):
    q, k, v = synth.attn_inputs(5000, seed=41)
    ws = M.attn_workspace(16, 2, 256, 100, DEV)
    with pytest.raises(M.MoeError) as ei:
        M.moe_attn_decode(dev_bits(M, q), dev_bits(M, k), dev_bits(M, v), ws=ws)
    assert ei.value.code == M.E_WORKSPACE
