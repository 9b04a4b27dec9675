"""GPU parity of the layer stack (pre-norm residual blocks h <- h + MoE_l(RMSNorm(h))) and of
its chunk loop, through the C ABI (moe_stack_forward).

The stack is checked teacher-forced, layer by layer: the oracle takes the GPU's bf16 input h of
layer l, forms the layer's input exactly as the stack defines it (RMSNorm of unit gain, rounded
once to bf16), runs its own fp64 MoE on it and adds h. Every row is compared: the GPU's output
of layer l must agree within the bf16 rounding of the residual stream plus 2e-2 of the RMS of
the layer's MoE output. Rows whose oracle top-k boundary lies inside the routing tie window
(margin below delta) are counted and may differ. Prompt chunking ("Optimizing On-Device
Inference for Apple Silicon", section "Bound temporary memory with prompt chunking") must not
change any output bit, and neither may splitting the stack over several calls.
"""
import numpy as np
import pytest
import torch

import oracle
from parity_util import BF16_TOL, delta_for
from routed_expert_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
EPS = float(np.float32(1e-6))   # the value the library receives as a float


@pytest.fixture(scope="module")
def M():
    from routed_expert_amd import moe
    moe.lib()
    return moe


def announce(msg):
    print(f"\n[stack] {msg}", flush=True)


def small_stack(M, n_layers, H=256, I=128, E=16, k=4, S=1):
    layers = [synth.make_int4_layer(300 + l, hidden=H, inter=I, n_experts=E, top_k=k,
                                    n_shared=S, router_std=0.1) for l in range(n_layers)]
    return layers, [M.DeviceLayer.from_host(L, DEV) for L in layers]


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def check_layer_step(layer, h_in_bits, h_out_bits, olayer=None):
    """Every row of one stack layer's GPU output against the oracle fed with the GPU's input.
    Returns the number of rows inside the routing tie window (not compared)."""
    h_in = oracle.to_f64(h_in_bits)
    n = oracle.stack_layer_input(h_in_bits, EPS)      # bf16(RMSNorm(h)), the layer's input
    ol = olayer if olayer is not None else oracle.OracleLayer(layer)
    _, _, margin = oracle.route(ol, n)
    y_ref = oracle.moe(ol, n)
    ref = h_in + y_ref
    got = oracle.to_f64(h_out_bits)
    sure = margin >= delta_for(layer.hidden)
    y_rms = np.sqrt(np.mean(y_ref[sure] ** 2))
    bound = 2.0 ** -8 * np.abs(ref) + BF16_TOL * y_rms
    d = np.abs(got - ref)[sure]
    assert np.all(d <= bound[sure]), float(np.max(d - bound[sure]))
    assert np.max(d) / np.sqrt(np.mean(ref[sure] ** 2)) <= BF16_TOL
    return int((~sure).sum())


@pytest.mark.parametrize("T,chunk", [(37, 16), (1, 16)])
def test_stack_teacher_forced_small(M, T, chunk):
    announce(f"moe_stack_forward 4 small int4 layers T={T} chunk={chunk}")
    layers, dls = small_stack(M, 4)
    h0 = M.bf16_from_bits(synth.bf16_activations(400 + T, (T, 256)), DEV)
    hs = [h0.clone()]
    for dl in dls:                              # one layer per call
        h = hs[-1].clone()
        M.moe_stack_forward([dl], h, chunk_tokens=chunk, eps=EPS)
        hs.append(h)
    whole = h0.clone()                           # all layers in one call
    M.moe_stack_forward(dls, whole, chunk_tokens=chunk, eps=EPS)
    torch.cuda.synchronize()
    assert torch.equal(whole, hs[-1])
    for l, layer in enumerate(layers):
        assert check_layer_step(layer, bits(hs[l]), bits(hs[l + 1])) <= max(1, T // 20)


def test_stack_chunked_equals_unchunked(M):
    announce("moe_stack_forward 3 small int4 layers T=300, chunks of 64 vs one chunk")
    _, dls = small_stack(M, 3)
    h0 = M.bf16_from_bits(synth.bf16_activations(401, (300, 256)), DEV)
    a, b = h0.clone(), h0.clone()
    M.moe_stack_forward(dls, a, chunk_tokens=64, eps=EPS)
    M.moe_stack_forward(dls, b, chunk_tokens=300, eps=EPS)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert not torch.equal(a, h0)


def test_stack_full_shape_layers(M):
    # two layers of the model's shape (H=2048, I=512, E=256, k=8, one shared expert), every
    # row of a 96-token prompt in chunks of 40 and of eight decode steps
    announce("moe_stack_forward 2 int4 layers H=2048 T=96 chunk=40, decode T=1 x 8")
    layers = [synth.decode_layer(l) for l in range(2)]
    dls = [M.DeviceLayer.from_host(L, DEV) for L in layers]
    h0 = M.bf16_from_bits(synth.bf16_activations(402, (96, 2048)), DEV)
    h1 = h0.clone()
    M.moe_stack_forward(dls[:1], h1, chunk_tokens=40, eps=EPS)
    h2 = h1.clone()
    M.moe_stack_forward(dls[1:], h2, chunk_tokens=40, eps=EPS)
    ws1 = M.stack_workspace(dls[:1], 1, DEV)
    dec = h0[:8].clone()                         # the decode path of the same stack
    for t in range(8):
        M.moe_stack_forward(dls[:1], dec[t:t + 1], chunk_tokens=1, eps=EPS, ws=ws1)
    torch.cuda.synchronize()
    unsure = check_layer_step(layers[0], bits(h0), bits(h1))
    unsure += check_layer_step(layers[1], bits(h1), bits(h2))
    unsure += check_layer_step(layers[0], bits(h0[:8]), bits(dec))
    assert unsure <= 3


def test_stack_fused_decode_norm_equals_rmsnorm_kernel(M):
    # the T = 1 stack step normalises inside the decode kernels; the RMSNorm kernel followed
    # by moe_decode on the same row must give the same bits, on many rows of several scales
    announce("stack decode step vs moe_rmsnorm + moe_decode, 48 rows, 3 scales")
    dl = M.DeviceLayer.from_host(synth.decode_layer(0), DEV)
    ws1 = M.stack_workspace([dl], 1, DEV)
    wsd = M.workspace(dl, 1, DEV)
    for scale_seed, scale in ((403, 1.0), (404, 37.0), (405, 0.01)):
        rows = synth.f32_to_bf16_bits(
            synth.bf16_bits_to_f32(synth.bf16_activations(scale_seed, (16, 2048))) * scale)
        hr = M.bf16_from_bits(rows, DEV)
        nr = M.moe_rmsnorm(hr, EPS)
        torch.cuda.synchronize()
        assert np.array_equal(bits(nr), oracle.stack_layer_input(rows, EPS))
        for t in range(16):
            fused = hr[t:t + 1].clone()
            M.moe_stack_forward([dl], fused, chunk_tokens=1, eps=EPS, ws=ws1)
            sep = M.moe_decode(dl, nr[t:t + 1], residual=hr[t:t + 1], ws=wsd)
            torch.cuda.synchronize()
            assert torch.equal(fused, sep), (scale, t)


# ---- the 40-layer stack at its benchmarked size -----------------------------------------
N_LAYERS, PROMPT, CHUNK, N_DEC = 40, 32768, 4096, 256


def prompt_rows_checked():
    """64 prompt rows: both sides of every chunk boundary, the first and last rows, and
    seeded rows in between."""
    edge = [0, PROMPT - 1] + [c * CHUNK + d for c in range(1, PROMPT // CHUNK) for d in (-1, 0)]
    rng = np.random.default_rng(44)
    rest = rng.choice(np.setdiff1d(np.arange(PROMPT), edge), 64 - len(edge), replace=False)
    return np.sort(np.concatenate([edge, rest])).astype(np.int64)


@pytest.mark.timeout(900)
def test_stack_40_layers_prompt_and_decode(M):
    """The 40-layer stack of decode-shaped int4 layers (layer l drawn from seed l): a
    32,768-token prompt in chunks of 4096 rows and 256 batch-1 decode tokens, teacher-forced
    per layer on 64 prompt rows (every chunk boundary from both sides) and every decode token.
    The whole stack in one call must then equal the layer-by-layer run bit for bit."""
    rows = prompt_rows_checked()
    announce(f"40 layers, prompt {PROMPT} in chunks of {CHUNK}, {N_DEC} decode tokens")
    x0 = synth.f32_to_bf16_bits(
        np.random.default_rng(3).standard_normal((PROMPT, 2048), dtype=np.float32))
    hp = M.bf16_from_bits(x0, DEV)
    hd = M.bf16_from_bits(np.concatenate(
        [synth.bf16_activations(2_000_000 + t, (1, 2048)) for t in range(N_DEC)]), DEV)
    rows_d = torch.from_numpy(rows).to(DEV)
    dls, ws_p, ws_d = [], None, None
    total_unsure = 0
    for l in range(N_LAYERS):
        layer = synth.decode_layer(l)
        dl = M.DeviceLayer.from_host(layer, DEV)
        dls.append(dl)
        if ws_p is None:
            ws_p = M.stack_workspace([dl], CHUNK, DEV)
            ws_d = M.stack_workspace([dl], 1, DEV)
        in_p, in_d = bits(hp[rows_d]), bits(hd)
        M.moe_stack_forward([dl], hp, chunk_tokens=CHUNK, eps=EPS, ws=ws_p)
        for t in range(N_DEC):
            M.moe_stack_forward([dl], hd[t:t + 1], chunk_tokens=1, eps=EPS, ws=ws_d)
        torch.cuda.synchronize()
        out_p, out_d = bits(hp[rows_d]), bits(hd)
        unsure = check_layer_step(layer, np.concatenate([in_p, in_d]),
                                  np.concatenate([out_p, out_d]))
        total_unsure += unsure
        print(f"[stack] layer {l}: {len(rows)} prompt rows + {N_DEC} decode tokens checked, "
              f"{unsure} in the tie window", flush=True)
        del layer
    assert total_unsure <= N_LAYERS * 2
    # the same stack in one call per prompt / per decode token
    h_all = M.bf16_from_bits(x0, DEV)
    M.moe_stack_forward(dls, h_all, chunk_tokens=CHUNK, eps=EPS)
    ws_all = M.stack_workspace(dls, 1, DEV)
    d_all = M.bf16_from_bits(np.concatenate(
        [synth.bf16_activations(2_000_000 + t, (1, 2048)) for t in range(N_DEC)]), DEV)
    for t in range(N_DEC):
        M.moe_stack_forward(dls, d_all[t:t + 1], chunk_tokens=1, eps=EPS, ws=ws_all)
    torch.cuda.synchronize()
    assert torch.equal(h_all, hp)
    assert torch.equal(d_all, hd)
    announce("40-layer calls equal the layer-by-layer run bit for bit")
