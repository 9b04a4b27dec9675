"""Host-side checks of the C-ABI library: it loads, exports every declared entry point,
and rejects bad arguments on the host before touching the GPU (no compute calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def M():
    from routed_expert_amd import build, moe
    if not os.path.exists(moe.LIB_PATH):
        build.build()
    moe.lib()
    return moe


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("moe_route", "moe_prefill", "moe_decode", "moe_workspace_bytes",
                     "moe_last_error", "moe_pack_weights", "moe_pack_bytes"):
        assert required in names


def test_library_exports_every_declared_symbol(M):
    lib = ctypes.CDLL(M.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(M.EXPORTS)


def test_single_hip_runtime(M):
    assert len(M.hip_runtimes_mapped()) <= 1


def fake_layer(M, **kw):
    """Descriptor with plausible aligned (never dereferenced) device addresses."""
    p = dict(abi_version=M.ABI_VERSION, hidden=2048, inter=512, n_experts=256, top_k=8,
             n_shared=1, w_format=M.W_INT4_G64, act_dtype=M.ACT_BF16, router_w=0x10000,
             router_b=None, w13_q=0x20000, w13_s=0x30000, w13_b=0x40000, w2_q=0x50000,
             w2_s=0x60000, w2_b=0x70000, w13_t=0x80000, w13_tsb=0x90000, w2_t=0xa0000,
             w2_tsb=0xb0000, router_planes=None)
    p.update(kw)
    return M.MoeLayer(*[p[f] for f, _ in M.MoeLayer._fields_])


def ws_bytes(M, layer, T):
    n = ctypes.c_size_t(0)
    st = M.lib().moe_workspace_bytes(ctypes.byref(layer), T, ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,code", [
    (dict(abi_version=99), -1),
    (dict(hidden=0), -1),
    (dict(top_k=0), -1),
    (dict(top_k=300, n_experts=256), -1),
    (dict(n_shared=2), -1),
    (dict(n_experts=512, top_k=8), -2),
    (dict(top_k=9), -2),
    (dict(hidden=2000), -2),
    (dict(inter=500), -2),
    (dict(hidden=384), -2),             # int4 needs hidden % 256 == 0
    (dict(inter=192), -2),              # int4 needs inter % 128 == 0
    (dict(act_dtype=0), -2),            # int4 weights with fp32 activations
    (dict(w_format=0), -2),             # fp32 weights with bf16 activations
    (dict(w_format=7), -1),
    (dict(router_w=None), -1),
    (dict(w13_s=None), -1),
    (dict(w13_q=0x20008), -1),          # codes must be 16-byte aligned
    (dict(router_b=0x10002), -1),
    (dict(router_planes=0x10008), -1),
    (dict(w2_b=0x70002), -1),           # scales and biases are read as dwords
])
def test_descriptor_validation(M, kw, code):
    st, _ = ws_bytes(M, fake_layer(M, **kw), 16)
    assert st == code
    assert M.lib().moe_last_error().decode() != ""


def test_workspace_size_grows_with_tokens(M):
    layer = fake_layer(M)
    sizes = [ws_bytes(M, layer, T) for T in (1, 64, 4096)]
    assert all(st == 0 for st, _ in sizes)
    assert sizes[0][1] < sizes[1][1] < sizes[2][1]
    assert ws_bytes(M, layer, 0)[0] == -1


def test_call_argument_errors_before_any_launch(M):
    L = M.lib()
    layer = fake_layer(M)
    ref = ctypes.byref(layer)
    _, need = ws_bytes(M, layer, 4096)
    x, y, ws = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000), ctypes.c_void_p(0x300000)
    # workspace too small
    assert L.moe_prefill(ref, x, 4096, y, None, None, ws, need - 1, None) == M.E_WORKSPACE
    assert "workspace" in L.moe_last_error().decode()
    # null / misaligned activations, bad T
    assert L.moe_prefill(ref, None, 4, y, None, None, ws, need, None) == M.E_INVALID
    assert L.moe_prefill(ref, ctypes.c_void_p(0x100002), 4, y, None, None, ws, need,
                         None) == M.E_INVALID
    assert L.moe_prefill(ref, x, -1, y, None, None, ws, need, None) == M.E_INVALID
    assert L.moe_decode(ref, x, None, None, ws, need, None) == M.E_INVALID
    assert L.moe_decode(ref, x, y, None, None, need, None) == M.E_INVALID
    # route outputs must all be given
    ro = M.MoeRouteOut(0x400000, 0x500000, 0x600000, 0x700000, None, 0x800000)
    assert L.moe_route(ref, x, 4, ctypes.byref(ro), ws, need, None) == M.E_INVALID
    assert L.moe_route(ref, x, 4, None, ws, need, None) == M.E_INVALID
    # empty input is a valid no-op that enqueues nothing
    assert L.moe_prefill(ref, x, 0, y, None, None, ws, need, None) == M.OK
    assert L.moe_last_error().decode() == ""
    assert L.moe_rmsnorm(x, 4, 2048, ctypes.c_float(-1.0), M.ACT_BF16, y, None) == M.E_INVALID
    # int4 prefill needs the tiled weights
    bare = fake_layer(M, w13_t=None)
    assert L.moe_prefill(ctypes.byref(bare), x, 4, y, None, None, ws, need, None) == M.E_INVALID
    assert "moe_pack_weights" in L.moe_last_error().decode()
    assert L.moe_prefill(ctypes.byref(fake_layer(M, w2_tsb=0xb0008)), x, 4, y, None, None, ws,
                         need, None) == M.E_INVALID
    assert L.moe_rmsnorm(x, 4, 2048, ctypes.c_float(1e-6), 5, y, None) == M.E_INVALID


def test_pack_size_and_argument_errors(M):
    L = M.lib()
    layer = fake_layer(M)
    n = ctypes.c_size_t(0)
    assert L.moe_pack_bytes(ctypes.byref(layer), ctypes.byref(n)) == M.OK
    # codes keep their size; {scale, bias} pairs of 4 groups per row and block
    E1, H, I = 257, 2048, 512
    codes = E1 * 2 * I * H // 2 + E1 * H * I // 2
    sb = E1 * (2 * I // 64) * (H // 256) * 64 * 16 + E1 * (H // 64) * (I // 256) * 64 * 16
    planes = 2 * (E1 - 1) * H * 2   # the router split into two fp16 planes
    assert n.value == codes + sb + planes
    out = M.MoeLayer()
    dst = ctypes.c_void_p(0x1000000)
    assert L.moe_pack_weights(ctypes.byref(layer), dst, n.value - 1, ctypes.byref(out),
                              None) == M.E_WORKSPACE
    assert L.moe_pack_weights(ctypes.byref(layer), ctypes.c_void_p(0x1000010), n.value,
                              ctypes.byref(out), None) == M.E_INVALID
    assert L.moe_pack_weights(ctypes.byref(layer), dst, n.value, None, None) == M.E_INVALID
    f32 = fake_layer(M, w_format=M.W_F32, act_dtype=M.ACT_F32)
    assert L.moe_pack_bytes(ctypes.byref(f32), ctypes.byref(n)) == M.E_UNSUPPORTED


def test_stack_argument_errors(M):
    L = M.lib()
    layers = (M.MoeLayer * 3)(fake_layer(M), fake_layer(M), fake_layer(M))
    n = ctypes.c_size_t(0)
    assert L.moe_stack_workspace_bytes(layers, 3, 4096, ctypes.byref(n)) == M.OK
    one = ctypes.c_size_t(0)
    assert L.moe_workspace_bytes(ctypes.byref(layers[0]), 4096, ctypes.byref(one)) == M.OK
    assert n.value == one.value + 4096 * 2048 * 2   # one layer workspace + normalised rows
    assert L.moe_stack_workspace_bytes(layers, 0, 4096, ctypes.byref(n)) == M.E_INVALID
    assert L.moe_stack_workspace_bytes(layers, 3, 0, ctypes.byref(n)) == M.E_INVALID
    odd = (M.MoeLayer * 2)(fake_layer(M), fake_layer(M, hidden=1024))
    assert L.moe_stack_workspace_bytes(odd, 2, 64, ctypes.byref(n)) == M.E_INVALID
    assert "hidden" in L.moe_last_error().decode()
    h, ws = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x300000)
    assert L.moe_stack_workspace_bytes(layers, 3, 64, ctypes.byref(n)) == M.OK
    f = ctypes.c_float(1e-6)
    assert L.moe_stack_forward(layers, 3, h, 64, 64, f, ws, n.value - 1, None) == M.E_WORKSPACE
    assert L.moe_stack_forward(layers, 3, h, 64, 64, ctypes.c_float(-1.0), ws, n.value,
                               None) == M.E_INVALID
    assert L.moe_stack_forward(layers, 3, None, 64, 64, f, ws, n.value, None) == M.E_INVALID
    assert L.moe_stack_forward(layers, 3, h, 0, 64, f, ws, n.value, None) == M.OK
    unpacked = (M.MoeLayer * 1)(fake_layer(M, w2_t=None))
    assert L.moe_stack_forward(unpacked, 1, h, 64, 64, f, ws, n.value, None) == M.E_INVALID


def test_profile_controls_without_records(M):
    M.profile_reset()
    M.profile_enable(False)
    assert M.profile_query("k_grouped_gateup") == (0.0, 0)


def test_ablation_workspace_and_argument_errors(M):
    L = M.lib()
    layer = fake_layer(M)
    ref = ctypes.byref(layer)
    sizes = {}
    for name, v in M.ABLATIONS.items():
        n = ctypes.c_size_t(0)
        assert L.moe_ablation_workspace_bytes(ref, 4096, v, ctypes.byref(n)) == M.OK
        sizes[name] = n.value
    # every variant needs at least the product workspace; the separate dequantisation pass
    # adds the expanded fp16 weights: 2 bytes per weight of all E+S experts
    _, base = ws_bytes(M, layer, 4096)
    assert min(sizes.values()) >= base
    E1, H, I = 257, 2048, 512
    assert sizes["separate_dequant"] - sizes["none"] >= E1 * 3 * H * I * 2
    n = ctypes.c_size_t(0)
    assert L.moe_ablation_workspace_bytes(ref, 16, 6, ctypes.byref(n)) == M.E_INVALID
    assert L.moe_ablation_workspace_bytes(ref, 16, -1, ctypes.byref(n)) == M.E_INVALID
    x, y, ws = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000), ctypes.c_void_p(0x300000)
    need = sizes["separate_dequant"]
    assert L.moe_prefill_ablation(ref, 9, x, 64, y, None, ws, need, None) == M.E_INVALID
    assert "ablation" in L.moe_last_error().decode()
    assert L.moe_prefill_ablation(ref, M.ABL_SEPARATE_DEQUANT, x, 4096, y, None, ws,
                                  sizes["none"], None) == M.E_WORKSPACE
    assert L.moe_prefill_ablation(ref, M.ABL_TILE_64, None, 4, y, None, ws, need,
                                  None) == M.E_INVALID
    assert L.moe_prefill_ablation(ref, M.ABL_NONE, x, 0, y, None, ws, need, None) == M.OK
    f32 = fake_layer(M, w_format=M.W_F32, act_dtype=M.ACT_F32)
    assert L.moe_prefill_ablation(ctypes.byref(f32), M.ABL_NONE, x, 4, y, None, ws, need,
                                  None) == M.E_UNSUPPORTED
    bare = fake_layer(M, w13_t=None)
    assert L.moe_prefill_ablation(ctypes.byref(bare), M.ABL_NONE, x, 4, y, None, ws, need,
                                  None) == M.E_INVALID


def test_attention_argument_errors_before_any_launch(M):
    L = M.lib()
    n = ctypes.c_size_t(0)
    assert L.moe_attn_workspace_bytes(16, 2, 256, 131072, ctypes.byref(n)) == M.OK
    need = n.value
    assert need >= 256 * 16 * 258 * 4
    assert L.moe_attn_workspace_bytes(16, 2, 128, 1000, ctypes.byref(n)) == M.E_UNSUPPORTED
    assert L.moe_attn_workspace_bytes(12, 4, 256, 1000, ctypes.byref(n)) == M.E_UNSUPPORTED
    assert L.moe_attn_workspace_bytes(16, 2, 256, 0, ctypes.byref(n)) == M.E_INVALID
    q, k, v, o, ws = (ctypes.c_void_p(a) for a in (0x100000, 0x200000, 0x300000, 0x400000,
                                                   0x500000))
    f = ctypes.c_float(0.0625)
    args = lambda ctx, stride, nbytes: (q, k, v, 16, 2, 256, ctx, stride, f, o, ws, nbytes, None)
    assert L.moe_attn_decode(*args(4096, 4096 * 256, 100)) == M.E_WORKSPACE
    assert L.moe_attn_decode(*args(0, 4096 * 256, need)) == M.E_INVALID
    assert L.moe_attn_decode(*args(4096, 4095 * 256, need)) == M.E_INVALID   # stride < ctx*D
    inf = ctypes.c_float(float("inf"))
    assert L.moe_attn_decode(q, k, v, 16, 2, 256, 64, 64 * 256, inf, o, ws, need,
                             None) == M.E_INVALID
    assert L.moe_attn_decode(q, k, v, 16, 2, 128, 64, 64 * 128, f, o, ws, need,
                             None) == M.E_UNSUPPORTED
    assert L.moe_attn_decode(q, None, v, 16, 2, 256, 64, 64 * 256, f, o, ws, need,
                             None) == M.E_INVALID
    assert L.moe_attn_decode_unpacked(ctypes.c_void_p(0x100008), k, v, 16, 2, 256, 64,
                                      64 * 256, f, o, ws, need, None) == M.E_INVALID


def test_gdn_argument_errors_before_any_launch(M):
    L = M.lib()
    p = [ctypes.c_void_p(a) for a in (0x100000, 0x200000, 0x300000, 0x400000, 0x500000)]
    st, out = ctypes.c_void_p(0x600000), ctypes.c_void_p(0x700000)
    assert L.moe_gdn_scan(*p, 64, 16, 32, 64, 128, st, out, None) == M.E_UNSUPPORTED
    assert L.moe_gdn_scan(*p, 64, 16, 24, 128, 128, st, out, None) == M.E_UNSUPPORTED
    assert L.moe_gdn_scan(*p, -1, 16, 32, 128, 128, st, out, None) == M.E_INVALID
    assert L.moe_gdn_scan(*p, 64, 16, 32, 128, 128, None, out, None) == M.E_INVALID
    assert L.moe_gdn_scan(*p, 0, 16, 32, 128, 128, st, out, None) == M.OK   # empty: no-op
    q_bad = ctypes.c_void_p(0x100008)
    assert L.moe_gdn_scan(q_bad, *p[1:], 64, 16, 32, 128, 128, st, out, None) == M.E_INVALID


def test_gdn_chunked_workspace_and_argument_errors(M):
    L = M.lib()
    n = ctypes.c_size_t(0)
    assert L.moe_gdn_chunked_workspace_bytes(2048, 16, 32, 128, 128, ctypes.byref(n)) == M.OK
    # 64 chunks x 32 heads x (two 32 x 128 factor blocks, two 32 x 32 tables, 2 x 32) floats
    assert n.value == 64 * 32 * (2 * 32 * 128 + 2 * 32 * 32 + 64) * 4
    need = n.value
    assert L.moe_gdn_chunked_workspace_bytes(2048, 16, 32, 64, 128, ctypes.byref(n)) == \
        M.E_UNSUPPORTED
    p = [ctypes.c_void_p(a) for a in (0x100000, 0x200000, 0x300000, 0x400000, 0x500000)]
    st, out, ws = ctypes.c_void_p(0x600000), ctypes.c_void_p(0x700000), ctypes.c_void_p(0x800000)
    assert L.moe_gdn_scan_chunked(*p, 2048, 16, 32, 128, 128, st, out, ws, need - 1,
                                  None) == M.E_WORKSPACE
    assert L.moe_gdn_scan_chunked(*p, 2048, 16, 32, 128, 128, st, out, None, need,
                                  None) == M.E_INVALID
    assert L.moe_gdn_scan_chunked(*p, 0, 16, 32, 128, 128, st, out, ws, 0, None) == M.OK


def test_calls_without_a_device_return_hip_error(M):
    """With no GPU present every call that passes the host checks fails at its first HIP
    call with MOE_E_HIP and a message, instead of crashing (the addresses are never used)."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: the fake addresses would be dereferenced")
    lib = M.lib()
    L = fake_layer(M)
    st, need = ws_bytes(M, L, 16)
    assert st == 0
    ws, x, y = ctypes.c_void_p(0x1000000), ctypes.c_void_p(0x2000000), ctypes.c_void_p(0x3000000)
    calls = {
        "moe_rmsnorm": lambda: lib.moe_rmsnorm(x, 4, 2048, ctypes.c_float(1e-6), M.ACT_BF16, y,
                                               None),
        "moe_decode": lambda: lib.moe_decode(ctypes.byref(L), x, y, None, ws, need, None),
        "moe_prefill": lambda: lib.moe_prefill(ctypes.byref(L), x, 16, y, None, None, ws, need,
                                               None),
    }
    for name, call in calls.items():
        assert call() == M.E_HIP, name
        assert lib.moe_last_error().decode(), name


def test_decode_noalloc_rejects_layers_beyond_its_scratch(M):
    """The no-allocation decode holds 4 MiB of scratch per GPU: a layer whose one-token
    workspace is larger is refused on the host (nothing is launched, the addresses are never
    used), one that fits passes the size check."""
    lib = M.lib()
    x, y = ctypes.c_void_p(0x2000000), ctypes.c_void_p(0x3000000)
    wide = fake_layer(M, hidden=8192)
    st, need = ws_bytes(M, wide, 1)
    assert st == 0 and need > (4 << 20)
    assert lib.moe_decode_noalloc(ctypes.byref(wide), x, y, None, None) == M.E_WORKSPACE
    assert b"scratch" in lib.moe_last_error()
    st, need = ws_bytes(M, fake_layer(M), 1)
    assert st == 0 and need <= (4 << 20)
    assert lib.moe_decode_noalloc(ctypes.byref(fake_layer(M)), x, None, None, None) == M.E_INVALID


def test_measurement_aids_argument_errors(M):
    """The read ceilings and the MFMA loop reject bad arguments on the host."""
    lib = M.lib()
    L = fake_layer(M)
    sink = ctypes.c_void_p(0x4000000)
    ids = ctypes.c_void_p(0x5000000)
    assert lib.moe_decode_read_ceiling(ctypes.byref(L), ids, 3, sink, None) == M.E_INVALID
    assert lib.moe_decode_read_ceiling(ctypes.byref(L), None, 1, sink, None) == M.E_INVALID
    assert lib.moe_decode_read_ceiling(ctypes.byref(L), ids, 1, None, None) == M.E_INVALID
    odd = fake_layer(M, inter=256)            # not the batch-1 fast path
    assert lib.moe_decode_read_ceiling(ctypes.byref(odd), ids, 1, sink, None) == M.E_UNSUPPORTED
    f = ctypes.c_double(0)
    assert lib.moe_mfma_ceiling(0, 0, sink, ctypes.byref(f), None) == M.E_INVALID
    assert lib.moe_mfma_ceiling(10, 0, sink, None, None) == M.E_INVALID
    assert lib.moe_mfma_ceiling(10, 2, sink, ctypes.byref(f), None) == M.E_INVALID
    assert lib.moe_mfma_ceiling(10, -1, sink, ctypes.byref(f), None) == M.E_INVALID
