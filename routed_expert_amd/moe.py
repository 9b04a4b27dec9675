"""Python binding of the C-ABI MoE library (``libmoe.so``, declared in include/moe.h).

Argument marshalling only: torch provides device memory and the current HIP stream,
every step of the layer runs in the library's HIP kernels. There is no fallback: if
the library is missing, or no GPU is present, the calls raise.

torch is imported before the library is loaded so that the library binds to the HIP
runtime torch already mapped (both carry the soname libamdhip64.so.7).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

ABI_VERSION = 4
OK, E_INVALID, E_UNSUPPORTED, E_WORKSPACE, E_HIP = 0, -1, -2, -3, -4
W_F32, W_INT4_G64 = 0, 1
ACT_F32, ACT_BF16 = 0, 1

EXPORTS = ("moe_abi_version", "moe_last_error", "moe_workspace_bytes", "moe_pack_bytes",
           "moe_pack_weights", "moe_route", "moe_prefill", "moe_decode", "moe_decode_noalloc",
           "moe_stack_workspace_bytes", "moe_stack_forward", "moe_rmsnorm",
           "moe_profile_enable", "moe_profile_query", "moe_profile_reset",
           "moe_ablation_workspace_bytes", "moe_prefill_ablation",
           "moe_attn_workspace_bytes", "moe_attn_decode", "moe_attn_decode_unpacked",
           "moe_gdn_scan", "moe_gdn_chunked_workspace_bytes", "moe_gdn_scan_chunked",
           "moe_decode_read_ceiling", "moe_mfma_ceiling")
(ABL_NONE, ABL_SEPARATE_DEQUANT, ABL_HOST_ROUTING, ABL_TILE_64, ABL_FIXED_TILE,
 ABL_TILE_128) = range(6)
ABLATIONS = {"none": ABL_NONE, "separate_dequant": ABL_SEPARATE_DEQUANT,
             "host_routing": ABL_HOST_ROUTING, "tile_64": ABL_TILE_64,
             "fixed_tile": ABL_FIXED_TILE, "tile_128": ABL_TILE_128}


class MoeLayer(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("w_format", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
                ("w13_q", ctypes.c_void_p), ("w13_s", ctypes.c_void_p),
                ("w13_b", ctypes.c_void_p), ("w2_q", ctypes.c_void_p),
                ("w2_s", ctypes.c_void_p), ("w2_b", ctypes.c_void_p),
                ("w13_t", ctypes.c_void_p), ("w13_tsb", ctypes.c_void_p),
                ("w2_t", ctypes.c_void_p), ("w2_tsb", ctypes.c_void_p),
                ("router_planes", ctypes.c_void_p)]


class MoeRouteOut(ctypes.Structure):
    _fields_ = [("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("counts", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("sorted_tok", ctypes.c_void_p), ("slot_of", ctypes.c_void_p)]


class MoeError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


_lib = None


def hip_runtimes_mapped() -> list[str]:
    """Distinct libamdhip64 files mapped into this process."""
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return sorted(paths)


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with routed_expert_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "moe_abi_version": ([], I32),
        "moe_last_error": ([], ctypes.c_char_p),
        "moe_workspace_bytes": ([P, I64, ctypes.POINTER(SZ)], ctypes.c_int),
        "moe_pack_bytes": ([P, ctypes.POINTER(SZ)], ctypes.c_int),
        "moe_pack_weights": ([P, P, SZ, P, P], ctypes.c_int),
        "moe_route": ([P, P, I64, P, P, SZ, P], ctypes.c_int),
        "moe_prefill": ([P, P, I64, P, P, P, P, SZ, P], ctypes.c_int),
        "moe_decode": ([P, P, P, P, P, SZ, P], ctypes.c_int),
        "moe_decode_noalloc": ([P, P, P, P, P], ctypes.c_int),
        "moe_stack_workspace_bytes": ([P, I32, I64, ctypes.POINTER(SZ)], ctypes.c_int),
        "moe_stack_forward": ([P, I32, P, I64, I64, ctypes.c_float, P, SZ, P], ctypes.c_int),
        "moe_rmsnorm": ([P, I64, I32, ctypes.c_float, I32, P, P], ctypes.c_int),
        "moe_profile_enable": ([I32], ctypes.c_int),
        "moe_profile_query": ([ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                               ctypes.POINTER(I64)], ctypes.c_int),
        "moe_profile_reset": ([], ctypes.c_int),
        "moe_ablation_workspace_bytes": ([P, I64, I32, ctypes.POINTER(SZ)], ctypes.c_int),
        "moe_prefill_ablation": ([P, I32, P, I64, P, P, P, SZ, P], ctypes.c_int),
        "moe_attn_workspace_bytes": ([I32, I32, I32, I64, ctypes.POINTER(SZ)], ctypes.c_int),
        "moe_attn_decode": ([P, P, P, I32, I32, I32, I64, I64, ctypes.c_float, P, P, SZ, P],
                            ctypes.c_int),
        "moe_attn_decode_unpacked": ([P, P, P, I32, I32, I32, I64, I64, ctypes.c_float, P, P,
                                      SZ, P], ctypes.c_int),
        "moe_gdn_scan": ([P, P, P, P, P, I64, I32, I32, I32, I32, P, P, P], ctypes.c_int),
        "moe_gdn_chunked_workspace_bytes": ([I64, I32, I32, I32, I32, ctypes.POINTER(SZ)],
                                            ctypes.c_int),
        "moe_gdn_scan_chunked": ([P, P, P, P, P, I64, I32, I32, I32, I32, P, P, P, SZ, P],
                                 ctypes.c_int),
        "moe_decode_read_ceiling": ([P, P, I32, P, P], ctypes.c_int),
        "moe_mfma_ceiling": ([I32, I32, P, ctypes.POINTER(ctypes.c_double), P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes, fn.restype = args, res
    if L.moe_abi_version() != ABI_VERSION:
        raise RuntimeError("libmoe.so ABI version mismatch")
    runtimes = hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError(f"two HIP runtimes mapped: {runtimes}")
    _lib = L
    return L


def _check(fn, code):
    if code != OK:
        raise MoeError(fn, code, lib().moe_last_error().decode())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(a, device, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device)


class DeviceLayer:
    """A layer's weights in device memory plus its C descriptor.

    Built from a host layer in interchange layout (routed_expert_amd.synth.Layer) or
    from device tensors already in that layout (``from_tensors``)."""

    def __init__(self, hidden, inter, n_experts, top_k, n_shared, fmt, tensors):
        self.hidden, self.inter = hidden, inter
        self.n_experts, self.top_k, self.n_shared = n_experts, top_k, n_shared
        self.fmt = fmt
        self.t = tensors
        g = tensors.get
        self.desc = MoeLayer(ABI_VERSION, hidden, inter, n_experts, top_k, n_shared,
                             W_INT4_G64 if fmt == "int4" else W_F32,
                             ACT_BF16 if fmt == "int4" else ACT_F32,
                             *[None if g(n) is None else g(n).data_ptr() for n in
                               ("router_w", "router_b", "w13_q", "w13_s", "w13_b",
                                "w2_q", "w2_s", "w2_b")])
        if fmt == "int4":
            self.desc = moe_pack_weights(self)

    def packed_bytes(self) -> int:
        n = ctypes.c_size_t(0)
        _check("moe_pack_bytes", lib().moe_pack_bytes(self.ref, ctypes.byref(n)))
        return n.value

    @classmethod
    def from_host(cls, layer, device="cuda"):
        t = {"router_w": _dev(layer.router_w, device),
             "router_b": None if layer.router_b is None else _dev(layer.router_b, device)}
        if layer.fmt == "int4":
            t.update(w13_q=_dev(layer.w13_q, device), w2_q=_dev(layer.w2_q, device),
                     w13_s=_dev(layer.w13_s.view(np.int16), device, torch.bfloat16),
                     w13_b=_dev(layer.w13_b.view(np.int16), device, torch.bfloat16),
                     w2_s=_dev(layer.w2_s.view(np.int16), device, torch.bfloat16),
                     w2_b=_dev(layer.w2_b.view(np.int16), device, torch.bfloat16))
        else:
            t.update(w13_q=_dev(layer.w13, device), w2_q=_dev(layer.w2, device))
        return cls(layer.hidden, layer.inter, layer.n_experts, layer.top_k, layer.n_shared,
                   layer.fmt, t)

    @classmethod
    def from_tensors(cls, hidden, inter, n_experts, top_k, n_shared, fmt, **tensors):
        return cls(hidden, inter, n_experts, top_k, n_shared, fmt, tensors)

    @property
    def ref(self):
        return ctypes.byref(self.desc)

    @property
    def act_dtype(self):
        return torch.bfloat16 if self.fmt == "int4" else torch.float32


def moe_pack_weights(layer: DeviceLayer, stream=None) -> MoeLayer:
    """Tiled copy of an int4 layer's expert weights (kept alive in layer.t["tiled"]);
    returns the descriptor that points at both layouts."""
    device = layer.t["w13_q"].device
    dst = torch.empty(layer.packed_bytes(), dtype=torch.uint8, device=device)
    if dst.data_ptr() % 256:
        raise RuntimeError("tiled weight buffer is not 256-byte aligned")
    packed = MoeLayer()
    _check("moe_pack_weights", lib().moe_pack_weights(layer.ref, _ptr(dst), dst.numel(),
                                                      ctypes.byref(packed), _stream(stream)))
    layer.t["tiled"] = dst
    return packed


def moe_workspace_bytes(layer: DeviceLayer, max_tokens: int) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_workspace_bytes", lib().moe_workspace_bytes(layer.ref, int(max_tokens),
                                                            ctypes.byref(n)))
    return n.value


def workspace(layer: DeviceLayer, max_tokens: int, device="cuda") -> torch.Tensor:
    """Zero-filled workspace for calls with up to max_tokens tokens."""
    return torch.zeros(moe_workspace_bytes(layer, max_tokens), dtype=torch.uint8, device=device)


def route_buffers(layer: DeviceLayer, T: int, device="cuda") -> dict:
    E, k = layer.n_experts, layer.top_k
    i32 = dict(dtype=torch.int32, device=device)
    return {"topk_ids": torch.empty((T, k), **i32),
            "topk_w": torch.empty((T, k), dtype=torch.float32, device=device),
            "counts": torch.empty(E, **i32), "offsets": torch.empty(E + 1, **i32),
            "sorted_tok": torch.empty(T * k, **i32), "slot_of": torch.empty((T, k), **i32)}


def _route_desc(b):
    return MoeRouteOut(*[b[n].data_ptr() for n in ("topk_ids", "topk_w", "counts", "offsets",
                                                    "sorted_tok", "slot_of")])


def _ws(layer, ws, T, device):
    return workspace(layer, max(T, 1), device) if ws is None else ws


def moe_route(layer: DeviceLayer, x: torch.Tensor, ws=None, out=None, stream=None) -> dict:
    T = x.shape[0]
    ws = _ws(layer, ws, T, x.device)
    out = route_buffers(layer, T, x.device) if out is None else out
    desc = _route_desc(out)
    _check("moe_route", lib().moe_route(layer.ref, _ptr(x), T, ctypes.byref(desc), _ptr(ws),
                                        ws.numel(), _stream(stream)))
    return out


def moe_prefill(layer: DeviceLayer, x: torch.Tensor, y=None, residual=None, ws=None,
                route_out=None, stream=None) -> torch.Tensor:
    T = x.shape[0]
    ws = _ws(layer, ws, T, x.device)
    y = torch.empty_like(x) if y is None else y
    rd = None if route_out is None else ctypes.byref(_route_desc(route_out))
    _check("moe_prefill", lib().moe_prefill(layer.ref, _ptr(x), T, _ptr(y), _ptr(residual), rd,
                                            _ptr(ws), ws.numel(), _stream(stream)))
    return y


def moe_decode(layer: DeviceLayer, x: torch.Tensor, y=None, residual=None, ws=None,
               stream=None) -> torch.Tensor:
    ws = _ws(layer, ws, 1, x.device)
    y = torch.empty_like(x) if y is None else y
    _check("moe_decode", lib().moe_decode(layer.ref, _ptr(x), _ptr(y), _ptr(residual),
                                          _ptr(ws), ws.numel(), _stream(stream)))
    return y


def moe_decode_noalloc(layer: DeviceLayer, x: torch.Tensor, y=None, residual=None,
                       stream=None) -> torch.Tensor:
    """moe_decode on the library's static scratch memory (no workspace argument)."""
    y = torch.empty_like(x) if y is None else y
    _check("moe_decode_noalloc", lib().moe_decode_noalloc(layer.ref, _ptr(x), _ptr(y),
                                                          _ptr(residual), _stream(stream)))
    return y


def ablation_workspace(layer: DeviceLayer, max_tokens: int, variant: int,
                       device="cuda") -> torch.Tensor:
    n = ctypes.c_size_t(0)
    _check("moe_ablation_workspace_bytes",
           lib().moe_ablation_workspace_bytes(layer.ref, int(max_tokens), int(variant),
                                              ctypes.byref(n)))
    return torch.zeros(n.value, dtype=torch.uint8, device=device)


def moe_prefill_ablation(layer: DeviceLayer, x: torch.Tensor, variant: int, y=None,
                         residual=None, ws=None, stream=None) -> torch.Tensor:
    """The prefill path with one mechanism replaced by the pages' rejected design
    (ABL_* constants); the result is bit-identical to moe_prefill's grouped path."""
    T = x.shape[0]
    ws = ablation_workspace(layer, max(T, 1), variant, x.device) if ws is None else ws
    y = torch.empty_like(x) if y is None else y
    _check("moe_prefill_ablation",
           lib().moe_prefill_ablation(layer.ref, int(variant), _ptr(x), T, _ptr(y),
                                      _ptr(residual), _ptr(ws), ws.numel(), _stream(stream)))
    return y


def attn_workspace(n_q: int, n_kv: int, head_dim: int, max_ctx: int,
                   device="cuda") -> torch.Tensor:
    n = ctypes.c_size_t(0)
    _check("moe_attn_workspace_bytes",
           lib().moe_attn_workspace_bytes(int(n_q), int(n_kv), int(head_dim), int(max_ctx),
                                          ctypes.byref(n)))
    return torch.empty(n.value, dtype=torch.uint8, device=device)


def moe_attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, ctx=None,
                    scale=None, out=None, ws=None, packed: bool = True,
                    stream=None) -> torch.Tensor:
    """Decode attention of one token. q [n_q, D] bf16; k_cache, v_cache [n_kv, cap, D] bf16
    (contiguous; the first ctx positions are attended, ctx defaults to cap); scale defaults
    to 1 / sqrt(D). Returns out [n_q, D] bf16."""
    n_q, D = q.shape
    n_kv, cap, D2 = k_cache.shape
    if D2 != D or v_cache.shape != k_cache.shape:
        raise ValueError("q / cache shapes do not match")
    if not (q.is_contiguous() and k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("q and the caches must be contiguous")
    ctx = cap if ctx is None else int(ctx)
    scale = D ** -0.5 if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    ws = attn_workspace(n_q, n_kv, D, ctx, q.device) if ws is None else ws
    fn = lib().moe_attn_decode if packed else lib().moe_attn_decode_unpacked
    _check("moe_attn_decode", fn(_ptr(q), _ptr(k_cache), _ptr(v_cache), n_q, n_kv, D, ctx,
                                 cap * D, ctypes.c_float(scale), _ptr(out), _ptr(ws),
                                 ws.numel(), _stream(stream)))
    return out


def moe_gdn_scan(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                 beta: torch.Tensor, state: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """Gated DeltaNet recurrence over T tokens. q, k [T, n_k, 128] bf16; v [T, n_v, 128] bf16;
    alpha, beta [T, n_v] fp32; state [n_v, 128, 128] fp32 (updated in place to S_T).
    Returns out [T, n_v, 128] bf16."""
    T, n_k, d_k = q.shape
    n_v, d_v = v.shape[1], v.shape[2]
    for t in (q, k, v, alpha, beta, state):
        if not t.is_contiguous():
            raise ValueError("DeltaNet tensors must be contiguous")
    out = torch.empty((T, n_v, d_v), dtype=torch.bfloat16, device=q.device) if out is None else out
    _check("moe_gdn_scan", lib().moe_gdn_scan(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                              T, n_k, n_v, d_k, d_v, _ptr(state), _ptr(out),
                                              _stream(stream)))
    return out


def gdn_chunked_workspace(T: int, n_k: int, n_v: int, device="cuda") -> torch.Tensor:
    n = ctypes.c_size_t(0)
    _check("moe_gdn_chunked_workspace_bytes",
           lib().moe_gdn_chunked_workspace_bytes(int(T), n_k, n_v, 128, 128, ctypes.byref(n)))
    return torch.empty(n.value, dtype=torch.uint8, device=device)


def moe_gdn_scan_chunked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                         beta: torch.Tensor, state: torch.Tensor, out=None, ws=None,
                         stream=None) -> torch.Tensor:
    """moe_gdn_scan in its chunked form (32-token chunks; workspace as gdn_chunked_workspace)."""
    T, n_k, d_k = q.shape
    n_v, d_v = v.shape[1], v.shape[2]
    for t in (q, k, v, alpha, beta, state):
        if not t.is_contiguous():
            raise ValueError("DeltaNet tensors must be contiguous")
    out = torch.empty((T, n_v, d_v), dtype=torch.bfloat16, device=q.device) if out is None else out
    ws = gdn_chunked_workspace(max(T, 1), n_k, n_v, q.device) if ws is None else ws
    _check("moe_gdn_scan_chunked",
           lib().moe_gdn_scan_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), T, n_k,
                                      n_v, d_k, d_v, _ptr(state), _ptr(out), _ptr(ws),
                                      ws.numel(), _stream(stream)))
    return out


def moe_rmsnorm(h: torch.Tensor, eps: float = 1e-6, out=None, stream=None) -> torch.Tensor:
    out = torch.empty_like(h) if out is None else out
    act = ACT_BF16 if h.dtype == torch.bfloat16 else ACT_F32
    _check("moe_rmsnorm", lib().moe_rmsnorm(_ptr(h), h.shape[0], h.shape[1], float(eps), act,
                                            _ptr(out), _stream(stream)))
    return out


def decode_read_ceiling(layer: DeviceLayer, ids: torch.Tensor, part: int, sink: torch.Tensor,
                        stream=None):
    """The weight loads of decode kernel `part` (0 router, 1 gate/up, 2 down) with the
    arithmetic taken out (a measurement aid); ids: device int32 [k] selected experts."""
    _check("moe_decode_read_ceiling",
           lib().moe_decode_read_ceiling(layer.ref, _ptr(ids), int(part), _ptr(sink),
                                         _stream(stream)))


CEIL_FULL_MANTISSA, CEIL_LOW_ENTROPY = 0, 1


def mfma_ceiling(iters: int, sink: torch.Tensor, operands: int = CEIL_FULL_MANTISSA,
                 stream=None) -> float:
    """Launches the dense MFMA loop on full-mantissa (0) or low-entropy (1) operands; returns
    the FLOP it executes."""
    f = ctypes.c_double(0)
    _check("moe_mfma_ceiling", lib().moe_mfma_ceiling(int(iters), int(operands), _ptr(sink),
                                                      ctypes.byref(f), _stream(stream)))
    return f.value


def profile_enable(on: bool = True):
    _check("moe_profile_enable", lib().moe_profile_enable(1 if on else 0))


def profile_reset():
    _check("moe_profile_reset", lib().moe_profile_reset())


def profile_query(kernel: str) -> tuple[float, int]:
    ms, n = ctypes.c_double(0), ctypes.c_int64(0)
    _check("moe_profile_query", lib().moe_profile_query(kernel.encode(), ctypes.byref(ms),
                                                        ctypes.byref(n)))
    return ms.value, n.value


def bf16_from_bits(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """Device bf16 tensor holding the given bf16 bit patterns."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def _layer_array(layers):
    arr = (MoeLayer * len(layers))(*[l.desc for l in layers])
    return arr


def stack_workspace(layers, chunk_tokens: int, device="cuda") -> torch.Tensor:
    n = ctypes.c_size_t(0)
    _check("moe_stack_workspace_bytes",
           lib().moe_stack_workspace_bytes(_layer_array(layers), len(layers), int(chunk_tokens),
                                           ctypes.byref(n)))
    return torch.zeros(n.value, dtype=torch.uint8, device=device)


def moe_stack_forward(layers, h: torch.Tensor, chunk_tokens: int = 4096, eps: float = 1e-6,
                      ws: torch.Tensor = None, stream=None) -> torch.Tensor:
    """h <- h + MoE_l(RMSNorm(h)) for every layer in order, in place on h [T, H]."""
    if not h.is_contiguous():
        raise ValueError("h must be contiguous")
    if ws is None:
        ws = stack_workspace(layers, chunk_tokens, h.device)
    arr = _layer_array(layers)
    _check("moe_stack_forward",
           lib().moe_stack_forward(arr, len(layers), _ptr(h), h.shape[0], int(chunk_tokens),
                                   ctypes.c_float(eps), _ptr(ws), ws.numel(), _stream(stream)))
    return h
