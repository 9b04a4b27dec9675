"""CPU oracle of the routed-expert MoE layer, of grouped-query decode attention and of the
Gated DeltaNet recurrence (plain C, fp64), with a ctypes wrapper.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module. The product path (the HIP
library and its binding) never imports, links or runs it, and shares no code with it.

Source of the arithmetic: "Optimizing On-Device Inference for Apple Silicon"
(sections "Qwen creates three distinct workload shapes", "Dequantize weights during
matrix multiplication", "Keep expert routing on the GPU", "Reduce intermediate and
state traffic"; attention: "Qwen creates three distinct workload shapes" and "Read the
attention cache efficiently"; DeltaNet: "Qwen creates three distinct workload shapes" and
"Keep recurrent state on chip"); the readings taken where the page is silent are listed in
``moe_oracle.c``.

Pinning: every function here is checked in ``tests/test_oracle_pins.py`` against
closed forms, invariants, library routines (torch fp64 linear/silu, scipy softmax)
and brute force on tiny inputs. Nothing in the oracle is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
FMT_F32, FMT_INT4 = 0, 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared",
                        "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Layer(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("fmt", ctypes.c_int32),
                ("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
                ("w13_q", ctypes.c_void_p), ("w2_q", ctypes.c_void_p),
                ("w13_s", ctypes.c_void_p), ("w13_b", ctypes.c_void_p),
                ("w2_s", ctypes.c_void_p), ("w2_b", ctypes.c_void_p),
                ("w13_f", ctypes.c_void_p), ("w2_f", ctypes.c_void_p)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = ctypes.CDLL(_LIB)
        P, I64, I32, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        sigs = {
            "oracle_check_layer": [P],
            "oracle_dequant": [P, P, P, I64, I64, P],
            "oracle_logits": [P, P, I64, P],
            "oracle_route": [P, P, I64, P, P, P],
            "oracle_group": [P, P, I64, P, P, P, P],
            "oracle_expert": [P, I32, P, P],
            "oracle_moe": [P, P, I64, P, ctypes.c_int],
            "oracle_rmsnorm": [P, I64, I32, D, P],
            "oracle_attn_decode": [P, P, P, I32, I32, I32, I64, I64, D, P],
            "oracle_gdn_scan": [P, P, P, P, P, I64, I32, I32, I32, I32, P, P, ctypes.c_int],
        }
        for name, args in sigs.items():
            fn = getattr(_lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        _lib.oracle_bf16_to_f64.argtypes = [P, I64, P]
        _lib.oracle_bf16_to_f64.restype = None
        _lib.oracle_round_bf16.argtypes = [P, I64, P]
        _lib.oracle_round_bf16.restype = None
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


class OracleLayer:
    """Keeps the numpy arrays of a layer alive and exposes the C descriptor."""

    def __init__(self, layer):
        c = lambda a, dt: None if a is None else np.ascontiguousarray(a, dtype=dt)
        self.layer = layer
        self._keep = {
            "router_w": c(layer.router_w, np.float32),
            "router_b": c(layer.router_b, np.float32),
            "w13_q": c(layer.w13_q, np.uint8), "w2_q": c(layer.w2_q, np.uint8),
            "w13_s": c(layer.w13_s, np.uint16), "w13_b": c(layer.w13_b, np.uint16),
            "w2_s": c(layer.w2_s, np.uint16), "w2_b": c(layer.w2_b, np.uint16),
            "w13_f": c(layer.w13, np.float32), "w2_f": c(layer.w2, np.float32),
        }
        k = self._keep
        self.desc = _Layer(layer.hidden, layer.inter, layer.n_experts, layer.top_k,
                           layer.n_shared, FMT_INT4 if layer.fmt == "int4" else FMT_F32,
                           *[_ptr(k[n]) for n in ("router_w", "router_b", "w13_q", "w2_q",
                                                   "w13_s", "w13_b", "w2_s", "w2_b",
                                                   "w13_f", "w2_f")])
        if _load().oracle_check_layer(ctypes.byref(self.desc)) != 0:
            raise ValueError("invalid layer for the oracle")

    @property
    def ref(self):
        return ctypes.byref(self.desc)


def _as_layer(layer):
    return layer if isinstance(layer, OracleLayer) else OracleLayer(layer)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed")


def to_f64(x) -> np.ndarray:
    """Activations to float64: uint16 arrays are bf16 bit patterns, float arrays as is."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        out = np.empty(x.shape, dtype=np.float64)
        _load().oracle_bf16_to_f64(x.ctypes.data, x.size, out.ctypes.data)
        return out
    return x.astype(np.float64)


def dequant(codes, scale, bias) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    rows, half = codes.shape
    out = np.empty((rows, 2 * half), dtype=np.float64)
    _check(_load().oracle_dequant(codes.ctypes.data,
                                  np.ascontiguousarray(scale, dtype=np.uint16).ctypes.data,
                                  np.ascontiguousarray(bias, dtype=np.uint16).ctypes.data,
                                  rows, 2 * half, out.ctypes.data), "dequant")
    return out


def logits(layer, x) -> np.ndarray:
    L = _as_layer(layer)
    x = to_f64(x)
    T = x.shape[0]
    z = np.empty((T, L.layer.n_experts), dtype=np.float64)
    _check(_load().oracle_logits(L.ref, x.ctypes.data, T, z.ctypes.data), "logits")
    return z


def route(layer, x):
    """Returns (ids int32 [T,k] ascending, w float64 [T,k], margin float64 [T])."""
    L = _as_layer(layer)
    x = to_f64(x)
    T, k = x.shape[0], L.layer.top_k
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    margin = np.empty(T, dtype=np.float64)
    _check(_load().oracle_route(L.ref, x.ctypes.data, T, ids.ctypes.data, w.ctypes.data,
                                margin.ctypes.data), "route")
    return ids, w, margin


def group(layer, ids):
    """Returns (counts [E], offsets [E+1], sorted_tok [kT], slot_of [T,k]) as int32."""
    L = _as_layer(layer)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, E, k = ids.shape[0], L.layer.n_experts, L.layer.top_k
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    sorted_tok = np.empty(T * k, dtype=np.int32)
    slot_of = np.empty((T, k), dtype=np.int32)
    _check(_load().oracle_group(L.ref, ids.ctypes.data, T, counts.ctypes.data,
                                offsets.ctypes.data, sorted_tok.ctypes.data,
                                slot_of.ctypes.data), "group")
    return counts, offsets, sorted_tok, slot_of


def expert(layer, e, x_row) -> np.ndarray:
    L = _as_layer(layer)
    x = to_f64(x_row).reshape(-1)
    out = np.empty(L.layer.hidden, dtype=np.float64)
    _check(_load().oracle_expert(L.ref, int(e), x.ctypes.data, out.ctypes.data), "expert")
    return out


def moe(layer, x, nthreads: int = 0) -> np.ndarray:
    L = _as_layer(layer)
    x = to_f64(x)
    T = x.shape[0]
    y = np.empty((T, L.layer.hidden), dtype=np.float64)
    _check(_load().oracle_moe(L.ref, x.ctypes.data, T, y.ctypes.data, int(nthreads)), "moe")
    return y


def rmsnorm(h, eps: float = 1e-6) -> np.ndarray:
    h = to_f64(h)
    T, H = h.shape
    out = np.empty_like(h)
    _check(_load().oracle_rmsnorm(h.ctypes.data, T, H, eps, out.ctypes.data), "rmsnorm")
    return out


def round_bf16(x) -> np.ndarray:
    """Nearest bf16 of each value (ties to even, one rounding from the exact value);
    returns uint16 bit patterns of the same shape."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_round_bf16(x.ctypes.data, x.size, out.ctypes.data)
    return out


def stack_layer_input(h, eps: float = 1e-6) -> np.ndarray:
    """What one layer of the stack reads: RMSNorm (unit gain) of the residual stream h,
    rounded to bf16 (bit patterns)."""
    return round_bf16(rmsnorm(h, eps))


def attn_decode(q, k, v, n_q: int, n_kv: int, scale: float) -> np.ndarray:
    """Decode attention of one token (fp64). q [n_q, D] (bf16 bits or floats); k, v bf16 bit
    patterns [n_kv, ctx, D]. Returns out [n_q, D] float64."""
    q = to_f64(q)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    n_kv_, ctx, D = k.shape
    if n_kv_ != n_kv or v.shape != k.shape or q.shape != (n_q, D):
        raise ValueError("attention shapes do not match")
    out = np.empty((n_q, D), dtype=np.float64)
    _check(_load().oracle_attn_decode(q.ctypes.data, k.ctypes.data, v.ctypes.data, n_q, n_kv,
                                      D, ctx, ctx * D, float(scale), out.ctypes.data),
           "attn_decode")
    return out


def gdn_scan(q, k, v, alpha, beta, n_k: int, n_v: int, state0=None, nthreads: int = 0):
    """Gated DeltaNet recurrence (fp64). q, k bf16 bits [T, n_k, d_k]; v bf16 bits
    [T, n_v, d_v]; alpha, beta float32 [T, n_v]; state0 [n_v, d_v, d_k] or None (zeros).
    Returns (out [T, n_v, d_v] float64, final state [n_v, d_v, d_k] float64)."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    alpha = np.ascontiguousarray(alpha, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    T, nk_, d_k = q.shape
    d_v = v.shape[2]
    if nk_ != n_k or k.shape != q.shape or v.shape[:2] != (T, n_v) or alpha.shape != (T, n_v) \
            or beta.shape != (T, n_v):
        raise ValueError("DeltaNet shapes do not match")
    state = np.zeros((n_v, d_v, d_k)) if state0 is None else np.array(state0, dtype=np.float64)
    out = np.empty((T, n_v, d_v), dtype=np.float64)
    _check(_load().oracle_gdn_scan(q.ctypes.data, k.ctypes.data, v.ctypes.data,
                                   alpha.ctypes.data, beta.ctypes.data, T, n_k, n_v, d_k, d_v,
                                   state.ctypes.data, out.ctypes.data, int(nthreads)),
           "gdn_scan")
    return out, state
