"""CPU oracle for the routed MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path
(``quantized_moe_transformer_amd``) never imports it and shares no code with it.

The arithmetic lives in ``moe_oracle.c`` (plain C, double precision, built with
gcc, no fused multiply-add contraction); this module only builds it and
marshals numpy arrays into it.  See the header of ``moe_oracle.c`` for the
passages of the pages each function follows and for the readings taken where
they are silent.

Pins (tests/test_oracle.py): a hand-worked superblock of each format (the two
K-quant ones and MXFP4, whose element values are also checked against the E2M1
table of the OCP MX specification), an
exhaustive closed-form sweep of every (scale, min, code) field, a brute-force
sort for the router on tiny inputs with constructed ties, closed-form FFN cases
(silu at +-ln 3, constant weights), a two-expert mixture with known softmax
weights, the dense-FFN special case, and the shard-sum invariant.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile moe_oracle.c into liboracle.so (gcc, -O2, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                               "-shared", "-fPIC", "-Wall", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


class _Layer(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("I", ctypes.c_int32), ("Is", ctypes.c_int32), ("shared_weight", ctypes.c_float),
                ("router_w", ctypes.c_void_p), ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p),
                ("down", ctypes.c_void_p), ("sh_gate", ctypes.c_void_p), ("sh_up", ctypes.c_void_p),
                ("sh_down", ctypes.c_void_p), ("fmt", ctypes.c_int32)]

SB_MXFP4 = 14   # oracle_dequant's code for the MXFP4 superblock


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_half_to_double.restype = ctypes.c_double
        L.oracle_e2m1.argtypes = [ctypes.c_int]
        L.oracle_e2m1.restype = ctypes.c_double
        L.oracle_e8m0.argtypes = [ctypes.c_int]
        L.oracle_e8m0.restype = ctypes.c_double
        L.oracle_dequant.argtypes = [P, ctypes.c_int, ctypes.c_int64, P]
        L.oracle_router.argtypes = [P, ctypes.c_int, ctypes.c_int, P, ctypes.c_int, ctypes.c_int,
                                    P, P, P, P]
        L.oracle_bucket.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P, P, P]
        L.oracle_forward.argtypes = [ctypes.POINTER(_Layer), P, ctypes.c_int, P, P,
                                     ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int]
        L.oracle_reduce.argtypes = [ctypes.POINTER(P), ctypes.c_int, ctypes.c_int64, P]
        L.oracle_forward_range.argtypes = [ctypes.POINTER(_Layer), P, ctypes.c_int, P, P,
                                           ctypes.c_int, ctypes.c_int, P, P, ctypes.c_int]
        L.oracle_sumsq.argtypes = [P, ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int, P]
        L.oracle_rmsnorm.argtypes = [P, ctypes.c_int, ctypes.c_int, P, ctypes.c_float, P]
        L.oracle_reduce_residual.argtypes = [ctypes.POINTER(P), ctypes.c_int, ctypes.c_int64, P, P]
        L.oracle_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with status {rc}")


def half_to_double(bits: int) -> float:
    return lib().oracle_half_to_double(bits)


def max_threads() -> int:
    return lib().oracle_max_threads()


def e2m1(code: int) -> float:
    return lib().oracle_e2m1(code)


def e8m0(s: int) -> float:
    return lib().oracle_e8m0(s)


def dequant(blob: np.ndarray, bits: int) -> np.ndarray:
    """Decode a flat blob of superblocks into fp32 (flat order); bits = 4 (Q4_K),
    5 (Q5_K) or SB_MXFP4."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8).reshape(-1)
    sbb = 176 if bits == 5 else 144
    if blob.size % sbb:
        raise ValueError("blob size is not a whole number of superblocks")
    n_sb = blob.size // sbb
    out = np.empty(n_sb * 256, dtype=np.float32)
    _check(lib().oracle_dequant(_p(blob), bits, n_sb, _p(out)), "dequant")
    return out


def router(x: np.ndarray, wr: np.ndarray, k: int):
    """(idx int32 [T][k], w fp32 [T][k], w double [T][k], logits double [T][E])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    wr = np.ascontiguousarray(wr, dtype=np.float32)
    T, H = x.shape
    E = wr.shape[1]
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    wd = np.empty((T, k), dtype=np.float64)
    logits = np.empty((T, E), dtype=np.float64)
    _check(lib().oracle_router(_p(x), T, H, _p(wr), E, k, _p(logits), _p(idx), _p(w), _p(wd)),
           "router")
    return idx, w, wd, logits


def bucket(idx: np.ndarray, E: int):
    """(counts [E], offsets [E+1], perm [T*k], inv_pos [T*k]) of a routing."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    inv = np.empty(T * k, np.int32)
    _check(lib().oracle_bucket(_p(idx), T, k, E, _p(counts), _p(offsets), _p(perm), _p(inv)),
           "bucket")
    return counts, offsets, perm, inv


class Layer:
    """Host-side layer description for the oracle (keeps the arrays alive)."""

    def __init__(self, arrays: dict, H: int, E: int, k: int, I: int, Is: int,
                 shared_weight: float = 1.0, fmt: int = 0):
        self.arrays = {n: np.ascontiguousarray(a) for n, a in arrays.items()}
        a = self.arrays
        self.c = _Layer(H, E, k, I, Is, shared_weight, _p(a["router_w"]), _p(a["gate"]),
                        _p(a["up"]), _p(a["down"]), _p(a.get("sh_gate")), _p(a.get("sh_up")),
                        _p(a.get("sh_down")), fmt)
        self.H, self.E, self.k, self.I, self.Is, self.fmt = H, E, k, I, Is, fmt

    @classmethod
    def from_shape(cls, arrays: dict, shape) -> "Layer":
        return cls(arrays, shape.H, shape.E, shape.k, shape.I, shape.Is, shape.shared_weight,
                   getattr(shape, "fmt", 0))


def forward(layer: Layer, x: np.ndarray, idx: Optional[np.ndarray] = None,
            w: Optional[np.ndarray] = None, shard: int = 0, num_shards: int = 1,
            nthreads: int = 0, want_double: bool = False):
    """The layer (or one shard of it) on token rows x fp32 [T][H].

    idx/w: a given routing (the synchronised router decision); None = route here.
    Returns fp32 [T][H] (and the unrounded double result if want_double)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    T = x.shape[0]
    out = np.empty((T, layer.H), np.float32)
    out_d = np.empty((T, layer.H), np.float64) if want_double else None
    if idx is not None:
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        w = np.ascontiguousarray(w, dtype=np.float32)
    _check(lib().oracle_forward(ctypes.byref(layer.c), _p(x), T, _p(idx), _p(w), shard,
                                num_shards, _p(out), _p(out_d), nthreads), "forward")
    return (out, out_d) if want_double else out


def reduce_partials(partials: Sequence[np.ndarray]) -> np.ndarray:
    ps = [np.ascontiguousarray(p, dtype=np.float32) for p in partials]
    n = ps[0].size
    arr = (ctypes.c_void_p * len(ps))(*[p.ctypes.data for p in ps])
    out = np.empty_like(ps[0])
    _check(lib().oracle_reduce(arr, len(ps), n, _p(out)), "reduce")
    return out


def sumsq(x: np.ndarray, c0: int = 0, c1: Optional[int] = None) -> np.ndarray:
    """Per-row sum of squares of columns [c0, c1) (double)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    T, H = x.shape
    c1 = H if c1 is None else c1
    out = np.empty(T, np.float64)
    _check(lib().oracle_sumsq(_p(x), T, H, c0, c1, _p(out)), "sumsq")
    return out


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of each row: g * x / sqrt(mean(x^2) + eps), fp32 result."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    g = np.ascontiguousarray(g, dtype=np.float32)
    T, H = x.shape
    out = np.empty_like(x)
    _check(lib().oracle_rmsnorm(_p(x), T, H, _p(g), ctypes.c_float(eps), _p(out)), "rmsnorm")
    return out


def reduce_residual(partials: Sequence[np.ndarray], residual: np.ndarray) -> np.ndarray:
    """(p_0 + ... + p_{n-1}) + residual, in double, rounded once."""
    ps = [np.ascontiguousarray(p, dtype=np.float32) for p in partials]
    r = np.ascontiguousarray(residual, dtype=np.float32)
    arr = (ctypes.c_void_p * len(ps))(*[p.ctypes.data for p in ps])
    out = np.empty_like(ps[0])
    _check(lib().oracle_reduce_residual(arr, len(ps), ps[0].size, _p(r), _p(out)), "reduce_residual")
    return out


def forward_range(layer: Layer, x: np.ndarray, idx: np.ndarray, w: np.ndarray, i_begin: int,
                  i_end: int, nthreads: int = 0, want_double: bool = False):
    """A shard of any width: intermediate rows [i_begin, i_end) of every routed
    expert and of the shared one, under the given routing."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    T = x.shape[0]
    out = np.empty((T, layer.H), np.float32)
    out_d = np.empty((T, layer.H), np.float64) if want_double else None
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    _check(lib().oracle_forward_range(ctypes.byref(layer.c), _p(x), T, _p(idx), _p(w), i_begin,
                                      i_end, _p(out), _p(out_d), nthreads), "forward_range")
    return (out, out_d) if want_double else out
