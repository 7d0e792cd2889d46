"""ctypes binding of libmoe_hip.so: argument marshalling only.

Every function here has the name of the C entry point it calls (include/moe.h)
and does nothing but turn torch device tensors into pointers, pick the current
HIP stream, call, and raise on a non-zero status.  All arithmetic runs in the
HIP kernels of the library; there is no fallback: if the library is missing
the import fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_hip.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_ELAUNCH, MOE_ENODEVICE = 0, -1, -2, -3, -4, -5
MOE_ETOOBIG = -6
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20
MOE_PATH_AUTO, MOE_PATH_GEMV, MOE_PATH_MFMA = 0, 1, 2
MOE_WFMT_KQUANT, MOE_WFMT_MXFP4 = 0, 1
MOE_SB_MXFP4 = 14
# kernel ids for moe_opts.kernel_events (include/moe.h MOE_K_*)
KERNEL_IDS = {"gemv_front": 0, "router_mfma": 1, "router_topk": 2, "gateup_gemv": 3,
              "down_gemv": 4, "x_f16": 5, "bucket_hist": 6, "bucket_scan": 7, "bucket_scatter": 8,
              "gemm_gateup": 9, "gemm_down": 10, "combine": 11, "x_mx": 12}
N_KERNEL_IDS = 13


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({moe_status_str(status)})")
        self.status = status


class moe_layer_desc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("shared_weight", ctypes.c_float),
                ("router_w", ctypes.c_void_p), ("gate_q", ctypes.c_void_p),
                ("up_q", ctypes.c_void_p), ("down_q", ctypes.c_void_p),
                ("sh_gate_q", ctypes.c_void_p), ("sh_up_q", ctypes.c_void_p),
                ("sh_down_q", ctypes.c_void_p), ("weight_format", ctypes.c_int32)]


class moe_opts(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("path_used", ctypes.POINTER(ctypes.c_int32)),
                ("kernel_events", ctypes.POINTER(ctypes.c_void_p)), ("n_kernel_events", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python quantized_moe_transformer_amd/build.py`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D = ctypes.POINTER(moe_layer_desc)
    O = ctypes.POINTER(moe_opts)
    L.moe_abi_version.restype = ctypes.c_int
    L.moe_status_str.argtypes = [ctypes.c_int]
    L.moe_status_str.restype = ctypes.c_char_p
    L.moe_workspace_bytes.argtypes = [D, I32, I32]
    L.moe_workspace_bytes.restype = SZ
    L.router_topk.argtypes = [D, P, I32, P, P, P, SZ, P]
    L.moe_layer_forward.argtypes = [D, P, I32, P, O, P, SZ, P]
    L.moe_layer_forward_noalloc.argtypes = [D, P, I32, P, O, P]
    L.moe_layer_forward_shard.argtypes = [D, P, I32, P, P, I32, I32, P, O, P, SZ, P]
    L.moe_layer_forward_range.argtypes = [D, P, I32, P, P, I32, I32, P, O, P, SZ, P]
    L.moe_reduce_partials.argtypes = [ctypes.POINTER(P), I32, I64, P, P]
    L.moe_dequant.argtypes = [P, I32, I64, I32, P, P]
    L.moe_route_bucket.argtypes = [D, P, I32, P, P, P, P, SZ, P]
    L.moe_reduce_residual.argtypes = [ctypes.POINTER(P), I32, I64, P, P, P]
    L.moe_rmsnorm.argtypes = [P, I32, I32, P, ctypes.c_float, P, P]
    L.moe_rmsnorm_sumsq.argtypes = [P, I32, I32, I64, P, P]
    L.moe_rmsnorm_apply.argtypes = [P, I32, I32, I64, ctypes.POINTER(P), I32, I32, P,
                                    ctypes.c_float, P, I64, P]
    for f in ("router_topk", "moe_layer_forward", "moe_layer_forward_shard", "moe_reduce_partials",
              "moe_layer_forward_noalloc",
              "moe_dequant", "moe_route_bucket", "moe_reduce_residual", "moe_rmsnorm",
              "moe_layer_forward_range",
              "moe_rmsnorm_sumsq", "moe_rmsnorm_apply"):
        getattr(L, f).restype = ctypes.c_int
    return L


lib = _load()


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status)


def moe_abi_version() -> int:
    return lib.moe_abi_version()


def moe_status_str(status: int) -> str:
    return lib.moe_status_str(status).decode()


def make_desc(hidden, n_experts, top_k, inter, shared_inter, shared_weight, router_w, gate_q,
              up_q, down_q, sh_gate_q=None, sh_up_q=None, sh_down_q=None,
              weight_format=MOE_WFMT_KQUANT) -> moe_layer_desc:
    """A descriptor over device tensors (the caller keeps the tensors alive)."""
    return moe_layer_desc(hidden, n_experts, top_k, inter, shared_inter, shared_weight,
                          _ptr(router_w), _ptr(gate_q), _ptr(up_q), _ptr(down_q),
                          _ptr(sh_gate_q), _ptr(sh_up_q), _ptr(sh_down_q), weight_format)


def moe_workspace_bytes(desc: moe_layer_desc, T: int, num_shards: int = 1) -> int:
    return lib.moe_workspace_bytes(ctypes.byref(desc), T, num_shards)


def router_topk(desc, x, T, topk_idx, topk_w, ws, stream=None):
    _check("router_topk", lib.router_topk(ctypes.byref(desc), _ptr(x), T, _ptr(topk_idx),
                                          _ptr(topk_w), _ptr(ws), _nbytes(ws), _stream(stream)))


def _opts(path: int, events=None):
    used = ctypes.c_int32(-1)
    if events is None:
        return moe_opts(path, ctypes.pointer(used), None, 0), used
    return moe_opts(path, ctypes.pointer(used), events, len(events)), used


def moe_layer_forward(desc, x, T, out, ws, path: int = MOE_PATH_AUTO, stream=None,
                      events=None) -> int:
    """Returns the path that ran.  `events`: optional ctypes array of hipEvent_t,
    start/stop pairs per kernel id (moe_opts.kernel_events in include/moe.h)."""
    o, used = _opts(path, events)
    _check("moe_layer_forward", lib.moe_layer_forward(ctypes.byref(desc), _ptr(x), T, _ptr(out),
                                                      ctypes.byref(o), _ptr(ws), _nbytes(ws),
                                                      _stream(stream)))
    return used.value


def moe_layer_forward_noalloc(desc, x, T, out, path: int = MOE_PATH_AUTO, stream=None,
                              events=None) -> int:
    """moe_layer_forward on the library's fixed per-device scratch (no
    workspace argument).  Returns the path that ran."""
    o, used = _opts(path, events)
    _check("moe_layer_forward_noalloc",
           lib.moe_layer_forward_noalloc(ctypes.byref(desc), _ptr(x), T, _ptr(out),
                                         ctypes.byref(o), _stream(stream)))
    return used.value


def moe_layer_forward_shard(desc, x, T, topk_idx, topk_w, shard, num_shards, partial, ws,
                            path: int = MOE_PATH_AUTO, stream=None, events=None) -> int:
    o, used = _opts(path, events)
    _check("moe_layer_forward_shard",
           lib.moe_layer_forward_shard(ctypes.byref(desc), _ptr(x), T, _ptr(topk_idx),
                                       _ptr(topk_w), shard, num_shards, _ptr(partial),
                                       ctypes.byref(o), _ptr(ws), _nbytes(ws), _stream(stream)))
    return used.value


def moe_layer_forward_range(desc, x, T, topk_idx, topk_w, i_begin, i_end, partial, ws,
                            path: int = MOE_PATH_AUTO, stream=None, events=None) -> int:
    o, used = _opts(path, events)
    _check("moe_layer_forward_range",
           lib.moe_layer_forward_range(ctypes.byref(desc), _ptr(x), T, _ptr(topk_idx),
                                       _ptr(topk_w), i_begin, i_end, _ptr(partial),
                                       ctypes.byref(o), _ptr(ws), _nbytes(ws), _stream(stream)))
    return used.value


def moe_reduce_partials(partials: Sequence, n_elems: int, out, stream=None):
    arr = (ctypes.c_void_p * len(partials))(*[_ptr(p) for p in partials])
    _check("moe_reduce_partials", lib.moe_reduce_partials(arr, len(partials), n_elems, _ptr(out),
                                                          _stream(stream)))


def moe_reduce_residual(partials: Sequence, n_elems: int, residual, out, stream=None):
    arr = (ctypes.c_void_p * len(partials))(*[_ptr(p) for p in partials])
    _check("moe_reduce_residual", lib.moe_reduce_residual(arr, len(partials), n_elems,
                                                          _ptr(residual), _ptr(out),
                                                          _stream(stream)))


def _rows(t):
    """(rows, columns, row stride in elements) of a 2-D fp32 view with unit
    column stride (a whole tensor, or a column slice of one)."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D view with contiguous columns")
    return t.shape[0], t.shape[1], t.stride(0)


def moe_rmsnorm(x, g, eps: float, y, stream=None):
    T, H, ld = _rows(x)
    if ld != H or y.shape != x.shape:
        raise ValueError("moe_rmsnorm takes whole contiguous rows")
    _check("moe_rmsnorm", lib.moe_rmsnorm(_ptr(x), T, H, _ptr(g), ctypes.c_float(eps), _ptr(y),
                                          _stream(stream)))


def moe_rmsnorm_sumsq(x, ssq, stream=None):
    T, cols, ld = _rows(x)
    _check("moe_rmsnorm_sumsq", lib.moe_rmsnorm_sumsq(_ptr(x), T, cols, ld, _ptr(ssq),
                                                      _stream(stream)))


def moe_rmsnorm_apply(x, ssq_parts: Sequence, H: int, g, eps: float, y, stream=None):
    T, cols, ldx = _rows(x)
    _, _, ldy = _rows(y)
    arr = (ctypes.c_void_p * len(ssq_parts))(*[_ptr(p) for p in ssq_parts])
    _check("moe_rmsnorm_apply", lib.moe_rmsnorm_apply(_ptr(x), T, cols, ldx, arr, len(ssq_parts),
                                                      H, _ptr(g), ctypes.c_float(eps), _ptr(y),
                                                      ldy, _stream(stream)))


def moe_dequant(sbs, bits: int, n_sb: int, out_dtype: int, out, stream=None):
    _check("moe_dequant", lib.moe_dequant(_ptr(sbs), bits, n_sb, out_dtype, _ptr(out),
                                          _stream(stream)))


def moe_route_bucket(desc, topk_idx, T, counts, offsets, perm, ws, stream=None):
    _check("moe_route_bucket", lib.moe_route_bucket(ctypes.byref(desc), _ptr(topk_idx), T,
                                                    _ptr(counts), _ptr(offsets), _ptr(perm),
                                                    _ptr(ws), _nbytes(ws), _stream(stream)))
