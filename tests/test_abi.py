"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments before touching a device.  No compute call runs here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def L():
    from quantized_moe_transformer_amd import _lib
    return _lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\([^;{]*\)\s*;", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for fn in ("router_topk", "moe_layer_forward", "moe_layer_forward_shard",
               "moe_reduce_partials", "moe_dequant", "moe_workspace_bytes", "moe_route_bucket",
               "moe_status_str", "moe_abi_version", "moe_reduce_residual", "moe_rmsnorm",
               "moe_layer_forward_range", "moe_layer_forward_noalloc",
               "moe_rmsnorm_sumsq", "moe_rmsnorm_apply"):
        assert fn in names


def test_library_exports_every_declared_symbol(L):
    for fn in declared_functions():
        assert hasattr(L.lib, fn), fn
    assert L.moe_abi_version() == 6
    assert L.moe_status_str(-3) == "workspace too small"


FAKE = 0x10000   # an aligned non-null address; validation never dereferences it


def desc(H=2048, E=256, k=8, I=512, Is=512, **kw):
    from quantized_moe_transformer_amd._lib import moe_layer_desc
    d = moe_layer_desc(H, E, k, I, Is, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    for n, v in kw.items():
        setattr(d, n, v)
    return d


def test_workspace_bytes_host_only(L):
    d = desc()
    w1 = L.moe_workspace_bytes(d, 1, 1)
    w4096 = L.moe_workspace_bytes(d, 4096, 1)
    assert 0 < w1 < w4096
    # the grouped path keeps per-slot fp16 rows: T*k*H*2 bytes at least
    assert w4096 >= 4096 * 8 * 2048 * 2
    assert L.moe_workspace_bytes(d, 4096, 2) <= w4096
    assert L.moe_workspace_bytes(desc(k=0), 1, 1) == 0
    assert L.moe_workspace_bytes(desc(H=300), 1, 1) == 0
    assert L.moe_workspace_bytes(d, -1, 1) == 0
    assert L.moe_workspace_bytes(d, 1, 3) == 0          # 512 % 3 != 0


def test_weight_format_is_checked(L):
    # MXFP4 layers keep tokens and h as three MX-FP8 terms (3 bytes per value
    # plus scales) where K-quant layers keep fp16 (2 bytes); an unknown format
    # is an argument error
    kq = L.moe_workspace_bytes(desc(), 4096, 1)
    mx = L.moe_workspace_bytes(desc(weight_format=1), 4096, 1)
    assert kq < mx < kq + 4096 * 9 * 512 * 2 + 4096 * 2048 * 2
    assert L.moe_workspace_bytes(desc(weight_format=2), 1, 1) == 0
    assert raw_forward(L, desc(weight_format=2), 1) == -1
    assert raw_forward(L, desc(weight_format=-1), 1) == -1
    assert L.lib.moe_dequant(FAKE, 6, 1, 0, FAKE, None) == -1
    assert L.lib.moe_dequant(FAKE, L.MOE_SB_MXFP4, 0, 0, FAKE, None) == 0


def raw_forward(L, d, T, x=FAKE, out=FAKE, ws=FAKE, ws_bytes=1 << 40, path=0):
    o = L.moe_opts(path, None, None, 0)
    return L.lib.moe_layer_forward(ctypes.byref(d), x, T, out, ctypes.byref(o), ws, ws_bytes, None)


def raw_shard(L, d, T, shard, n, ws_bytes=1 << 40, idx=FAKE, w=FAKE):
    return L.lib.moe_layer_forward_shard(ctypes.byref(d), FAKE, T, idx, w, shard, n, FAKE, None,
                                         FAKE, ws_bytes, None)


def raw_range(L, d, T, i_begin, i_end, ws_bytes=1 << 40, idx=FAKE, w=FAKE):
    return L.lib.moe_layer_forward_range(ctypes.byref(d), FAKE, T, idx, w, i_begin, i_end, FAKE,
                                         None, FAKE, ws_bytes, None)


def test_argument_errors_before_any_launch(L):
    assert raw_forward(L, desc(k=0), 1) == L.MOE_EINVAL
    assert raw_forward(L, desc(k=17, E=32), 1) == L.MOE_EINVAL
    assert raw_forward(L, desc(k=9, E=8), 1) == L.MOE_EINVAL
    assert raw_forward(L, desc(router_w=None), 1) == L.MOE_EINVAL
    assert raw_forward(L, desc(sh_down_q=None), 1) == L.MOE_EINVAL
    assert raw_forward(L, desc(H=2304), 1) == L.MOE_EUNSUPPORTED     # 9 superblocks per row
    assert raw_forward(L, desc(I=500, Is=500), 1) == L.MOE_EUNSUPPORTED
    assert raw_forward(L, desc(Is=256), 1) == L.MOE_EUNSUPPORTED
    assert raw_forward(L, desc(gate_q=FAKE + 8), 1) == L.MOE_EUNSUPPORTED   # misaligned
    assert raw_forward(L, desc(), -1) == L.MOE_EINVAL
    assert raw_forward(L, desc(), 1, x=None) == L.MOE_EINVAL
    assert raw_forward(L, desc(), 1, ws_bytes=1024) == L.MOE_EWORKSPACE
    assert raw_forward(L, desc(), 1, path=7) == L.MOE_EINVAL
    assert raw_shard(L, desc(), 1, 2, 2) == L.MOE_EINVAL
    assert raw_shard(L, desc(), 1, -1, 2) == L.MOE_EINVAL
    assert raw_shard(L, desc(), 1, 0, 16) == L.MOE_EUNSUPPORTED     # 512/16 = 32 columns
    assert raw_shard(L, desc(), 1, 0, 2, idx=None) == L.MOE_EINVAL
    # moe_layer_forward_range: empty, reversed, out-of-range or misaligned rows
    assert raw_range(L, desc(), 1, 64, 64) == L.MOE_EINVAL
    assert raw_range(L, desc(), 1, 128, 64) == L.MOE_EINVAL
    assert raw_range(L, desc(), 1, 0, 576) == L.MOE_EINVAL
    assert raw_range(L, desc(), 1, -64, 64) == L.MOE_EINVAL
    assert raw_range(L, desc(), 1, 0, 160) == L.MOE_EUNSUPPORTED
    assert raw_range(L, desc(), 1, 0, 192, ws_bytes=1024) == L.MOE_EWORKSPACE
    # moe_reduce_partials: wrong shard count or a lost shard
    arr = (ctypes.c_void_p * 2)(FAKE, None)
    assert L.lib.moe_reduce_partials(arr, 2, 16, FAKE, None) == L.MOE_EINVAL
    assert L.lib.moe_reduce_partials(arr, 0, 16, FAKE, None) == L.MOE_EINVAL
    assert L.lib.moe_reduce_partials(arr, 17, 16, FAKE, None) == L.MOE_EINVAL
    assert L.lib.moe_dequant(FAKE, 6, 1, 0, FAKE, None) == L.MOE_EINVAL
    assert L.lib.moe_dequant(FAKE, 4, 1, 3, FAKE, None) == L.MOE_EINVAL


def test_norm_and_residual_argument_errors(L):
    f = ctypes.c_float
    # moe_rmsnorm: bad T, null pointers, negative or NaN eps, width or alignment
    assert L.lib.moe_rmsnorm(FAKE, -1, 2048, FAKE, f(1e-6), FAKE, None) == L.MOE_EINVAL
    assert L.lib.moe_rmsnorm(None, 4, 2048, FAKE, f(1e-6), FAKE, None) == L.MOE_EINVAL
    assert L.lib.moe_rmsnorm(FAKE, 4, 2048, FAKE, f(-1.0), FAKE, None) == L.MOE_EINVAL
    assert L.lib.moe_rmsnorm(FAKE, 4, 2048, FAKE, f(float("nan")), FAKE, None) == L.MOE_EINVAL
    assert L.lib.moe_rmsnorm(FAKE, 4, 2046, FAKE, f(1e-6), FAKE, None) == L.MOE_EUNSUPPORTED
    assert L.lib.moe_rmsnorm(FAKE + 4, 4, 2048, FAKE, f(1e-6), FAKE, None) == L.MOE_EUNSUPPORTED
    assert L.lib.moe_rmsnorm(None, 0, 2048, None, f(1e-6), None, None) == L.MOE_OK   # T = 0
    # shard form: row stride below the width, too many or no partial sums, H < cols
    assert L.lib.moe_rmsnorm_sumsq(FAKE, 4, 1024, 512, FAKE, None) == L.MOE_EUNSUPPORTED
    arr = (ctypes.c_void_p * 2)(FAKE, FAKE)
    assert L.lib.moe_rmsnorm_apply(FAKE, 4, 1024, 2048, arr, 0, 2048, FAKE, f(1e-6), FAKE,
                                   2048, None) == L.MOE_EINVAL
    assert L.lib.moe_rmsnorm_apply(FAKE, 4, 1024, 2048, arr, 17, 2048, FAKE, f(1e-6), FAKE,
                                   2048, None) == L.MOE_EINVAL
    assert L.lib.moe_rmsnorm_apply(FAKE, 4, 1024, 2048, arr, 2, 512, FAKE, f(1e-6), FAKE,
                                   2048, None) == L.MOE_EINVAL
    lost = (ctypes.c_void_p * 2)(FAKE, None)
    assert L.lib.moe_rmsnorm_apply(FAKE, 4, 1024, 2048, lost, 2, 2048, FAKE, f(1e-6), FAKE,
                                   2048, None) == L.MOE_EINVAL
    # moe_reduce_residual: the residual is required
    assert L.lib.moe_reduce_residual(arr, 2, 16, None, FAKE, None) == L.MOE_EINVAL
    assert L.lib.moe_reduce_residual(lost, 2, 16, FAKE, FAKE, None) == L.MOE_EINVAL
    assert L.lib.moe_reduce_residual(arr, 2, 0, None, None, None) == L.MOE_OK


def test_empty_batch_is_a_no_op(L):
    # T = 0 passes validation and enqueues nothing (no device needed)
    used = ctypes.c_int32(-1)
    o = L.moe_opts(0, ctypes.pointer(used), None, 0)
    d = desc()
    assert L.lib.moe_layer_forward(ctypes.byref(d), None, 0, None, ctypes.byref(o), None, 0,
                                   None) == L.MOE_OK
    assert used.value == L.MOE_PATH_GEMV
    assert L.lib.router_topk(ctypes.byref(d), None, 0, None, None, None, 0, None) == L.MOE_OK
    assert L.lib.moe_dequant(None, 4, 0, 0, None, None) == L.MOE_OK


@pytest.mark.parametrize("fmt,cases", [
    (0, [(1, 0, 1), (17, 0, 1), (18, 0, 2), (32, 0, 2), (1, 2, 2), (4096, 1, 1)]),
    (1, [(1, 0, 1), (26, 0, 1), (27, 0, 2), (4096, 0, 2), (1, 2, 2)]),
])
def test_path_choice_reported(L, fmt, cases):
    # the automatic rule's crossover depends on the weight format
    d = desc(weight_format=fmt)
    for T, path, expect in cases:
        used = ctypes.c_int32(-1)
        o = L.moe_opts(path, ctypes.pointer(used), None, 0)
        # a too-small workspace stops the call after the path is chosen
        rc = L.lib.moe_layer_forward(ctypes.byref(d), FAKE, T, FAKE, ctypes.byref(o), FAKE, 16,
                                     None)
        assert rc == L.MOE_EWORKSPACE
        assert used.value == expect


def test_noalloc_host_checks(L):
    # moe_layer_forward_noalloc: T = 0 is a no-op, bad arguments are rejected,
    # and rows whose workspace would exceed the fixed scratch give MOE_ETOOBIG
    # before any device is touched
    f = L.lib.moe_layer_forward_noalloc
    used = ctypes.c_int32(-1)
    o = L.moe_opts(0, ctypes.pointer(used), None, 0)
    d = desc()
    assert f(ctypes.byref(d), None, 0, None, ctypes.byref(o), None) == L.MOE_OK
    assert used.value == L.MOE_PATH_GEMV
    assert f(ctypes.byref(desc(k=0)), FAKE, 1, FAKE, ctypes.byref(o), None) == L.MOE_EINVAL
    assert f(ctypes.byref(d), FAKE, -1, FAKE, ctypes.byref(o), None) == L.MOE_EINVAL
    fits = [T for T in range(1, 4097) if L.moe_workspace_bytes(d, T, 1) <= L.MOE_NOALLOC_SCRATCH_BYTES]
    big = max(fits) + 1
    assert fits == list(range(1, big)) and big > 256     # every decode and mid-size T fits
    assert f(ctypes.byref(d), FAKE, big, FAKE, ctypes.byref(o), None) == L.MOE_ETOOBIG
    assert f(ctypes.byref(d), FAKE, 4096, FAKE, ctypes.byref(o), None) == L.MOE_ETOOBIG
    assert L.moe_status_str(L.MOE_ETOOBIG) == "input too large for the no-allocation scratch"
