"""GPU parity of the MXFP4 weight format (through the C ABI) against the oracle.

Same bars as the K-quant layer: decoded weights bit-exact (fp32, and the
round-to-nearest-even fp16 / bf16 of that value); layer outputs within
max|err|/RMS <= 1e-4 on the fp32 GEMV path and <= 1e-2 on the fp16 MFMA path;
shard partials against the oracle's partials and their reduction against the
whole layer.
"""
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import moe_inputs as mi  # noqa: E402
import oracle  # noqa: E402
from kquant_pack import pack_mx_sb, read_fixture  # noqa: E402
from parity_util import GEMV_TOL, MFMA_TOL, rel_err, topk_check  # noqa: E402

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import quantized_moe_transformer_amd as qm  # noqa: E402
from quantized_moe_transformer_amd.layer import DeviceLayer  # noqa: E402
from test_gpu_parity import (DEV, check_dequant_bitwise, check_layer, dev_layer,  # noqa: E402
                             gpu, gpu_dequant, rel_scale, run_router, run_shard, say)

SB = qm.MOE_SB_MXFP4


def test_mx_dequant_handworked():
    fx = read_fixture(os.path.join(os.path.dirname(__file__), "golden", "mxfp4_handworked.txt"))
    blob = np.frombuffer(fx["scales"] + fx["reserved"] + fx["mx_qs"], np.uint8)
    w = gpu_dequant(blob, SB, 0).numpy()
    for i, v in fx["mx_values"].items():
        assert w[i] == np.float32(float(v)), (i, w[i], v)
        if v.startswith("-"):
            assert np.signbit(w[i]), i
    check_dequant_bitwise(blob, SB)


def test_mx_dequant_every_code_and_scale():
    # every code under every scale byte 2..254 (products from normal fp32 up
    # to overflow), and the workload's random superblocks
    blobs = [pack_mx_sb([s] * 8, list(range(16)) * 16) for s in range(2, 255)]
    check_dequant_bitwise(np.concatenate(blobs), SB)
    check_dequant_bitwise(mi.mxfp4_blob(mi._rng(3, 77), 2048), SB)
    nan_sb = pack_mx_sb([255] + [127] * 7, list(range(16)) * 16)
    w = gpu_dequant(nan_sb, SB, 0).numpy()
    assert np.isnan(w[:32]).all() and np.isfinite(w[32:]).all()


@pytest.mark.parametrize("name,T,path,tol,stream", [
    ("tiny_mx", 4, qm.MOE_PATH_GEMV, GEMV_TOL, None),
    ("tiny_mx", 4, qm.MOE_PATH_MFMA, MFMA_TOL, None),
    ("tiny_mx", 131, qm.MOE_PATH_MFMA, MFMA_TOL, 3),
    ("decode_mx", 1, qm.MOE_PATH_AUTO, GEMV_TOL, None),
    ("decode_mx", 1, qm.MOE_PATH_AUTO, GEMV_TOL, 5),
    ("decode_mx", 12, qm.MOE_PATH_GEMV, GEMV_TOL, 2),
    ("decode_mx", 32, qm.MOE_PATH_GEMV, GEMV_TOL, 1),
    ("decode_mx", 67, qm.MOE_PATH_MFMA, MFMA_TOL, 9),
])
def test_mx_layer(name, T, path, tol, stream):
    _, used = check_layer(name, T, path, tol, stream=stream)
    if path != qm.MOE_PATH_AUTO:
        assert used == path


def test_mx_auto_path_switch():
    # MXFP4's automatic rule: GEMV up to 26 rows, the grouped GEMM from 27 rows on
    _, used = check_layer("decode_mx", 26, qm.MOE_PATH_AUTO, GEMV_TOL, stream=6)
    assert used == qm.MOE_PATH_GEMV
    _, used = check_layer("decode_mx", 27, qm.MOE_PATH_AUTO, MFMA_TOL, stream=6)
    assert used == qm.MOE_PATH_MFMA


def test_mx_prefill_4096_all_rows():
    _, used = check_layer("prefill4096_mx", 4096, qm.MOE_PATH_AUTO, MFMA_TOL)
    assert used == qm.MOE_PATH_MFMA


@pytest.mark.parametrize("name,T,path,cuts", [
    ("decode_mx", 1, qm.MOE_PATH_GEMV, (0, 256, 512)),
    ("decode_mx", 1, qm.MOE_PATH_GEMV, (0, 192, 512)),
    ("decode_mx", 32, qm.MOE_PATH_MFMA, (0, 256, 512)),
    ("prefill4096_mx", 512, qm.MOE_PATH_MFMA, (0, 256, 512)),
    ("prefill4096_mx", 512, qm.MOE_PATH_MFMA, (0, 128, 320, 512)),   # down ranges off superblocks
    ("tiny_mx", 4, qm.MOE_PATH_GEMV, (0, 64, 128)),
    ("tiny_mx", 4, qm.MOE_PATH_MFMA, (0, 64, 128)),
])
def test_mx_range_shards(name, T, path, cuts):
    w, layer, dl, ol = dev_layer(name)
    tol = GEMV_TOL if path == qm.MOE_PATH_GEMV else MFMA_TOL
    x = mi.make_tokens(w.shape, w.seed, T, stream=w.x_stream)
    say(f"mx range shards {name} T={T} path={path} cuts={cuts}")
    oi, ow, _, _ = oracle.router(x, layer["router_w"], w.shape.k)
    full = oracle.forward(ol, x, oi, ow)
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        part = torch.full((T, dl.H), float("nan"), device=DEV)
        used = qm.moe_layer_forward_range(dl.desc, gpu(x), T, gpu(oi), gpu(ow), a, b, part,
                                          dl.workspace(T), path=path)
        torch.cuda.synchronize()
        assert used == path
        ref = oracle.forward_range(ol, x, oi, ow, a, b)
        assert rel_err(part.cpu().numpy(), ref) <= tol * rel_scale(ref, full)
        parts.append(part)
    out = torch.empty((T, dl.H), device=DEV)
    qm.moe_reduce_partials(parts, T * dl.H, out)
    torch.cuda.synchronize()
    assert rel_err(out.cpu().numpy(), full) <= tol


def test_mx_two_shards_with_device_routing():
    w, layer, dl, ol = dev_layer("decode_mx")
    T = 4
    x = mi.make_tokens(w.shape, w.seed, T, stream=11)
    say("mx two shards, device routing")
    gi, gw = run_router(dl, x)
    oi, ow, _, logits = oracle.router(x, layer["router_w"], w.shape.k)
    exact, exempt, wrong = topk_check(gi, oi, logits)
    assert len(wrong) == 0
    parts = [run_shard(dl, x, oi, ow, s, 2, qm.MOE_PATH_GEMV)[0] for s in range(2)]
    out = torch.empty((T, dl.H), device=DEV)
    qm.moe_reduce_partials(parts, T * dl.H, out)
    torch.cuda.synchronize()
    assert rel_err(out.cpu().numpy(), oracle.forward(ol, x, oi, ow)) <= GEMV_TOL


def test_mx_bit_identical_reruns():
    w, layer, dl, ol = dev_layer("prefill4096_mx")
    x = mi.make_tokens(w.shape, w.seed, 1024)
    say("mx determinism T=1024")
    from test_gpu_parity import run_forward
    a, _ = run_forward(dl, x, qm.MOE_PATH_MFMA)
    b, _ = run_forward(dl, x, qm.MOE_PATH_MFMA)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.isfinite(a).all()


@pytest.mark.parametrize("scales", [(100, 150), (40, 80), (116, 132)])
@pytest.mark.parametrize("path,tol", [(qm.MOE_PATH_GEMV, GEMV_TOL), (qm.MOE_PATH_MFMA, MFMA_TOL)])
def test_mx_wide_scale_bytes(scales, path, tol):
    """E8M0 scale bytes far outside 114..128, the range in which the E2M1
    weights would survive an fp16 weight stage exactly: (100, 150) reaches
    weights of 6 * 2^23 (beyond fp16's 65504), (40, 80) weights of 2^-88
    (below fp16's subnormals).  The fp32 GEMV decodes them exactly and the
    block-scaled matrix cores apply them exactly; both paths against the
    oracle at their tolerances (the ranges keep every intermediate inside
    fp32's normal range)."""
    shp = mi.LayerShape(H=512, E=8, k=2, I=256, Is=256, fmt=1, mx_scales=scales)
    layer = mi.make_layer(shp, seed=61)
    assert layer["gate"][:, :8].min() == scales[0] or layer["down"][:, :8].min() == scales[0]
    x = mi.make_tokens(shp, 61, 70)
    dl = DeviceLayer.from_shape(layer, shp)
    ol = oracle.Layer.from_shape(layer, shp)
    say(f"mx wide scales {scales} path={path}")
    T = x.shape[0]
    out = torch.full((T, shp.H), float("nan"), device=DEV)
    used = qm.moe_layer_forward(dl.desc, gpu(x), T, out, dl.workspace(T), path=path)
    torch.cuda.synchronize()
    assert used == path
    got = out.cpu().numpy()
    ref = oracle.forward(ol, x)
    assert np.isfinite(ref).all() and np.isfinite(got).all()
    oi, _, _, logits = oracle.router(x, layer["router_w"], shp.k)
    gi, _ = run_router(dl, x)
    exact, _, wrong = topk_check(gi, oi, logits)
    assert len(wrong) == 0
    err = rel_err(got[exact], ref[exact])
    say(f"  max|err|/RMS = {err:.3e}")
    assert err <= tol


@pytest.mark.parametrize("path,tol", [(qm.MOE_PATH_GEMV, GEMV_TOL), (qm.MOE_PATH_MFMA, MFMA_TOL)])
def test_mx_nan_scale_propagates(path, tol):
    """E8M0 byte 255 is the format's NaN.  Give it to the first 32-weight
    block of expert 0's down row 5: every token routed to expert 0 gets a NaN
    in output feature 5 in the oracle.  The fp32 GEMV path must reproduce that
    NaN pattern exactly.  The MFMA path carries the per-slot rows as 16-bit
    block floating point, in which a block of 8 values holding a NaN reads
    back as 8 NaNs: its NaNs must cover the oracle's and lie in the same rows
    and 8-column groups.  Every other value matches at the path's tolerance."""
    shp = mi.LayerShape(H=512, E=8, k=2, I=256, Is=256, fmt=1)
    layer = mi.make_layer(shp, seed=62)
    per_row = shp.I // 256                      # 144-byte superblocks per down row
    down = layer["down"].copy()                 # [E][rows * per_row * 144] bytes
    down[0, 5 * per_row * 144] = 255            # expert 0, row 5, scale of block 0
    layer = dict(layer, down=down)
    x = mi.make_tokens(shp, 62, 70)
    dl = DeviceLayer.from_shape(layer, shp)
    ol = oracle.Layer.from_shape(layer, shp)
    say(f"mx NaN scale path={path}")
    T = x.shape[0]
    out = torch.zeros((T, shp.H), device=DEV)
    used = qm.moe_layer_forward(dl.desc, gpu(x), T, out, dl.workspace(T), path=path)
    torch.cuda.synchronize()
    assert used == path
    got = out.cpu().numpy()
    ref = oracle.forward(ol, x)
    oi, _, _, logits = oracle.router(x, layer["router_w"], shp.k)
    gi, _ = run_router(dl, x)
    exact, _, wrong = topk_check(gi, oi, logits)
    assert len(wrong) == 0
    nan_ref, nan_got = np.isnan(ref), np.isnan(got)
    routed0 = (oi == 0).any(axis=1)
    assert routed0.any() and (~routed0).any()
    assert np.array_equal(nan_ref[:, 5], routed0) and nan_ref.sum() == routed0.sum()
    if path == qm.MOE_PATH_GEMV:
        assert np.array_equal(nan_got, nan_ref)
    else:
        assert (nan_got | ~nan_ref).all()                       # covers the oracle's NaNs
        groups = np.repeat(nan_ref.reshape(T, -1, 8).any(axis=2), 8, axis=1)
        assert (~nan_got | groups).all()                        # within their 8-column groups
    fin = ~nan_ref & ~nan_got
    assert np.isfinite(got[fin]).all()
    err = float(np.abs(got[fin] - ref[fin]).max() / np.sqrt(np.mean(ref[fin] ** 2)))
    say(f"  NaNs oracle {int(nan_ref.sum())}, GPU {int(nan_got.sum())}; finite max|err|/RMS = {err:.3e}")
    assert err <= tol
