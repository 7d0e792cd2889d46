"""moe_layer_forward_noalloc (the library's fixed per-device scratch in place of
a caller workspace) against moe_layer_forward on the same inputs.

Both run the same kernels in the same order, and the layer is deterministic,
so their outputs must be bit-identical; each is also checked against the CPU
oracle to its path's tolerance.  Two calls in a row, the second with fewer
rows (the scratch keeps the first call's contents), then an oversized call
that must be refused with nothing written.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import moe_inputs as mi  # noqa: E402
import oracle  # noqa: E402
from parity_util import GEMV_TOL, MFMA_TOL, rel_err, workload  # noqa: E402

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import quantized_moe_transformer_amd as qm  # noqa: E402
from quantized_moe_transformer_amd import _lib  # noqa: E402
from quantized_moe_transformer_amd.layer import DeviceLayer  # noqa: E402


def say(msg):
    print(f"[noalloc] {msg}", flush=True)


def both(dl, x):
    T = x.shape[0]
    xd = torch.from_numpy(x).cuda()
    ref = torch.full((T, dl.H), float("nan"), device="cuda")
    got = torch.full((T, dl.H), float("nan"), device="cuda")
    p_ref = qm.moe_layer_forward(dl.desc, xd, T, ref, dl.workspace(T))
    p_got = qm.moe_layer_forward_noalloc(dl.desc, xd, T, got)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy(), p_ref, p_got


@pytest.mark.parametrize("name,T1,T2", [("decode", 64, 1), ("prefill4096", 600, 20),
                                        ("tiny_mx", 131, 4)])
def test_noalloc_matches_workspace_call(name, T1, T2):
    w, layer = workload(name)
    dl = DeviceLayer.from_shape(layer, w.shape)
    ol = oracle.Layer.from_shape(layer, w.shape)
    for T, stream in ((T1, 3), (T2, 4)):
        x = mi.make_tokens(w.shape, w.seed, T, stream=stream, zipf=w.zipf)
        say(f"{name} T={T}")
        ref, got, p_ref, p_got = both(dl, x)
        assert p_got == p_ref
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
        tol = GEMV_TOL if p_got == qm.MOE_PATH_GEMV else MFMA_TOL
        oi, ow, _, _ = oracle.router(x, layer["router_w"], w.shape.k)
        gi = torch.empty((T, w.shape.k), dtype=torch.int32, device="cuda")
        gw = torch.empty((T, w.shape.k), dtype=torch.float32, device="cuda")
        qm.router_topk(dl.desc, torch.from_numpy(x).cuda(), T, gi, gw, dl.workspace(T))
        torch.cuda.synchronize()
        same = np.all(gi.cpu().numpy() == oi, axis=1)   # rows routed as the oracle routes them
        assert same.sum() >= T - 2
        assert rel_err(got[same], oracle.forward(ol, x)[same]) <= tol


def test_noalloc_refuses_oversized_input():
    w, layer = workload("decode")
    dl = DeviceLayer.from_shape(layer, w.shape)
    T = 4096
    assert qm.moe_workspace_bytes(dl.desc, T) > _lib.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, dl.H), device="cuda")
    out = torch.full((T, dl.H), 7.0, device="cuda")
    with pytest.raises(qm.MoeError) as e:
        qm.moe_layer_forward_noalloc(dl.desc, x, T, out)
    assert e.value.status == _lib.MOE_ETOOBIG
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
