"""HIP-graph replay of the layer against its eager result.

The bench times steps replayed from HIP graphs, so every path is captured
here and replayed several times.  Between replays the same workspace is
used by eager calls on other token rows, with synchronisations in between,
so that a kernel that relied on workspace state left by an earlier call
(counters, histograms, tile lists) would show as a changed replay.  The
kernels are deterministic, so every replay must equal the eager output bit
for bit.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

import moe_inputs as mi  # noqa: E402
from parity_util import workload  # noqa: E402

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import quantized_moe_transformer_amd as qm  # noqa: E402
from quantized_moe_transformer_amd.layer import DeviceLayer  # noqa: E402

REPLAYS = 3


def say(msg):
    print(f"[graph] {msg}", flush=True)


def tokens(w, seed):
    return torch.from_numpy(np.ascontiguousarray(
        mi.make_tokens(w.shape, seed, w.T, stream=w.x_stream, zipf=w.zipf))).cuda()


def replay_check(step, out, other):
    """Eager result of step(), then REPLAYS replays of its graph, each after
    other() has reused the workspace; every replay must equal the eager one."""
    step()
    torch.cuda.synchronize()
    want = out.clone()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for r in range(REPLAYS):
        out.fill_(float("nan"))
        other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {r} differs from the eager result"
    del g


@pytest.mark.parametrize("name,path", [
    ("decode", qm.MOE_PATH_AUTO),            # GEMV, router in the front kernel
    ("decode_batched", qm.MOE_PATH_MFMA),    # 32 rows: few-row router, grouped GEMM
    ("prefill512_zipf", qm.MOE_PATH_AUTO),   # matrix-core router, bucketing in one kernel
    ("prefill4096", qm.MOE_PATH_AUTO),       # top-k makes the bucketing's counts
    ("decode_mx", qm.MOE_PATH_AUTO),
    ("prefill4096_mx", qm.MOE_PATH_AUTO),    # block-scaled matrix cores
])
def test_forward_graph_replays(name, path):
    w, layer = workload(name)
    shp = w.shape
    T = w.T
    say(f"{name} T={T} path={path}")
    dl = DeviceLayer.from_shape(layer, shp)
    x = tokens(w, w.seed)
    x2 = tokens(w, w.seed + 1000)
    out = torch.empty((T, shp.H), device="cuda")
    out2 = torch.empty((T, shp.H), device="cuda")
    ws = dl.workspace(T)

    def step():
        qm.moe_layer_forward(dl.desc, x, T, out, ws, path=path)

    def other():
        qm.moe_layer_forward(dl.desc, x2, T, out2, ws, path=path)

    replay_check(step, out, other)


@pytest.mark.parametrize("name", ["decode_sharded", "prefill4096"])
def test_shard_graph_replays(name):
    """router_topk once, the two 256/256 shards and the reduce, as one graph."""
    w, layer = workload(name)
    shp = w.shape
    T = w.T
    say(f"{name} two shards T={T}")
    dl = DeviceLayer.from_shape(layer, shp)
    x = tokens(w, w.seed)
    x2 = tokens(w, w.seed + 1000)
    idx = torch.empty((T, shp.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, shp.k), dtype=torch.float32, device="cuda")
    parts = [torch.empty((T, shp.H), device="cuda") for _ in range(2)]
    out = torch.empty((T, shp.H), device="cuda")
    out2 = torch.empty((T, shp.H), device="cuda")
    ws_r = dl.workspace(T)
    ws = [dl.workspace(T, 2) for _ in range(2)]

    def run(xv, o):
        qm.router_topk(dl.desc, xv, T, idx, wts, ws_r)
        for s in range(2):
            qm.moe_layer_forward_shard(dl.desc, xv, T, idx, wts, s, 2, parts[s], ws[s])
        qm.moe_reduce_partials(parts, T * shp.H, o)

    replay_check(lambda: run(x, out), out, lambda: run(x2, out2))


@pytest.mark.parametrize("name", ["decode", "prefill512_zipf"])
def test_noalloc_graph_replays(name):
    """The entry point that allocates nothing, for callers under graph
    capture: its fixed scratch is shared by the replays and the eager calls."""
    w, layer = workload(name)
    shp = w.shape
    T = w.T
    say(f"{name} no-alloc T={T}")
    dl = DeviceLayer.from_shape(layer, shp)
    x = tokens(w, w.seed)
    x2 = tokens(w, w.seed + 1000)
    out = torch.empty((T, shp.H), device="cuda")
    out2 = torch.empty((T, shp.H), device="cuda")
    replay_check(lambda: qm.moe_layer_forward_noalloc(dl.desc, x, T, out), out,
                 lambda: qm.moe_layer_forward_noalloc(dl.desc, x2, T, out2))
