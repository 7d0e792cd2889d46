"""Comparison helpers shared by the GPU parity tests and the smoke check."""
import functools

import numpy as np

# Tolerances, max|gpu - ref| / RMS(ref) over every compared output of a call:
GEMV_TOL = 1e-4      # fp32 dequant-GEMV path
MFMA_TOL = 1e-2      # fp16-operand MFMA path (fp32 accumulation)
TOPK_GAP = 1e-5      # top-k may differ only between experts whose logits are closer than this


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.abs(got - ref).max() / rms) if ref.size else 0.0


def fp16_operand_reference(layer, shp, x, idx, w, sw=1.0):
    """The K-quant layer with the MFMA path's operand roundings and nothing
    else: tokens, the oracle's exact weights and h = silu(g) u * 2^-4 each
    rounded to the nearest fp16 once, every product and sum in float64.
    Separates what the fp16 operands cost from any defect of the kernels.
    Only the experts that idx selects are decoded."""
    import oracle
    H, k, I, Is = shp.H, shp.k, shp.I, shp.Is
    g_sb = I * H // 256 * 144     # bytes of one expert's gate (or up) matrix
    d_sb = H * I // 256 * 176     # of its down matrix

    def f16(a):
        return np.asarray(a).astype(np.float16).astype(np.float64)

    def deq(blob, bits, rows, cols):
        return f16(oracle.dequant(np.asarray(blob).reshape(-1), bits).reshape(rows, cols))

    cache = {}

    def expert(e):
        if e not in cache:
            gb = np.asarray(layer["gate"]).reshape(-1)[e * g_sb:(e + 1) * g_sb]
            ub = np.asarray(layer["up"]).reshape(-1)[e * g_sb:(e + 1) * g_sb]
            db = np.asarray(layer["down"]).reshape(-1)[e * d_sb:(e + 1) * d_sb]
            cache[e] = (deq(gb, 4, I, H), deq(ub, 4, I, H), deq(db, 5, H, I))
        return cache[e]

    def ffn(g_w, u_w, d_w, xv):
        g = g_w @ xv
        u = u_w @ xv
        h = f16(g / (1.0 + np.exp(-g)) * u * 2.0 ** -4)
        return (d_w @ h) * 2.0 ** 4

    sh = None
    if Is:
        sh = (deq(layer["sh_gate"], 4, Is, H), deq(layer["sh_up"], 4, Is, H),
              deq(layer["sh_down"], 5, H, Is))
    xs = f16(x)
    out = np.zeros((x.shape[0], H))
    for t in range(x.shape[0]):
        for j in range(k):
            out[t] += float(w[t, j]) * ffn(*expert(int(idx[t, j])), xs[t])
        if sh is not None:
            out[t] += sw * ffn(*sh, xs[t])
    return out


def topk_check(gpu_idx, ora_idx, ora_logits, gap=TOPK_GAP):
    """Classify rows: exact match, exempt (every differing slot is a swap
    between experts whose oracle logits differ by < gap), or wrong.
    Returns (exact_rows, exempt_rows, wrong_rows) as index arrays."""
    gpu_idx = np.asarray(gpu_idx)
    ora_idx = np.asarray(ora_idx)
    exact, exempt, wrong = [], [], []
    for t in range(gpu_idx.shape[0]):
        g, o = gpu_idx[t], ora_idx[t]
        if np.array_equal(g, o):
            exact.append(t)
            continue
        ok = len(set(g.tolist())) == len(g) and all(0 <= e < ora_logits.shape[1] for e in g)
        for j in range(len(g)):
            if g[j] != o[j] and abs(ora_logits[t, g[j]] - ora_logits[t, o[j]]) >= gap:
                ok = False
        (exempt if ok else wrong).append(t)
    return np.array(exact, int), np.array(exempt, int), np.array(wrong, int)


@functools.lru_cache(maxsize=4)
def workload(name):
    """Host arrays of a named workload (cached per process)."""
    import moe_inputs as mi
    w = mi.WORKLOADS[name]
    layer = mi.make_layer(w.shape, w.seed, zipf=w.zipf)
    return w, layer
