"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes its expected value: a hand-worked fixture, a closed
form, an identity of the mathematics, a special case that reduces to a
textbook computation, or brute force on tiny inputs.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from kquant_pack import pack_mx_sb, pack_sb, read_fixture

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kquant_handworked.txt")
FX = read_fixture(GOLDEN)
SC = [1, 2, 3, 4, 33, 47, 62, 63]
M = [0, 5, 10, 63, 17, 32, 48, 1]

ONE_F16 = 0x3C00     # 1.0
ZERO_F16 = 0x0000


# --------------------------------------------------------------------------
# fp16 field decoding
# --------------------------------------------------------------------------

def test_half_decode_all_patterns():
    """Every finite fp16 bit pattern decodes to numpy's float16 value (library routine)."""
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.all(np.isinf(got[np.isinf(ref)]))
    assert np.all(np.isnan(got[np.isnan(ref)]))


# --------------------------------------------------------------------------
# superblock decoding: hand-worked fixture
# --------------------------------------------------------------------------

def _q4_codes():
    return [(i % 16) if (i // 32) % 2 == 0 else 15 - (i % 16) for i in range(256)]


def _q5_codes():
    return [(7 * i) % 32 for i in range(256)]


def test_packer_matches_fixture():
    """The test-side packer reproduces the hand-derived bytes of the fixture."""
    head = bytes([0x00, 0x1C, 0x00, 0x18]) + FX["scales"]
    sb4 = pack_sb(FX["d_bits"], FX["dmin_bits"], SC, M, _q4_codes(), 4)
    assert sb4.tobytes() == head + FX["q4_qs"]
    sb5 = pack_sb(FX["d_bits"], FX["dmin_bits"], SC, M, _q5_codes(), 5)
    assert sb5.tobytes() == head + FX["q5_qh"] + FX["q5_qs"]


def test_handworked_q4k():
    blob = np.frombuffer(bytes([0x00, 0x1C, 0x00, 0x18]) + FX["scales"] + FX["q4_qs"], np.uint8)
    w = oracle.dequant(blob, 4)
    for i, n in FX["q4_w512"].items():
        assert w[i] == np.float32(n / 512), (i, w[i], n)
    # every element: 512*w = 2*sc_j*q_i - m_j for this hand-chosen block
    q = _q4_codes()
    expect = np.array([(2 * SC[i // 32] * q[i] - M[i // 32]) / 512 for i in range(256)], np.float32)
    assert np.array_equal(w, expect)


def test_handworked_q5k():
    blob = np.frombuffer(bytes([0x00, 0x1C, 0x00, 0x18]) + FX["scales"] + FX["q5_qh"] + FX["q5_qs"],
                         np.uint8)
    w = oracle.dequant(blob, 5)
    for i, n in FX["q5_w512"].items():
        assert w[i] == np.float32(n / 512), (i, w[i], n)
    q = _q5_codes()
    expect = np.array([(2 * SC[i // 32] * q[i] - M[i // 32]) / 512 for i in range(256)], np.float32)
    assert np.array_equal(w, expect)


# --------------------------------------------------------------------------
# superblock decoding: exhaustive closed form
# --------------------------------------------------------------------------

def _f16_bits(v):
    return int(np.array([v], np.float16).view(np.uint16)[0])


@pytest.mark.parametrize("bits", [4, 5])
@pytest.mark.parametrize("dpair", [(1e-3, 4e-3), (3.1e-3, 1.7e-3), (2.0 ** -20, 65504.0),
                                   (0.7, 2.0 ** -24)])
def test_closed_form_every_field(bits, dpair):
    """Every (scale, min, code) combination decodes to RNE_fp32(d*sc*q - dmin*m),
    the exact value computed here with rational arithmetic."""
    d_bits, dm_bits = _f16_bits(dpair[0]), _f16_bits(dpair[1])
    d = Fraction(float(np.uint16(d_bits).view(np.float16)))
    dm = Fraction(float(np.uint16(dm_bits).view(np.float16)))
    nq = 16 if bits == 4 else 32
    pairs = [(s, m) for s in range(64) for m in range(64)]
    blobs, expect = [], []
    rng = np.random.default_rng(7)
    for b in range(0, len(pairs), 8):
        grp = pairs[b:b + 8]
        sc = [p[0] for p in grp]
        mm = [p[1] for p in grp]
        # each sub-block walks every code (twice for 4-bit), in a shuffled order
        q = []
        for j in range(8):
            codes = np.tile(np.arange(nq), 32 // nq)
            rng.shuffle(codes)
            q.extend(int(c) for c in codes)
        blobs.append(pack_sb(d_bits, dm_bits, sc, mm, q, bits))
        for i in range(256):
            exact = d * sc[i // 32] * q[i] - dm * mm[i // 32]
            expect.append(np.float32(float(exact)))  # exact fits a double; one RNE to fp32
    w = oracle.dequant(np.concatenate(blobs), bits)
    assert np.array_equal(w, np.array(expect, np.float32))


def test_zero_codes_and_mins_give_zero():
    sb = pack_sb(_f16_bits(3e-3), _f16_bits(2e-3), [63] * 8, [0] * 8, [0] * 256, 5)
    assert np.all(oracle.dequant(sb, 5) == 0)


def test_rejects_partial_superblock():
    with pytest.raises(ValueError):
        oracle.dequant(np.zeros(143, np.uint8), 4)


def test_flat_layout_spans_rows():
    """A 128-wide matrix: superblock b holds rows 2b and 2b+1 (flat row-major)."""
    rows, K = 4, 128
    blobs = []
    for b in range(rows * K // 256):
        # codes encode the element position within the superblock's first row / second row
        q = [(b + 1) if i < 128 else (b + 9) for i in range(256)]
        blobs.append(pack_sb(ONE_F16, ZERO_F16, [1] * 8, [0] * 8, q, 5))
    W = oracle.dequant(np.concatenate(blobs), 5).reshape(rows, K)
    for r in range(rows):
        assert np.all(W[r] == (r // 2 + 1 if r % 2 == 0 else r // 2 + 9))


# --------------------------------------------------------------------------
# router
# --------------------------------------------------------------------------

def _dyadic(rng, shape, scale_bits=6, lim=8):
    """Small dyadic values: every sum of products below is exact in double."""
    return (rng.integers(-lim, lim + 1, size=shape) / 2.0 ** scale_bits).astype(np.float32)


@pytest.mark.parametrize("seed", range(20))
def test_router_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    T, H, E, k = 6, 16, 8, 2
    x = _dyadic(rng, (T, H))
    wr = _dyadic(rng, (H, E))
    wr[:, 5] = wr[:, 2]           # experts 2 and 5 always tie exactly
    idx, w, wd, logits = oracle.router(x, wr, k)
    for t in range(T):
        exact = [sum(Fraction(float(x[t, h])) * Fraction(float(wr[h, e])) for h in range(H))
                 for e in range(E)]
        assert [float(v) for v in exact] == list(logits[t])
        order = sorted(range(E), key=lambda e: (-exact[e], e))   # brute-force sort
        assert list(idx[t]) == order[:k]
        assert abs(sum(wd[t]) - 1.0) < 1e-15
        # ratio of two selected weights = exp(logit difference)
        r = wd[t, 0] / wd[t, 1]
        assert math.isclose(r, math.exp(float(exact[order[0]] - exact[order[1]])), rel_tol=1e-14)


def test_router_equal_logits_split_evenly():
    H, E, k = 4, 8, 4
    x = np.zeros((1, H), np.float32)
    x[0, 0] = 1.0
    wr = np.zeros((H, E), np.float32)
    wr[0] = [0.5, 0.25, 0.5, 0.5, -1.0, 0.5, 0.0, 0.25]
    idx, w, wd, _ = oracle.router(x, wr, k)
    assert list(idx[0]) == [0, 2, 3, 5]          # four-way tie, lower indices first
    assert np.all(w[0] == np.float32(0.25))


def test_router_weights_ignore_unselected_logits():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 64)).astype(np.float32)
    wr = (0.1 * rng.standard_normal((64, 16))).astype(np.float32)
    idx, _, wd, logits = oracle.router(x, wr, 4)
    worst = [e for e in np.argsort(logits[0])[:3]]
    wr2 = wr.copy()
    wr2[:, worst] -= 0.5 * np.sign(x[0])[:, None]     # push unselected logits further down
    idx2, _, wd2, _ = oracle.router(x, wr2, 4)
    assert np.array_equal(idx, idx2)
    assert np.allclose(wd, wd2, rtol=1e-14, atol=0)


def test_router_orders_exact_logits():
    # logits 1 and 1 + 2^-30 are equal once rounded to fp32; the exact order
    # puts expert 1 first (an oracle that ranked fp32-rounded logits would keep
    # the lower index, expert 0, first)
    x = np.array([[1.0, 2.0 ** -30]], np.float32)
    wr = np.array([[1.0, 1.0], [0.0, 1.0]], np.float32)
    idx, _, wd, logits = oracle.router(x, wr, 2)
    assert np.float32(logits[0, 0]) == np.float32(logits[0, 1])
    assert logits[0, 1] - logits[0, 0] == 2.0 ** -30
    assert list(idx[0]) == [1, 0]
    assert math.isclose(wd[0, 0] / wd[0, 1], math.exp(2.0 ** -30), rel_tol=1e-15)


def test_router_k_equals_e_is_full_softmax():
    x = np.array([[1.0]], np.float32)
    wr = np.array([[0.0, 1.0, 2.0]], np.float32)
    idx, _, wd, _ = oracle.router(x, wr, 3)
    assert list(idx[0]) == [2, 1, 0]
    z = 1 + math.e + math.e ** 2
    assert np.allclose(wd[0], [math.e ** 2 / z, math.e / z, 1 / z], rtol=1e-15)


# --------------------------------------------------------------------------
# bucketing
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(5))
def test_bucket_is_stable_sort(seed):
    rng = np.random.default_rng(seed)
    T, k, E = 37, 3, 7
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    counts, offsets, perm, inv = oracle.bucket(idx, E)
    flat = idx.ravel()
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert list(perm) == sorted(range(T * k), key=lambda s: (flat[s], s))
    assert np.array_equal(perm[inv], np.arange(T * k))


# --------------------------------------------------------------------------
# expert FFN and combine: closed forms
# --------------------------------------------------------------------------

def _const_matrix(rows, K, bits, d_bits=ONE_F16, q=1):
    """A [rows][K] matrix whose every weight is d*q (sc=1, m=0)."""
    n_sb = rows * K // 256
    sb = pack_sb(d_bits, ZERO_F16, [1] * 8, [0] * 8, [q] * 256, bits)
    return np.tile(sb, n_sb)


def _const_layer(H, E, k, I, Is, down_codes, sh_code=1):
    layer = {
        "router_w": np.zeros((H, E), np.float32),
        "gate": np.stack([_const_matrix(I, H, 4)] * E),
        "up": np.stack([_const_matrix(I, H, 4)] * E),
        "down": np.stack([_const_matrix(H, I, 5, q=c) for c in down_codes]),
    }
    if Is:
        layer["sh_gate"] = _const_matrix(Is, H, 4)
        layer["sh_up"] = _const_matrix(Is, H, 4)
        layer["sh_down"] = _const_matrix(H, Is, 5, q=sh_code)
    return layer


def test_silu_identity_and_value_at_ln3():
    """One expert, all weights 1, x = (a, 0, ...): g = u = a, out_o = I*silu(a)*a.
    silu(a) - silu(-a) = a for any a (sigmoid(z)+sigmoid(-z) = 1), and
    sigmoid(ln 3) = 3/4."""
    H, I = 256, 256
    L = oracle.Layer(_const_layer(H, 1, 1, I, 0, [1]), H, 1, 1, I, 0)
    for a in [np.float32(math.log(3.0)), np.float32(2.5), np.float32(20.0)]:
        xp = np.zeros((1, H), np.float32); xp[0, 0] = a
        xm = -xp
        _, op = oracle.forward(L, xp, want_double=True)
        _, om = oracle.forward(L, xm, want_double=True)
        # op = I*a*silu(a), om = I*(-a)*silu(-a)  ->  op + om = I*a*(silu(a)-silu(-a)) = I*a^2
        assert np.allclose(op + om, I * float(a) ** 2, rtol=1e-13)
        assert np.all(op[0] == op[0, 0])
    a = float(np.float32(math.log(3.0)))
    xp = np.zeros((1, H), np.float32); xp[0, 0] = a
    _, op = oracle.forward(L, xp, want_double=True)
    assert math.isclose(op[0, 0], I * 0.75 * a * a, rel_tol=1e-6)   # a = ln 3 to fp32
    # silu(1) = 1/(1+e^-1)
    x1 = np.zeros((1, H), np.float32); x1[0, 0] = 1.0
    _, o1 = oracle.forward(L, x1, want_double=True)
    assert math.isclose(o1[0, 0], I * 0.7310585786300049, rel_tol=1e-14)


def test_two_expert_mixture_and_shared():
    """E=4, k=2; expert e's down weights all equal c_e, the shared one c_s.
    With x = e_0, g = u = 1 everywhere, so out_o = I*silu(1)*(w_a c_a + w_b c_b + c_s)."""
    H, E, k, I, Is = 256, 4, 2, 256, 256
    codes = [1, 2, 3, 4]
    arrays = _const_layer(H, E, k, I, Is, codes, sh_code=5)
    arrays["router_w"][0] = [0.25, 1.0, 1.0, -2.0]      # experts 1 and 2 tie -> 1/2 each
    L = oracle.Layer(arrays, H, E, k, I, Is)
    x = np.zeros((1, H), np.float32); x[0, 0] = 1.0
    _, o = oracle.forward(L, x, want_double=True)
    s1 = 0.7310585786300049
    assert np.allclose(o, I * s1 * (0.5 * 2 + 0.5 * 3 + 5), rtol=1e-14)
    # unequal logits: w ratio = e^(l_a - l_b); with l = (ln3, 0) the weights are 3/4, 1/4
    arrays["router_w"][0] = [np.float32(math.log(3.0)), 0.0, -1.0, -2.0]
    L = oracle.Layer(arrays, H, E, k, I, Is)
    _, o = oracle.forward(L, x, want_double=True)
    assert np.allclose(o, I * s1 * (0.75 * 1 + 0.25 * 2 + 5), rtol=1e-6)
    # shared expert with weight 0 and no shared expert both drop the shared term
    L0 = oracle.Layer(arrays, H, E, k, I, Is, shared_weight=0.0)
    _, o0 = oracle.forward(L0, x, want_double=True)
    assert np.allclose(o0, I * s1 * (0.75 * 1 + 0.25 * 2), rtol=1e-6)


def test_given_routing_is_used_verbatim():
    H, E, k, I, Is = 256, 4, 2, 256, 0
    arrays = _const_layer(H, E, k, I, Is, [1, 2, 3, 4])
    L = oracle.Layer(arrays, H, E, k, I, Is)
    x = np.zeros((1, H), np.float32); x[0, 0] = 1.0
    idx = np.array([[3, 0]], np.int32)
    w = np.array([[0.25, 0.75]], np.float32)
    _, o = oracle.forward(L, x, idx, w, want_double=True)
    assert np.allclose(o, I * 0.7310585786300049 * (0.25 * 4 + 0.75 * 1), rtol=1e-14)


def test_dense_ffn_special_case():
    """E=1, k=1, no shared expert: the layer is a dense SwiGLU FFN
    y = Wd (silu(Wg x) * (Wu x)) on the decoded weights (rows = output features)."""
    import moe_inputs as mi
    shp = mi.LayerShape(H=256, E=1, k=1, I=128, Is=0)
    arrays = mi.make_layer(shp, seed=11)
    L = oracle.Layer.from_shape(arrays, shp)
    x = mi.make_tokens(shp, 11, 3)
    o = oracle.forward(L, x)
    Wg = oracle.dequant(arrays["gate"][0], 4).reshape(128, 256).astype(np.float64)
    Wu = oracle.dequant(arrays["up"][0], 4).reshape(128, 256).astype(np.float64)
    Wd = oracle.dequant(arrays["down"][0], 5).reshape(256, 128).astype(np.float64)
    g = x.astype(np.float64) @ Wg.T
    u = x.astype(np.float64) @ Wu.T
    ref = ((g / (1 + np.exp(-g))) * u) @ Wd.T
    assert np.allclose(o, ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())


def test_zero_weights_give_zero_output():
    H, I = 256, 128
    zero4 = np.tile(pack_sb(ONE_F16, ONE_F16, [5] * 8, [0] * 8, [0] * 256, 4), I * H // 256)
    zero5 = np.tile(pack_sb(ONE_F16, ONE_F16, [5] * 8, [0] * 8, [0] * 256, 5), I * H // 256)
    arrays = {"router_w": np.ones((H, 2), np.float32), "gate": np.stack([zero4] * 2),
              "up": np.stack([zero4] * 2), "down": np.stack([zero5] * 2),
              "sh_gate": zero4, "sh_up": zero4, "sh_down": zero5}
    L = oracle.Layer(arrays, H, 2, 1, I, I)
    x = np.random.default_rng(0).standard_normal((3, H)).astype(np.float32)
    assert np.all(oracle.forward(L, x) == 0)


# --------------------------------------------------------------------------
# shard algebra: the partials add to the unsplit layer
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n", [2, 4])
def test_shard_partials_sum_to_whole(n):
    import moe_inputs as mi
    layer, x = mi.workload_inputs("tiny")
    L = oracle.Layer.from_shape(layer, mi.TINY)
    idx, w, _, _ = oracle.router(x, layer["router_w"], mi.TINY.k)
    _, full = oracle.forward(L, x, idx, w, want_double=True)
    parts = [oracle.forward(L, x, idx, w, s, n, want_double=True)[1] for s in range(n)]
    rms = np.sqrt(np.mean(full ** 2))
    assert np.abs(sum(parts) - full).max() <= 1e-12 * rms
    # unforced routing equals forcing the oracle's own decision (w rounded to fp32 aside)
    own = oracle.forward(L, x)
    assert np.abs(own - full).max() <= 1e-6 * rms


def test_reduce_partials_ascending_order():
    a = np.array([1.0, 1e8], np.float32)
    b = np.array([2.0 ** -30, -1e8], np.float32)
    out = oracle.reduce_partials([a, b])
    assert out[0] == np.float32(1.0) and out[1] == 0.0


def test_empty_batch():
    import moe_inputs as mi
    layer, _ = mi.workload_inputs("tiny")
    L = oracle.Layer.from_shape(layer, mi.TINY)
    out = oracle.forward(L, np.zeros((0, 256), np.float32))
    assert out.shape == (0, 256)


# --------------------------------------------------------------------------
# RMSNorm before the layer and the residual after it (page "Distributed CPU:
# Zip Fusion Beyond Tensor Parallelism", "What Must Cross the Fabric: The
# Reduction Algebra"; page "CKE Zip: From Splitting Tokens To Splitting
# Qwen3.5 Weights", "What PR #382 Now Splits").  Pinned by closed forms.
# --------------------------------------------------------------------------

def test_rmsnorm_constant_row_is_sign_times_weight():
    # every column equal to c, eps = 0: mean(x^2) = c^2, so y = g * c / |c|
    # (a sum in place of the mean would give g / sqrt(H) instead)
    H = 64
    g = np.linspace(-2.0, 3.0, H).astype(np.float32)
    x = np.stack([np.full(H, 3.0), np.full(H, -0.25)]).astype(np.float32)
    y = oracle.rmsnorm(x, g, 0.0)
    assert np.array_equal(y[0], g)
    assert np.array_equal(y[1], -g)


def test_rmsnorm_one_hot_row():
    # x = a e_i, eps = 0: mean(x^2) = a^2 / H, so y_i = g_i sqrt(H) sign(a), all
    # other columns 0
    H = 256
    g = np.full(H, 0.5, np.float32)
    x = np.zeros((1, H), np.float32)
    x[0, 37] = -7.0
    y = oracle.rmsnorm(x, g, 0.0)
    assert y[0, 37] == np.float32(-0.5 * 16.0)
    assert np.count_nonzero(y) == 1


def test_rmsnorm_three_four_five():
    # H = 2, x = (3, 4): mean(x^2) = 25/2, y = x * sqrt(2) / 5 = (0.6, 0.8) * sqrt(2)
    y = oracle.rmsnorm(np.array([[3.0, 4.0]], np.float32), np.ones(2, np.float32), 0.0)
    assert np.array_equal(y[0], np.array([0.6 * math.sqrt(2.0), 0.8 * math.sqrt(2.0)], np.float32))


def test_rmsnorm_eps_scale_and_sign():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 96)).astype(np.float32)
    g = rng.standard_normal(96).astype(np.float32)
    # eps = 0: invariant under positive scaling by a power of two, odd in x
    y = oracle.rmsnorm(x, g, 0.0)
    assert np.array_equal(oracle.rmsnorm(x * np.float32(8.0), g, 0.0), y)
    assert np.array_equal(oracle.rmsnorm(-x, g, 0.0), -y)
    # eps enters under the root: for a row scaled to mean(x^2) = 1, y = g x / sqrt(1 + eps)
    z = x / np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=1, keepdims=True))
    z = z.astype(np.float32)
    ms = np.mean(z.astype(np.float64) ** 2, axis=1, keepdims=True)
    want = (g.astype(np.float64) * z / np.sqrt(ms + 0.25)).astype(np.float32)
    assert np.abs(oracle.rmsnorm(z, g, 0.25) - want).max() <= 1e-6
    assert np.abs(ms - 1.0).max() < 1e-6
    # a zero row stays zero (no 0/0) once eps > 0
    assert not np.any(oracle.rmsnorm(np.zeros((1, 96), np.float32), g, 1e-6))


@pytest.mark.parametrize("cuts", [(0, 1024, 2048), (0, 512, 1024, 1536, 2048), (0, 640, 2048)])
def test_rmsnorm_sum_of_squares_splits_into_shard_scalars(cuts):
    # the reduction algebra: the row's sum of squares is the sum of the
    # shards' partial sums (exactly up to double rounding)
    rng = np.random.default_rng(len(cuts))
    x = rng.standard_normal((9, 2048)).astype(np.float32) * 3.0
    full = oracle.sumsq(x)
    parts = [oracle.sumsq(x, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    assert np.abs(sum(parts) - full).max() <= 1e-12 * full.max()
    # and the per-column squares add up to the same (independent check)
    assert np.abs((x.astype(np.float64) ** 2).sum(axis=1) - full).max() <= 1e-12 * full.max()


def test_reduce_residual_order_and_cancellation():
    p0 = np.array([1.0, 1e8, 3.0], np.float32)
    p1 = np.array([2.0 ** -30, -1e8, -3.0], np.float32)
    r = np.array([0.5, 2.0 ** -26, 7.0], np.float32)
    out = oracle.reduce_residual([p0, p1], r)
    # exact sums rounded once: 1.5 (+2^-30 lost), 2^-26, 7
    assert np.array_equal(out, np.array([1.5, 2.0 ** -26, 7.0], np.float32))
    # one partial: the layer output plus the residual
    assert np.array_equal(oracle.reduce_residual([p0], -p0), np.zeros(3, np.float32))


@pytest.mark.parametrize("cuts", [(0, 48, 128), (0, 32, 64, 96, 128), (0, 96, 128), (0, 64, 128), (0, 128)])
def test_uneven_shard_ranges_sum_to_whole(cuts):
    # page "Distributed CPU: Zip Fusion Beyond Tensor Parallelism", "Heterogeneous
    # Topology": shards sized to each lane's throughput, not equal; any
    # partition of the intermediate rows adds up to the layer
    import moe_inputs as mi
    layer, x = mi.workload_inputs("tiny")
    L = oracle.Layer.from_shape(layer, mi.TINY)
    idx, w, _, _ = oracle.router(x, layer["router_w"], mi.TINY.k)
    _, full = oracle.forward(L, x, idx, w, want_double=True)
    parts = [oracle.forward_range(L, x, idx, w, a, b, want_double=True)[1]
             for a, b in zip(cuts[:-1], cuts[1:])]
    rms = np.sqrt(np.mean(full ** 2))
    assert np.abs(sum(parts) - full).max() <= 1e-12 * rms
    # an equal split through the range form is the equal-shard form, bit for bit
    if len(cuts) == 3 and cuts[1] == 64:
        assert np.array_equal(parts[0], oracle.forward(L, x, idx, w, 0, 2, want_double=True)[1])
    # an empty range contributes nothing
    assert not np.any(oracle.forward_range(L, x, idx, w, 64, 64))


# --------------------------------------------------------------------------
# MXFP4 superblocks
# --------------------------------------------------------------------------

MX_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_handworked.txt")
MX = read_fixture(MX_GOLDEN)
MX_SCALES = [127, 126, 128, 121, 130, 113, 125, 140]
# FP4 E2M1 values of codes 0..15 as the OCP MX specification tabulates them
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
              -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def _mx_blob():
    return np.frombuffer(MX["scales"] + MX["reserved"] + MX["mx_qs"], np.uint8)


def test_e2m1_matches_the_spec_table():
    for code, v in enumerate(E2M1_TABLE):
        got = oracle.e2m1(code)
        assert got == v and math.copysign(1.0, got) == math.copysign(1.0, v), code


def test_e8m0_scales():
    assert oracle.e8m0(127) == 1.0
    assert oracle.e8m0(120) == 1.0 / 128
    assert oracle.e8m0(140) == 8192.0
    assert oracle.e8m0(0) == 2.0 ** -127
    assert oracle.e8m0(254) == 2.0 ** 127
    assert math.isnan(oracle.e8m0(255))


def test_mx_packer_matches_fixture():
    q = _q4_codes()   # i mod 16 in even sub-blocks, 15 - (i mod 16) in odd ones
    assert MX["scales"] == bytes(MX_SCALES) and MX["reserved"] == bytes(8)
    assert pack_mx_sb(MX_SCALES, q).tobytes() == _mx_blob().tobytes()


def test_handworked_mxfp4():
    w = oracle.dequant(_mx_blob(), oracle.SB_MXFP4)
    for i, v in MX["mx_values"].items():
        ref = float(Fraction(v))
        assert w[i] == np.float32(ref), (i, w[i], v)
        if v.startswith("-"):
            assert np.signbit(w[i]), i          # -0 keeps its sign
    # every element: the spec's table value of its code times its block's
    # power of two (exact fractions)
    q = _q4_codes()
    expect = np.array([float(Fraction(E2M1_TABLE[q[i]]) * Fraction(2) ** (MX_SCALES[i // 32] - 127))
                       for i in range(256)], np.float32)
    assert np.array_equal(w, expect)


def test_mx_every_code_and_scale():
    """Each (code, scale byte) pair in one block: table value times 2^(s-127),
    for every scale byte whose products stay normal in fp32."""
    for s in list(range(1, 120, 7)) + list(range(120, 141)) + list(range(141, 250, 9)):
        q = list(range(16)) * 16
        w = oracle.dequant(pack_mx_sb([s] * 8, q), oracle.SB_MXFP4)
        expect = np.array([float(Fraction(E2M1_TABLE[c]) * Fraction(2) ** (s - 127)) for c in q],
                          np.float32)
        assert np.array_equal(w, expect), s


def test_mx_dense_ffn_special_case():
    """E=1, k=1, no shared expert, MXFP4 weights: a dense SwiGLU FFN on the
    decoded weights (numpy float64)."""
    import moe_inputs as mi
    shp = mi.LayerShape(H=256, E=1, k=1, I=128, Is=0, fmt=1)
    arrays = mi.make_layer(shp, seed=12)
    assert arrays["down"].shape == (1, 256 * 128 // 256 * mi.MXFP4_SB_BYTES)
    L = oracle.Layer.from_shape(arrays, shp)
    x = mi.make_tokens(shp, 12, 3)
    o = oracle.forward(L, x)
    Wg = oracle.dequant(arrays["gate"][0], oracle.SB_MXFP4).reshape(128, 256).astype(np.float64)
    Wu = oracle.dequant(arrays["up"][0], oracle.SB_MXFP4).reshape(128, 256).astype(np.float64)
    Wd = oracle.dequant(arrays["down"][0], oracle.SB_MXFP4).reshape(256, 128).astype(np.float64)
    g = x.astype(np.float64) @ Wg.T
    u = x.astype(np.float64) @ Wu.T
    ref = ((g / (1 + np.exp(-g))) * u) @ Wd.T
    assert np.allclose(o, ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())


def test_mx_shard_partials_sum_to_whole():
    """An MXFP4 layer's shard partials add up to the whole layer."""
    import moe_inputs as mi
    layer, x = mi.workload_inputs("tiny_mx")
    Lmx = oracle.Layer.from_shape(layer, mi.TINY_MX)
    idx, w, _, _ = oracle.router(x, layer["router_w"], mi.TINY_MX.k)
    _, full = oracle.forward(Lmx, x, idx, w, want_double=True)
    parts = [oracle.forward(Lmx, x, idx, w, s, 2, want_double=True)[1] for s in range(2)]
    rms = np.sqrt(np.mean(full ** 2))
    assert rms > 0 and np.all(np.isfinite(full))
    assert np.abs(sum(parts) - full).max() <= 1e-12 * rms
