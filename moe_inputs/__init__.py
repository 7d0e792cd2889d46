"""Seeded synthetic workloads for the routed Mixture-of-Experts layer.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It draws random numbers and nothing else: it holds none of the
layer's arithmetic (no dequantisation, routing, FFN or combine).

Workloads follow the shapes of a Qwen3.5-35B-A3B routed MoE layer as described
on the page "CKE Zip: From Splitting Tokens To Splitting Qwen3.5 Weights"
(section "What PR #382 Now Splits": 256 routed experts, eight selected per
token, 4-bit K-quant gate/up, 5-bit K-quant down, a shared expert, a 256/256
intermediate split).  Real weights are not available; every tensor here is a
seeded stand-in with the distributions stated below.

K-quant blobs
-------------
A superblock (SB) holds 256 weights.  Its first four bytes are the fp16 fields
``d`` and ``dmin`` (little endian); the remaining bytes (140 for the 4-bit
format, 172 for the 5-bit one) hold the packed 6-bit scales/mins, the code
nibbles and, for 5 bits, the high code bits.  Every one of those remaining bits
is used exactly once by the format, so uniform random bytes give exactly the
workload's distributions: scales and mins uniform on 0..63, codes uniform on
0..15 (4-bit) or 0..31 (5-bit).  ``d`` and ``dmin`` are fp16 roundings (round to
nearest even) of fp32 draws uniform on [1e-3, 4e-3].

MXFP4 blobs
-----------
The second weight format (``LayerShape.fmt == 1``; gate, up and down all use
it): a 144-byte superblock of 256 weights, bytes 0..7 the E8M0 scale bytes of
its eight 32-weight blocks, bytes 8..15 zero (reserved), bytes 16..143 the
4-bit E2M1 codes in the nibble order of the 4-bit K-quant superblock.  Scale
bytes are uniform on ``LayerShape.mx_scales`` (by default 116..132, block
scales 2^-11 .. 2^5) and codes uniform on 0..15.

Weight matrices are stored one row per output feature with the reduction
dimension contiguous, quantised in flat row-major order in 256-element
superblocks (so a superblock may span several rows when the row is shorter
than 256).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

Q4K_SB_BYTES = 144   # fp16 d, fp16 dmin, 12 scale bytes, 128 code bytes
Q5K_SB_BYTES = 176   # as Q4K plus 32 bytes of high code bits
MXFP4_SB_BYTES = 144  # 8 E8M0 scale bytes, 8 reserved bytes, 128 code bytes
MXFP4_SCALE_RANGE = (116, 132)   # E8M0 scale bytes drawn uniformly (inclusive), by default
SB_WEIGHTS = 256

# Stream ids: every tensor (and every expert of it) draws from its own stream
# so that one expert can be regenerated without the others.
_S_ROUTER, _S_GATE, _S_UP, _S_DOWN = 1, 2, 3, 4
_S_SH_GATE, _S_SH_UP, _S_SH_DOWN = 5, 6, 7
_S_X, _S_ZIPF_V, _S_ZIPF_RANK = 8, 9, 10


@dataclass(frozen=True)
class LayerShape:
    H: int          # hidden width
    E: int          # routed experts
    k: int          # experts selected per token
    I: int          # routed-expert intermediate width
    Is: int         # shared-expert intermediate width (0 = no shared expert)
    shared_weight: float = 1.0
    fmt: int = 0    # 0: Q4_K gate/up and Q5_K down; 1: MXFP4 gate, up and down
    mx_scales: tuple = MXFP4_SCALE_RANGE   # MXFP4: E8M0 scale bytes drawn uniformly (inclusive)

    def sb_counts(self):
        """Superblocks per matrix: gate/up (I x H), down (H x I), shared ones."""
        return (self.I * self.H // SB_WEIGHTS, self.H * self.I // SB_WEIGHTS,
                self.Is * self.H // SB_WEIGHTS, self.H * self.Is // SB_WEIGHTS)


QWEN35_MOE = LayerShape(H=2048, E=256, k=8, I=512, Is=512)
TINY = LayerShape(H=256, E=8, k=2, I=128, Is=128)
QWEN35_MOE_MX = LayerShape(H=2048, E=256, k=8, I=512, Is=512, fmt=1)
TINY_MX = LayerShape(H=256, E=8, k=2, I=128, Is=128, fmt=1)


@dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    seed: int
    T: int
    zipf: bool = False          # non-uniform (Zipf-like) expert load
    shards: int = 1             # 1 = unsharded; 2 = the 256/256 split
    x_stream: int = 0           # which independent token set of the seed
    note: str = ""


# Zipf-like load: strength of the per-expert logit offset.  Fitted once with
# the oracle's router so that a log-log fit of realised per-expert slot counts
# at T=512 has slope -1.0 +- 0.1 (checked by tests/test_inputs.py).
ZIPF_BETA = 1.0

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", TINY, seed=0, T=4,
                     note="tiny layer, seed 0, T=4"),
    "decode": Workload("decode", QWEN35_MOE, seed=1, T=1,
                       note="Qwen3.5-35B-A3B-shaped layer, decode T=1"),
    "decode_sharded": Workload("decode_sharded", QWEN35_MOE, seed=2, T=1, shards=2,
                               note="same layer, 256/256 two-shard decode T=1"),
    "decode_batched": Workload("decode_batched", QWEN35_MOE, seed=2, T=32, shards=2, x_stream=1,
                               note="same layer, batched decode T=32 (sharded and not)"),
    "prefill512_zipf": Workload("prefill512_zipf", QWEN35_MOE, seed=3, T=512, zipf=True,
                                note="same layer, prefill T=512, Zipf-like expert load"),
    "prefill4096": Workload("prefill4096", QWEN35_MOE, seed=4, T=4096, shards=2,
                            note="same layer, prefill T=4096, uniform router (unsharded and 2-shard)"),
    # the same shapes with MXFP4 expert weights
    "tiny_mx": Workload("tiny_mx", TINY_MX, seed=5, T=4,
                        note="tiny layer, MXFP4 weights, seed 5, T=4"),
    "decode_mx": Workload("decode_mx", QWEN35_MOE_MX, seed=6, T=1,
                          note="Qwen3.5-35B-A3B-shaped layer, MXFP4 weights, decode T=1"),
    "prefill4096_mx": Workload("prefill4096_mx", QWEN35_MOE_MX, seed=7, T=4096, shards=2,
                               note="same layer, MXFP4 weights, prefill T=4096, uniform router"),
}


def _rng(seed: int, stream: int, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, sub])))


def kquant_blob(rng: np.random.Generator, n_sb: int, bits: int) -> np.ndarray:
    """``n_sb`` random superblocks of the 4- or 5-bit format as a flat uint8 array."""
    sb_bytes = Q4K_SB_BYTES if bits == 4 else Q5K_SB_BYTES
    d = rng.uniform(1e-3, 4e-3, size=n_sb).astype(np.float32).astype(np.float16)
    dmin = rng.uniform(1e-3, 4e-3, size=n_sb).astype(np.float32).astype(np.float16)
    body = np.frombuffer(rng.bytes(n_sb * (sb_bytes - 4)), dtype=np.uint8)
    blob = np.empty((n_sb, sb_bytes), dtype=np.uint8)
    blob[:, 0:2] = d.astype("<f2").view(np.uint8).reshape(n_sb, 2)
    blob[:, 2:4] = dmin.astype("<f2").view(np.uint8).reshape(n_sb, 2)
    blob[:, 4:] = body.reshape(n_sb, sb_bytes - 4)
    return blob.reshape(-1)


def mxfp4_blob(rng: np.random.Generator, n_sb: int, scales=MXFP4_SCALE_RANGE) -> np.ndarray:
    """``n_sb`` random MXFP4 superblocks as a flat uint8 array, scale bytes
    uniform on ``scales`` (inclusive)."""
    lo, hi = scales
    blob = np.zeros((n_sb, MXFP4_SB_BYTES), dtype=np.uint8)
    blob[:, 0:8] = rng.integers(lo, hi + 1, size=(n_sb, 8), dtype=np.uint8)
    blob[:, 16:] = np.frombuffer(rng.bytes(n_sb * 128), dtype=np.uint8).reshape(n_sb, 128)
    return blob.reshape(-1)


def weight_blob(rng: np.random.Generator, n_sb: int, bits: int, fmt: int,
                mx_scales=MXFP4_SCALE_RANGE) -> np.ndarray:
    """Superblocks of a layer's format: K-quant of ``bits`` bits, or MXFP4."""
    return mxfp4_blob(rng, n_sb, mx_scales) if fmt == 1 else kquant_blob(rng, n_sb, bits)


def _zipf_parts(shape: LayerShape, seed: int):
    """Unit vector v and per-expert offsets b (b_e = -beta * ln(rank_e))."""
    rv = _rng(seed, _S_ZIPF_V)
    v = rv.standard_normal(shape.H)
    v = (v / np.sqrt(np.dot(v, v))).astype(np.float32)
    ranks = _rng(seed, _S_ZIPF_RANK).permutation(shape.E) + 1
    b = (-ZIPF_BETA * np.log(ranks.astype(np.float64))).astype(np.float32)
    return v, b, ranks


def make_layer(shape: LayerShape, seed: int, zipf: bool = False) -> Dict[str, np.ndarray]:
    """All weights of one layer as host arrays.

    router_w  fp32 [H][E]             ~ N(0, 0.02^2)  (+ v b^T for the Zipf workload)
    gate, up  uint8 [E][I*H/256*144]  4-bit superblocks, rows = I outputs, K = H
    down      uint8 [E][H*I/256*176]  5-bit superblocks, rows = H outputs, K = I
    sh_gate, sh_up, sh_down           the shared expert, same formats, width Is
    (shape.fmt == 1: every matrix in 144-byte MXFP4 superblocks instead)
    """
    n_gu, n_d, n_sgu, n_sd = shape.sb_counts()
    wr = _rng(seed, _S_ROUTER).normal(0.0, 0.02, size=(shape.H, shape.E)).astype(np.float32)
    if zipf:
        v, b, _ = _zipf_parts(shape, seed)
        wr = (wr + np.outer(v, b)).astype(np.float32)

    f = shape.fmt

    ms = shape.mx_scales

    def stack(stream, n_sb, bits):
        return np.stack([weight_blob(_rng(seed, stream, e), n_sb, bits, f, ms)
                         for e in range(shape.E)])

    layer = {
        "router_w": np.ascontiguousarray(wr),
        "gate": stack(_S_GATE, n_gu, 4),
        "up": stack(_S_UP, n_gu, 4),
        "down": stack(_S_DOWN, n_d, 5),
    }
    if shape.Is > 0:
        layer["sh_gate"] = weight_blob(_rng(seed, _S_SH_GATE), n_sgu, 4, f, ms)
        layer["sh_up"] = weight_blob(_rng(seed, _S_SH_UP), n_sgu, 4, f, ms)
        layer["sh_down"] = weight_blob(_rng(seed, _S_SH_DOWN), n_sd, 5, f, ms)
    return layer


def make_tokens(shape: LayerShape, seed: int, T: int, stream: int = 0,
                zipf: bool = False) -> np.ndarray:
    """Token rows x fp32 [T][H] ~ N(0, 1) (plus the unit vector v for the Zipf workload).

    ``stream`` selects independent token sets of the same workload (e.g. a pool
    of decode tokens, or the batched-decode rows)."""
    x = _rng(seed, _S_X, stream).standard_normal((T, shape.H)).astype(np.float32)
    if zipf:
        v, _, _ = _zipf_parts(shape, seed)
        x = (x + v[None, :]).astype(np.float32)
    return np.ascontiguousarray(x)


def workload_inputs(name: str, T: Optional[int] = None, stream: Optional[int] = None):
    """(layer, x) for a named workload."""
    w = WORKLOADS[name]
    layer = make_layer(w.shape, w.seed, zipf=w.zipf)
    x = make_tokens(w.shape, w.seed, w.T if T is None else T,
                    stream=w.x_stream if stream is None else stream, zipf=w.zipf)
    return layer, x
