"""Test-side K-quant packer: fields -> superblock bytes.

Written from the layout in tests/golden/kquant_handworked.txt, independently of
both the oracle's and the GPU library's decoders.  It is itself pinned by the
literal bytes of that fixture (test_oracle.py::test_packer_matches_fixture).
"""
import numpy as np


def pack_scales(sc, m):
    """Eight 6-bit (scale, min) pairs -> the 12 packed scale bytes."""
    b = [0] * 12
    for j in range(4):
        b[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        b[j + 4] = (m[j] & 63) | ((m[j + 4] >> 4) << 6)
        b[j + 8] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    return bytes(b)


def pack_sb(d_bits, dmin_bits, sc, m, q, bits):
    """One superblock from fp16 bit patterns, 8 scales, 8 mins and 256 codes."""
    q = [int(v) for v in q]
    assert len(q) == 256 and all(0 <= v < (16 if bits == 4 else 32) for v in q)
    qs = bytearray(128)
    qh = bytearray(32)
    for c in range(4):
        for l in range(32):
            lo, hi = q[64 * c + l], q[64 * c + 32 + l]
            qs[32 * c + l] = (lo & 15) | ((hi & 15) << 4)
            if bits == 5:
                qh[l] |= ((lo >> 4) & 1) << (2 * c)
                qh[l] |= ((hi >> 4) & 1) << (2 * c + 1)
    head = bytes([d_bits & 255, d_bits >> 8, dmin_bits & 255, dmin_bits >> 8]) + pack_scales(sc, m)
    body = (bytes(qh) if bits == 5 else b"") + bytes(qs)
    return np.frombuffer(head + body, dtype=np.uint8).copy()


def read_fixture(path):
    """Parse kquant_handworked.txt into a dict of byte strings / value maps."""
    out = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, rest = line.split(None, 1)
        if key.endswith("_w512"):
            out[key] = {int(a): int(b) for a, b in (t.split(":") for t in rest.split())}
        elif key.endswith("_values"):
            out[key] = {int(a): b for a, b in (t.split(":") for t in rest.split())}
        elif key.endswith("_bits"):
            out[key] = int(rest, 16)
        else:
            out.setdefault(key, b"")
            out[key] += bytes(int(t, 16) for t in rest.split())
    return out


def pack_mx_sb(scales, q):
    """One MXFP4 superblock from 8 E8M0 scale bytes and 256 codes (0..15), in the
    layout of tests/golden/mxfp4_handworked.txt."""
    q = [int(v) for v in q]
    assert len(q) == 256 and all(0 <= v < 16 for v in q) and len(scales) == 8
    qs = bytearray(128)
    for c in range(4):
        for l in range(32):
            qs[32 * c + l] = q[64 * c + l] | (q[64 * c + 32 + l] << 4)
    return np.frombuffer(bytes(scales) + bytes(8) + bytes(qs), dtype=np.uint8).copy()
