"""Test-side helpers: byte writers for hand-chosen block fields (exact-integer
GEMM cases), comparison rules, and input plumbing shared by the GPU tests.

The writers below are checked against the oracle's decoder on the CPU
(tests/test_packers.py), which is itself pinned to hand-built golden blocks.
"""

import numpy as np


def _f16b(x):
    return np.asarray(x, dtype="<f2").view(np.uint8).reshape(np.shape(x) + (2,))


def _nibbles(q):
    q = np.asarray(q, dtype=np.uint8)
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def pack_b4_32(d, q):
    """d [rows][nb] float, q [rows][nb][32] ints 0..15 -> bytes [rows][nb*18]."""
    d = np.asarray(d, dtype=np.float64)
    out = np.concatenate([_f16b(d), _nibbles(q)], axis=-1)
    return out.reshape(d.shape[0], -1)


def pack_b4_256(d, dmin, sc, m, q):
    """d, dmin [rows][nsb]; sc, m [rows][nsb][8] ints 0..63; q [rows][nsb][256]."""
    rows, nsb = np.shape(d)
    f = np.concatenate([sc, m], axis=-1).astype(np.int64)          # [rows][nsb][16]
    bits = np.zeros((rows, nsb, 96), dtype=np.uint8)
    for i in range(16):
        for b in range(6):
            bits[..., 6 * i + b] = (f[..., i] >> b) & 1
    fb = np.packbits(bits, axis=-1, bitorder="little")
    out = np.concatenate([_f16b(d), _f16b(dmin), fb, _nibbles(q)], axis=-1)
    return out.reshape(rows, -1)


def pack_b6_256(d, sc, q):
    """d [rows][nsb]; sc [rows][nsb][16] int8; q [rows][nsb][256] ints 0..63."""
    rows, nsb = np.shape(d)
    q = np.asarray(q, dtype=np.uint8)
    lo = _nibbles(q & 15)
    h = (q >> 4) & 3
    hi = (h[..., 0::4] | (h[..., 1::4] << 2) | (h[..., 2::4] << 4) | (h[..., 3::4] << 6))
    scb = np.asarray(sc, dtype=np.int8).view(np.uint8)
    out = np.concatenate([lo, hi.astype(np.uint8), scb, _f16b(d)], axis=-1)
    return out.reshape(rows, -1)


def logits_close(g, o, rtol=1e-3, atol=1e-4):
    """Elementwise |g - o| <= atol + rtol |o| (the workloads' logits bar)."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    bad = np.abs(g - o) > atol + rtol * np.abs(o)
    return not bad.any(), int(bad.sum()), float(np.max(np.abs(g - o)))


def top2_gap(row):
    row = np.asarray(row, dtype=np.float64)
    i = int(np.argmax(row))
    rest = np.delete(row, i)
    return row[i] - rest.max()
