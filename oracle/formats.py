"""Decode the canonical block formats into fp64 weights, field by field.

The three formats are the ones the workloads fix: a 4-bit format in blocks of
32 with an fp16 scale (w = d*(q-8)); a 4-bit super-block of 256 made of eight
32-weight sub-blocks with 6-bit scale and min and fp16 super scale and super
min (read as w = d*sc_j*q - dmin*m_j); a 6-bit super-block of 256 made of
sixteen 16-weight sub-blocks with signed 8-bit scales and an fp16 super scale
(read as w = d*sc_j*(q-32)).  The byte layout inside a block is this
project's own (no GGUF artifact is involved):

b4_32  18 B: d fp16 | 16 B codes (code k in byte k//2, low nibble if k even)
b4_256 144 B: d fp16 | dmin fp16 | 12 B bitstream of sixteen 6-bit fields,
       field i at bits [6i, 6i+6) counted LSB-first from byte 0
       (sc_0..sc_7 then m_0..m_7) | 128 B codes as in b4_32
b6_256 210 B: 128 B low nibbles as in b4_32 | 64 B high bits (bits 4..5 of
       code k at byte k//4, bit offset 2*(k%4)) | 16 B int8 sc_j | d fp16

A tensor with `rows` output features and `cols` inputs is stored row by row,
each row being cols/block_size blocks in order of k.
"""

import numpy as np

BLOCK = {"b4_32": (32, 18), "b4_256": (256, 144), "b6_256": (256, 210)}


def _f16(two_bytes: np.ndarray) -> np.ndarray:
    """uint8 [..., 2] little-endian fp16 -> fp64 [...]."""
    b = np.ascontiguousarray(two_bytes, dtype=np.uint8)
    return b.view("<f2")[..., 0].astype(np.float64)


def _nibble(byts: np.ndarray, k: np.ndarray) -> np.ndarray:
    """code k out of a nibble array (byte k//2, low nibble for even k)."""
    return (byts[..., k // 2] >> (4 * (k % 2)).astype(np.uint8)) & np.uint8(0xF)


def decode_b4_32(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    blk = np.asarray(raw, dtype=np.uint8).reshape(rows, cols // 32, 18)
    d = _f16(blk[..., 0:2])
    k = np.arange(32)
    q = _nibble(blk[..., 2:18], k).astype(np.float64)
    return (d[..., None] * (q - 8.0)).reshape(rows, cols)


def decode_b4_256(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    blk = np.asarray(raw, dtype=np.uint8).reshape(rows, cols // 256, 144)
    d = _f16(blk[..., 0:2])
    dmin = _f16(blk[..., 2:4])
    bits = np.unpackbits(blk[..., 4:16], axis=-1, bitorder="little")  # [..,96]
    fields = np.zeros(bits.shape[:-1] + (16,), dtype=np.int64)
    for i in range(16):
        for b in range(6):
            fields[..., i] |= bits[..., 6 * i + b].astype(np.int64) << b
    sc = fields[..., 0:8].astype(np.float64)
    mn = fields[..., 8:16].astype(np.float64)
    k = np.arange(256)
    q = _nibble(blk[..., 16:144], k).astype(np.float64)
    j = k // 32
    w = d[..., None] * sc[..., j] * q - dmin[..., None] * mn[..., j]
    return w.reshape(rows, cols)


def decode_b6_256(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    blk = np.asarray(raw, dtype=np.uint8).reshape(rows, cols // 256, 210)
    k = np.arange(256)
    lo = _nibble(blk[..., 0:128], k).astype(np.int64)
    hi = ((blk[..., 128 + k // 4] >> (2 * (k % 4)).astype(np.uint8)) & 3).astype(np.int64)
    q = (lo | (hi << 4)).astype(np.float64)
    sc = np.ascontiguousarray(blk[..., 192:208]).view(np.int8).astype(np.float64)
    d = _f16(blk[..., 208:210])
    w = d[..., None] * sc[..., k // 16] * (q - 32.0)
    return w.reshape(rows, cols)


_DECODERS = {"b4_32": decode_b4_32, "b4_256": decode_b4_256, "b6_256": decode_b6_256}


def decode(fmt: str, raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    return _DECODERS[fmt](raw, rows, cols)


def decode_rows(fmt: str, raw: np.ndarray, cols: int, r0: int, r1: int) -> np.ndarray:
    """Decode output rows [r0, r1) of a tensor whose bytes are `raw` [rows][B]."""
    raw = np.asarray(raw, dtype=np.uint8)
    return decode(fmt, raw[r0:r1], r1 - r0, cols)
