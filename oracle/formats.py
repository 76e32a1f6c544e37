"""Decode the canonical block formats into fp64 weights, field by field.

TEST INFRASTRUCTURE (part of the oracle): see oracle/__init__.py.

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

Each weight is formed by the formula of its format, evaluated left to right
in fp64: (d*sc_j)*q - dmin*m_j and (d*sc_j)*(q-32).  Sub-blocks are selected
by reshaping a block's codes into [sub-block][weight] and broadcasting the
sub-block's factors over it.
"""

import numpy as np

BLOCK = {"b4_32": (32, 18), "b4_256": (256, 144), "b6_256": (256, 210)}


def _f16(two_bytes: np.ndarray) -> np.ndarray:
    """uint8 [..., 2] little-endian fp16 -> fp64 [...]."""
    b = np.ascontiguousarray(two_bytes, dtype=np.uint8)
    return b.view("<f2")[..., 0].astype(np.float64)


def _codes4(byts: np.ndarray) -> np.ndarray:
    """Nibble array [..., n] -> codes [..., 2n]: code k is in byte k//2, the
    low nibble for even k and the high nibble for odd k."""
    lo = byts & np.uint8(0xF)
    hi = byts >> np.uint8(4)
    return np.stack([lo, hi], axis=-1).reshape(byts.shape[:-1] + (2 * byts.shape[-1],))


def _fields6(byts: np.ndarray, n: int) -> np.ndarray:
    """n 6-bit fields from an LSB-first bitstream [..., bytes] -> int64 [..., n]."""
    bits = np.unpackbits(byts, axis=-1, bitorder="little")[..., : 6 * n]
    bits = bits.reshape(bits.shape[:-1] + (n, 6)).astype(np.int64)
    return bits @ (np.int64(1) << np.arange(6, dtype=np.int64))


def decode_b4_32(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    blk = np.asarray(raw, dtype=np.uint8).reshape(rows, cols // 32, 18)
    d = _f16(blk[..., 0:2])                                   # [rows][blocks]
    q = _codes4(blk[..., 2:18]).astype(np.float64)            # [rows][blocks][32]
    return (d[..., None] * (q - 8.0)).reshape(rows, cols)


def decode_b4_256(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    nsb = cols // 256
    blk = np.asarray(raw, dtype=np.uint8).reshape(rows, nsb, 144)
    d = _f16(blk[..., 0:2])
    dmin = _f16(blk[..., 2:4])
    f = _fields6(blk[..., 4:16], 16)
    sc = f[..., 0:8].astype(np.float64)                       # [rows][nsb][8]
    mn = f[..., 8:16].astype(np.float64)
    q = _codes4(blk[..., 16:144]).astype(np.float64).reshape(rows, nsb, 8, 32)
    scale = d[..., None] * sc                                 # d * sc_j
    offset = dmin[..., None] * mn                             # dmin * m_j
    w = scale[..., None] * q - offset[..., None]
    return w.reshape(rows, cols)


def decode_b6_256(raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    nsb = cols // 256
    blk = np.asarray(raw, dtype=np.uint8).reshape(rows, nsb, 210)
    lo = _codes4(blk[..., 0:128])                              # bits 0..3 of code k
    h = blk[..., 128:192]                                      # byte k//4, bits 2*(k%4)
    hi = np.stack([h & 3, (h >> 2) & 3, (h >> 4) & 3, h >> 6], axis=-1)
    hi = hi.reshape(rows, nsb, 256)
    q = (lo | (hi << np.uint8(4))).astype(np.float64).reshape(rows, nsb, 16, 16)
    sc = np.ascontiguousarray(blk[..., 192:208]).view(np.int8).astype(np.float64)
    d = _f16(blk[..., 208:210])
    scale = d[..., None] * sc                                  # d * sc_j
    w = scale[..., None] * (q - 32.0)
    return w.reshape(rows, cols)


_DECODERS = {"b4_32": decode_b4_32, "b4_256": decode_b4_256, "b6_256": decode_b6_256}


def decode(fmt: str, raw: np.ndarray, rows: int, cols: int) -> np.ndarray:
    return _DECODERS[fmt](raw, rows, cols)


def decode_rows(fmt: str, raw: np.ndarray, cols: int, r0: int, r1: int) -> np.ndarray:
    """Decode output rows [r0, r1) of a tensor whose bytes are `raw` [rows][B]."""
    raw = np.asarray(raw, dtype=np.uint8)
    return decode(fmt, raw[r0:r1], r1 - r0, cols)
