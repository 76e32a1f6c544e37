"""Quantizers that turn random fp32 weights into the canonical block bytes.

This is artifact construction (choosing codes and scales for given weights),
not part of the verify round: the round only decodes.  The canonical byte
layouts are defined here and, independently, in the oracle's decoder; the
header include/specverify.h states them for library users.

b4_32  (32 weights, 18 B):  [d fp16][16 B codes]; code k in byte k/2, low
       nibble for even k.  w_k = d * (q_k - 8).
b4_256 (256 weights, 144 B): [d fp16][dmin fp16][12 B: sixteen 6-bit fields,
       LSB-first bitstream: sc_0..sc_7 then m_0..m_7][128 B codes as b4_32].
       Sub-block j = k/32.  w_k = d*sc_j*q_k - dmin*m_j.
b6_256 (256 weights, 210 B): [128 B low nibbles as b4_32][64 B high 2-bit
       fields: code k's bits 4..5 at byte k/4, bit 2*(k%4)][16 B int8 sc_j]
       [d fp16].  Sub-block j = k/16.  w_k = d*sc_j*(q_k - 32).

All functions take a float32 torch tensor [rows][cols] on any device and return
uint8 [rows][cols/block * bytes] on the same device.
"""

import torch


def _f16_bytes(x: torch.Tensor) -> torch.Tensor:
    """fp16 tensor [..] -> uint8 [.., 2] little-endian."""
    x = x.to(torch.float16).contiguous()
    return x.view(torch.uint8).reshape(*x.shape, 2)


def _safe_inv(x: torch.Tensor) -> torch.Tensor:
    return torch.where(x > 0, 1.0 / torch.where(x > 0, x, torch.ones_like(x)),
                       torch.zeros_like(x))


def _pack_nibbles(q: torch.Tensor) -> torch.Tensor:
    """uint8 codes [.., 2n] -> [.., n]: code k in byte k/2, low nibble for even k."""
    return (q[..., 0::2] | (q[..., 1::2] << 4)).to(torch.uint8)


def quantize_b4_32(w: torch.Tensor) -> torch.Tensor:
    rows, cols = w.shape
    assert cols % 32 == 0
    b = w.float().reshape(rows, cols // 32, 32)
    amax = b.abs().amax(-1)
    d16 = (amax / 7.0).to(torch.float16)
    inv = _safe_inv(d16.float())
    q = torch.clamp(torch.round(b * inv[..., None]) + 8, 0, 15).to(torch.uint8)
    out = torch.cat([_f16_bytes(d16), _pack_nibbles(q)], dim=-1)
    return out.reshape(rows, -1).contiguous()


def quantize_b4_256(w: torch.Tensor) -> torch.Tensor:
    rows, cols = w.shape
    assert cols % 256 == 0
    b = w.float().reshape(rows, cols // 256, 8, 32)
    lo = torch.clamp(b.amin(-1), max=0.0)
    hi = b.amax(-1)
    step = (hi - lo) / 15.0           # per sub-block step
    off = -lo                         # per sub-block offset, >= 0
    d16 = (step.amax(-1) / 63.0).to(torch.float16)
    dm16 = (off.amax(-1) / 63.0).to(torch.float16)
    sc = torch.clamp(torch.round(step * _safe_inv(d16.float())[..., None]), 0, 63)
    m = torch.clamp(torch.round(off * _safe_inv(dm16.float())[..., None]), 0, 63)
    scale = d16.float()[..., None] * sc            # effective sub-block step
    zero = dm16.float()[..., None] * m             # effective sub-block offset
    q = torch.clamp(torch.round((b + zero[..., None]) * _safe_inv(scale)[..., None]),
                    0, 15).to(torch.uint8)
    # sixteen 6-bit fields, LSB-first: four 24-bit groups of four fields
    f = torch.cat([sc, m], dim=-1).to(torch.int64)            # [rows, nsb, 16]
    g = f.reshape(rows, cols // 256, 4, 4)
    v = g[..., 0] | (g[..., 1] << 6) | (g[..., 2] << 12) | (g[..., 3] << 18)
    fb = torch.stack([v & 0xFF, (v >> 8) & 0xFF, (v >> 16) & 0xFF], dim=-1)
    fb = fb.reshape(rows, cols // 256, 12).to(torch.uint8)
    codes = _pack_nibbles(q.reshape(rows, cols // 256, 256))
    out = torch.cat([_f16_bytes(d16), _f16_bytes(dm16), fb, codes], dim=-1)
    return out.reshape(rows, -1).contiguous()


def quantize_b6_256(w: torch.Tensor) -> torch.Tensor:
    rows, cols = w.shape
    assert cols % 256 == 0
    b = w.float().reshape(rows, cols // 256, 16, 16)
    amax = b.abs().amax(-1)
    step = amax / 31.0
    d16 = (step.amax(-1) / 127.0).to(torch.float16)
    sc = torch.clamp(torch.round(step * _safe_inv(d16.float())[..., None]), -128, 127)
    scale = d16.float()[..., None] * sc
    q = torch.clamp(torch.round(b * _safe_inv(scale)[..., None]) + 32, 0, 63)
    q = q.to(torch.uint8).reshape(rows, cols // 256, 256)
    low = _pack_nibbles(q & 15)
    h = (q >> 4) & 3
    high = (h[..., 0::4] | (h[..., 1::4] << 2) | (h[..., 2::4] << 4)
            | (h[..., 3::4] << 6)).to(torch.uint8)
    scb = sc.to(torch.int8).view(torch.uint8)
    out = torch.cat([low, high, scb, _f16_bytes(d16)], dim=-1)
    return out.reshape(rows, -1).contiguous()


QUANTIZERS = {"b4_32": quantize_b4_32, "b4_256": quantize_b4_256,
              "b6_256": quantize_b6_256}


def quantize(fmt: str, w: torch.Tensor) -> torch.Tensor:
    return QUANTIZERS[fmt](w)
