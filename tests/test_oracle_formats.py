"""Pins of the oracle's block decoders.

* Hand-built blocks (tests/golden/format_blocks.json) whose decoded values are
  closed forms of k fixed by the format definitions: scale factors, code
  offsets (8 and 32), nibble order, 6-bit field order and the 2-bit plane.
* Round trip: the generator's quantizer (an independent writer of the same
  byte layout) followed by the oracle's decoder reproduces random weights to
  within half a quantization step per weight.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle.formats import decode, BLOCK
from synth.quant import quantize


def _blocks(golden_dir):
    with open(os.path.join(golden_dir, "format_blocks.json")) as f:
        return json.load(f)["blocks"]


def test_golden_blocks(golden_dir):
    blocks = _blocks(golden_dir)
    assert len(blocks) == 5
    for b in blocks:
        raw = np.frombuffer(bytes.fromhex(b["hex"]), dtype=np.uint8)
        n, nb = BLOCK[b["format"]]
        assert raw.size == nb
        got = decode(b["format"], raw, 1, n)[0]
        k = np.arange(n)
        want = np.array([eval(b["closed_form"], {}, {"k": int(kk)}) for kk in k],
                        dtype=np.float64)
        np.testing.assert_array_equal(got, want, err_msg=b["name"])


def test_multi_row_multi_block_order():
    """Row-major rows, blocks in k order: two rows of two b4_32 blocks with
    distinct scales land where they should."""
    def blk(d_hex, code):
        return bytes.fromhex(d_hex) + bytes([code | (code << 4)] * 16)
    raw = blk("003c", 9) + blk("0040", 10) + blk("0044", 7) + blk("0048", 8)
    w = decode("b4_32", np.frombuffer(raw, np.uint8), 2, 64)
    np.testing.assert_array_equal(w[0, :32], 1.0)      # d=1, q-8 = 1
    np.testing.assert_array_equal(w[0, 32:], 4.0)      # d=2, q-8 = 2
    np.testing.assert_array_equal(w[1, :32], -4.0)     # d=4, q-8 = -1
    np.testing.assert_array_equal(w[1, 32:], 0.0)      # d=8, q-8 = 0


@pytest.mark.parametrize("fmt", ["b4_32", "b4_256", "b6_256"])
def test_quantize_roundtrip_half_step(fmt):
    torch.manual_seed(5)
    rows, cols = 24, 512
    w = torch.randn(rows, cols) * 0.02
    raw = quantize(fmt, w).numpy()
    n, nb = BLOCK[fmt]
    assert raw.shape == (rows, cols // n * nb)
    deq = decode(fmt, raw, rows, cols)
    err = np.abs(deq - w.double().numpy())
    if fmt == "b4_32":
        d = np.frombuffer(raw.reshape(rows, -1, 18)[..., :2].tobytes(), "<f2")
        step = np.repeat(d.astype(np.float64).reshape(rows, -1), 32, axis=1)
        bound = 0.5 * step
        # the clamp at q = 0 (-8 d) can exceed half a step only beyond -7.5 d
    elif fmt == "b4_256":
        # rounding sc and m to 6 bits can shift the code grid's ends by up to
        # half a super step each: err <= scale_j/2 + dmin/2 + 7.5 d
        blk = raw.reshape(rows, -1, 144)
        d = np.frombuffer(blk[..., 0:2].tobytes(), "<f2").astype(np.float64)
        dmin = np.frombuffer(blk[..., 2:4].tobytes(), "<f2").astype(np.float64)
        bits = np.unpackbits(blk[..., 4:16], axis=-1, bitorder="little")
        sc = np.zeros(bits.shape[:-1] + (8,))
        for i in range(8):
            sc[..., i] = sum(bits[..., 6 * i + b].astype(np.int64) << b for b in range(6))
        d = d.reshape(rows, -1, 1)
        dmin = dmin.reshape(rows, -1, 1)
        bound = (0.5 * d * sc + 0.5 * dmin + 7.5 * d)
        bound = np.repeat(bound.reshape(rows, -1), 32, axis=1)
    else:
        blk = raw.reshape(rows, -1, 210)
        d = np.frombuffer(blk[..., 208:210].tobytes(), "<f2").astype(np.float64)
        sc = blk[..., 192:208].view(np.int8).astype(np.float64)
        step = np.repeat((d.reshape(rows, -1, 1) * np.abs(sc)).reshape(rows, -1), 16,
                         axis=1)
        dd = np.repeat(d.reshape(rows, -1), 256, axis=1)
        bound = 0.5 * step + 16 * dd
    assert np.all(err <= bound + 1e-12), float((err - bound).max())
    # and the quantization is not vacuous: relative RMS error is small
    rel = np.sqrt(np.mean(err ** 2)) / 0.02
    assert rel < {"b4_32": 0.12, "b4_256": 0.12, "b6_256": 0.04}[fmt], rel
