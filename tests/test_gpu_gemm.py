"""GPU parity of the dequant-fused GEMM (sv_qgemm, the kernels every
projection and the lm_head run), against the oracle's decode and an fp64
product.

* exact integers: unit scales and small integer activations make every
  product and sum an integer below 2^24, so the GPU result must equal the
  integer result bit for bit (catches any code, scale or index mistake);
* random weights: |y - y64| <= 1e-5 * sum_k |x_k w_k| + 1e-7, the bound of
  fp32 accumulation of fp16-split activations (hi + lo carry 22 bits);
* row invariance: a row's bits do not depend on how many rows the call has,
  nor on which kernel runs it (up to 32 rows: one wave per K split; more
  rows on tensors with whole 256-column sets: the wide-M kernel, with 1, 2
  or 3 M-tiles per workgroup and a ragged last M group);
* sampled columns at the workloads' full lm_head shapes.
"""

import numpy as np
import pytest
import torch

import target_verification_amd as tva
from oracle.formats import decode
from synth.quant import quantize
from tests.gpu_util import pack_b4_32, pack_b4_256, pack_b6_256

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _int_case(fmt, rows, cols, rng):
    if fmt == "b4_32":
        q = rng.integers(0, 16, size=(rows, cols // 32, 32))
        raw = pack_b4_32(np.ones((rows, cols // 32)), q)
    elif fmt == "b4_256":
        nsb = cols // 256
        raw = pack_b4_256(np.ones((rows, nsb)), np.ones((rows, nsb)),
                          rng.integers(0, 64, size=(rows, nsb, 8)),
                          rng.integers(0, 64, size=(rows, nsb, 8)),
                          rng.integers(0, 16, size=(rows, nsb, 256)))
    else:
        nsb = cols // 256
        raw = pack_b6_256(np.ones((rows, nsb)), rng.integers(-128, 128, size=(rows, nsb, 16)),
                          rng.integers(0, 64, size=(rows, nsb, 256)))
    return raw


@pytest.mark.parametrize("fmt", ["b4_32", "b4_256", "b6_256"])
@pytest.mark.parametrize("M", [1, 5, 16, 33])
def test_qgemm_exact_integers(fmt, M):
    rng = np.random.default_rng(100 + M)
    rows, cols = 256, 512          # 256 rows: M > 32 runs the wide-M kernel
    raw = _int_case(fmt, rows, cols, rng)
    W = decode(fmt, raw, rows, cols)
    x = rng.integers(-3, 4, size=(M, cols)).astype(np.float64)
    want = x @ W.T
    assert np.abs(want).max() < 2 ** 24
    qw = tva.QWeight(fmt, torch.from_numpy(raw).to(DEV), rows, cols)
    got = qw.gemm(torch.from_numpy(x).float().to(DEV)).cpu().numpy()
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("fmt,rows,cols", [("b4_32", 96, 512), ("b4_256", 160, 1024),
                                           ("b6_256", 96, 768), ("b4_256", 256, 5120),
                                           ("b6_256", 64, 3584)])
def test_qgemm_random_parity_and_row_invariance(fmt, rows, cols):
    g = torch.Generator(device=DEV)
    g.manual_seed(rows * 7 + cols)
    w = torch.randn((rows, cols), generator=g, device=DEV) * 0.02
    raw = quantize(fmt, w)
    W = decode(fmt, raw.cpu().numpy(), rows, cols)
    qw = tva.QWeight(fmt, raw, rows, cols)
    x = torch.randn((40, cols), generator=g, device=DEV) * 1.5
    y40 = qw.gemm(x).cpu().numpy()
    xd = x.double().cpu().numpy()
    ref = xd @ W.T
    bound = 1e-5 * (np.abs(xd) @ np.abs(W).T) + 1e-7
    assert np.all(np.abs(y40 - ref) <= bound), float(np.max(np.abs(y40 - ref) / bound))
    # M <= 8 (and the 8-row last tile of M = 24) run the packed-row kernel,
    # whose rows must equal those of the unpacked launches bit for bit
    for M in (1, 3, 8, 9, 16, 17, 24):
        yM = qw.gemm(x[:M]).cpu().numpy()
        np.testing.assert_array_equal(yM, y40[:M])
    # per-row scale argument
    sc = torch.rand(40, generator=g, device=DEV) + 0.5
    ys = qw.gemm(x, sc).cpu().numpy()
    np.testing.assert_array_equal(ys, (torch.from_numpy(y40).to(DEV) * sc[:, None]).cpu().numpy())


@pytest.mark.parametrize("rows,cols", [(152064, 5120), (248320, 5120)])
def test_qgemm_full_lm_head_sampled(rows, cols):
    g = torch.Generator(device=DEV)
    g.manual_seed(rows)
    raw = torch.empty((rows, cols // 256 * 210), dtype=torch.uint8, device=DEV)
    for r0 in range(0, rows, 16384):
        r1 = min(rows, r0 + 16384)
        raw[r0:r1] = quantize("b6_256", torch.randn((r1 - r0, cols), generator=g,
                                                    device=DEV) * 0.02)
    qw = tva.QWeight("b6_256", raw, rows, cols)
    x = torch.randn((9, cols), generator=g, device=DEV)
    y = qw.gemm(x).cpu().numpy()
    pick = np.unique(np.concatenate([np.arange(0, 64), np.arange(rows - 64, rows),
                                     np.random.default_rng(0).integers(0, rows, 512)]))
    Wp = decode("b6_256", raw[torch.from_numpy(pick).to(DEV)].cpu().numpy(), len(pick), cols)
    xd = x.double().cpu().numpy()
    ref = xd @ Wp.T
    bound = 1e-5 * (np.abs(xd) @ np.abs(Wp).T) + 1e-7
    assert np.all(np.abs(y[:, pick] - ref) <= bound)


@pytest.mark.parametrize("fmt", ["b4_32", "b4_256", "b6_256"])
def test_qgemm_wide_rows_match_small_kernel(fmt):
    """25600 x 512 (100 column sets of 256, two K splits of one super-block):
    M = 40 runs 2 M-tiles per workgroup, M = 70 and 200 run 3 with a ragged
    last group; every row equals the small kernel's bits (M <= 16) and the
    fp64 product within the accumulation bound."""
    rows, cols = 25600, 512
    g = torch.Generator(device=DEV)
    g.manual_seed(4242)
    w = torch.randn((rows, cols), generator=g, device=DEV) * 0.02
    raw = quantize(fmt, w)
    W = decode(fmt, raw.cpu().numpy(), rows, cols)
    qw = tva.QWeight(fmt, raw, rows, cols)
    x = torch.randn((200, cols), generator=g, device=DEV) * 1.5
    y200 = qw.gemm(x).cpu().numpy()
    xd = x.double().cpu().numpy()
    ref = xd @ W.T
    bound = 1e-5 * (np.abs(xd) @ np.abs(W).T) + 1e-7
    assert np.all(np.abs(y200 - ref) <= bound), float(np.max(np.abs(y200 - ref) / bound))
    for M in (16, 40, 70):
        np.testing.assert_array_equal(qw.gemm(x[:M]).cpu().numpy(), y200[:M])
    y_small = np.concatenate([qw.gemm(x[m:m + 16]).cpu().numpy() for m in range(0, 200, 16)])
    np.testing.assert_array_equal(y_small, y200)


@pytest.mark.parametrize("fmt", ["b4_32", "b4_256", "b6_256"])
def test_qgemm_few_column_sets_run_small_kernel_per_tile_pair(fmt):
    """1280 x 512 (20 column sets): up to 200 rows the wide kernel would
    leave most CUs idle, so the small kernel runs once per pair of M-tiles;
    every row still equals its 16-row computation bit for bit and the fp64
    product within the accumulation bound."""
    rows, cols = 1280, 512
    g = torch.Generator(device=DEV)
    g.manual_seed(99)
    w = torch.randn((rows, cols), generator=g, device=DEV) * 0.02
    raw = quantize(fmt, w)
    W = decode(fmt, raw.cpu().numpy(), rows, cols)
    qw = tva.QWeight(fmt, raw, rows, cols)
    x = torch.randn((200, cols), generator=g, device=DEV) * 1.5
    ref = x.double().cpu().numpy() @ W.T
    bound = 1e-5 * (np.abs(x.double().cpu().numpy()) @ np.abs(W).T) + 1e-7
    y_small = np.concatenate([qw.gemm(x[m:m + 16]).cpu().numpy() for m in range(0, 200, 16)])
    for M in (40, 70, 200):
        y = qw.gemm(x[:M]).cpu().numpy()
        np.testing.assert_array_equal(y, y_small[:M])
        assert np.all(np.abs(y - ref[:M]) <= bound[:M])
