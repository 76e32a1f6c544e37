"""The test-side byte writers produce blocks that the (pinned) oracle decoder
reads back as the intended integer weights."""

import numpy as np

from oracle.formats import decode
from tests.gpu_util import pack_b4_32, pack_b4_256, pack_b6_256


def test_pack_b4_32_roundtrip():
    rng = np.random.default_rng(0)
    q = rng.integers(0, 16, size=(3, 4, 32))
    raw = pack_b4_32(np.ones((3, 4)), q)
    np.testing.assert_array_equal(decode("b4_32", raw, 3, 128), (q - 8).reshape(3, 128))


def test_pack_b4_256_roundtrip():
    rng = np.random.default_rng(1)
    sc, m = rng.integers(0, 64, size=(2, 3, 8)), rng.integers(0, 64, size=(2, 3, 8))
    q = rng.integers(0, 16, size=(2, 3, 256))
    raw = pack_b4_256(np.ones((2, 3)), np.ones((2, 3)), sc, m, q)
    j = np.arange(256) // 32
    want = sc[..., j] * q - m[..., j]
    np.testing.assert_array_equal(decode("b4_256", raw, 2, 768), want.reshape(2, 768))


def test_pack_b6_256_roundtrip():
    rng = np.random.default_rng(2)
    sc = rng.integers(-128, 128, size=(2, 2, 16))
    q = rng.integers(0, 64, size=(2, 2, 256))
    raw = pack_b6_256(np.full((2, 2), 0.5), sc, q)
    j = np.arange(256) // 16
    want = 0.5 * sc[..., j] * (q - 32)
    np.testing.assert_array_equal(decode("b6_256", raw, 2, 512), want.reshape(2, 512))
