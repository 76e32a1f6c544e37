"""Counter-based uniforms for the stochastic verify decision.

The random numbers the sampler draws are pre-generated here and handed to both
the oracle and the GPU library as an input array, so neither side implements a
generator.  Each uniform is keyed by (seed, sequence, absolute position, lane):

* lane 0 at position len+r+1 decides the acceptance test of draft row r;
* lane 1 at position len+1 is the residual / bonus draw of the round;
* lane 2 at position P is the target sampler's draw of the token at P
  (exact-match sampled verify, and plain one-token-at-a-time sampling).

Because the key is the absolute position, the sampler's stream state is the
committed length: it moves by exactly the number of emitted tokens, and an
untested rejected suffix consumes nothing (its positions are re-keyed by the
next round, which the drafter never saw).

Mixing function: the SplitMix64 output function (Steele, Lea and Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014), applied as a
keyed hash chain.  Uniforms take the top 53 bits: u = (z >> 11) * 2**-53, so
u lies in [0, 1).
"""

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB


def splitmix64_stream(state: int, n: int):
    """Plain sequential SplitMix64: returns n outputs starting from `state`."""
    out = []
    for _ in range(n):
        state = (state + GAMMA) & MASK64
        z = state
        z = ((z ^ (z >> 30)) * _M1) & MASK64
        z = ((z ^ (z >> 27)) * _M2) & MASK64
        out.append(z ^ (z >> 31))
    return out


def fmix64(x: np.ndarray) -> np.ndarray:
    """SplitMix64 output function on a uint64 array (wrapping arithmetic)."""
    x = np.asarray(x, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = x ^ (x >> np.uint64(30))
        z = z * np.uint64(_M1)
        z = z ^ (z >> np.uint64(27))
        z = z * np.uint64(_M2)
        z = z ^ (z >> np.uint64(31))
    return z


def keyed_u64(seed, seq, pos, lane) -> np.ndarray:
    """Hash chain over the four key fields (broadcasting uint64 arrays)."""
    g = np.uint64(GAMMA)
    seed = np.asarray(seed, dtype=np.uint64)
    with np.errstate(over="ignore"):
        h = fmix64(seed + g)
        h = fmix64((h ^ np.asarray(seq, dtype=np.uint64)) + g * np.uint64(2))
        h = fmix64((h ^ np.asarray(pos, dtype=np.uint64)) + g * np.uint64(3))
        h = fmix64((h ^ np.asarray(lane, dtype=np.uint64)) + g * np.uint64(4))
    return h


def uniform(seed, seq, pos, lane) -> np.ndarray:
    z = keyed_u64(seed, seq, pos, lane)
    return (z >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def round_uniforms(seed: int, lens, nt: int) -> np.ndarray:
    """fp64 [n_seq][nt]: [:, r] (r < nt-1) acceptance draw of draft row r,
    [:, nt-1] the residual / bonus draw."""
    lens = np.asarray(lens, dtype=np.int64)
    s = np.arange(len(lens), dtype=np.uint64)[:, None]
    out = np.empty((len(lens), nt), dtype=np.float64)
    if nt > 1:
        r = np.arange(nt - 1, dtype=np.int64)[None, :]
        pos = (lens[:, None] + r + 1).astype(np.uint64)
        out[:, : nt - 1] = uniform(seed, s, pos, 0)
    out[:, nt - 1] = uniform(seed, s[:, 0], (lens + 1).astype(np.uint64), 1)
    return out


def sample_uniforms(seed: int, lens, nt: int) -> np.ndarray:
    """fp64 [n_seq][nt]: [:, r] the target sampler's draw for row r, i.e. for
    the token at absolute position len + r + 1 (lane 2)."""
    lens = np.asarray(lens, dtype=np.int64)
    s = np.arange(len(lens), dtype=np.uint64)[:, None]
    pos = (lens[:, None] + np.arange(nt, dtype=np.int64)[None, :] + 1).astype(np.uint64)
    return uniform(seed, s, pos, 2)
