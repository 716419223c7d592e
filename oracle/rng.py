"""Counter-based dropout -- [DO] sections "RNG：counter-based" and
"dropout 节点的 backward", and the fp32 decision rule of
"与既有特性的组合" (bf16 only loads and stores the activation).

What the page fixes: each element draws its keep/drop decision from a pure
function of the 64-bit seed and the element's own index (no generator state
is carried between elements), so the same (seed, index) pair always gives
the same decision and a re-run reproduces the mask.  Here the index is the
logical row-major position r*cols + c; it is spread over 64 bits by a
multiply with the golden-ratio constant and mixed into the seed with an
exclusive or; the hash of that key supplies 24 uniform bits, read as a
fraction in [0, 1) exactly representable in f32; an element is kept when
that fraction is at least p (p rounded to f32), and a kept element is
scaled by the f32 value of 1/(1-p) (inverted dropout).  The backward uses
the same mask and scale on the incoming gradient.  ``dropout_mask`` and the
functions below carry the exact constants and shifts.

Reading for "splitmix64" (the page only says "a few rounds of xorshift and
multiply"): the output of Steele, Lea and Flood's SplitMix64 generator
(OOPSLA 2014, "Fast splittable pseudorandom number generators"; the variant
with Stafford's "Mix13" finalizer used by Vigna's public-domain splitmix64.c)
whose state is ``key``: advance the state by the golden gamma, then
z ^= z>>30; z *= 0xBF58476D1CE4E5B9; z ^= z>>27; z *= 0x94D049BB133111EB;
z ^= z>>31.  All arithmetic here is exact unsigned 64-bit integer work plus
exact f32 comparisons, so the mask is reproducible bit for bit.
"""
from __future__ import annotations

import numpy as np

GOLDEN_GAMMA = 0x9E3779B97F4A7C15
MIX_1 = 0xBF58476D1CE4E5B9
MIX_2 = 0x94D049BB133111EB
_M64 = (1 << 64) - 1


def splitmix64(state: int) -> int:
    """First output of a SplitMix64 generator whose state is ``state``
    (pure Python integers, reduced mod 2^64)."""
    z = (state + GOLDEN_GAMMA) & _M64
    z = ((z ^ (z >> 30)) * MIX_1) & _M64
    z = ((z ^ (z >> 27)) * MIX_2) & _M64
    return z ^ (z >> 31)


def splitmix64_stream(state: int, n: int):
    """n successive outputs of the generator (state advancing by the gamma
    each step), for comparison with published output sequences."""
    out = []
    for _ in range(n):
        out.append(splitmix64(state))
        state = (state + GOLDEN_GAMMA) & _M64
    return out


def _splitmix64_np(key: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = key + np.uint64(GOLDEN_GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(MIX_1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(MIX_2)
        return z ^ (z >> np.uint64(31))


def uniform24(seed: int, index: np.ndarray) -> np.ndarray:
    """u in [0,1) for each element index, as exact float64 (it is a 24-bit
    fraction, so equal to its f32 value)."""
    idx = np.asarray(index, dtype=np.uint64)
    with np.errstate(over="ignore"):
        key = np.uint64(seed & _M64) ^ (idx * np.uint64(GOLDEN_GAMMA))
    h = _splitmix64_np(key)
    return (h >> np.uint64(40)).astype(np.float64) * (2.0 ** -24)


def keep_scale(p: float) -> float:
    """s = 1/(1-p) evaluated in IEEE f32 (returned as the exact f64 value)."""
    one = np.float32(1.0)
    return float(one / (one - np.float32(p)))


def dropout_mask(shape, p: float, seed: int, index_offset: int = 0) -> np.ndarray:
    """u8 mask (1 = keep) for a row-major tensor of ``shape``; element i of
    the tensor uses counter index_offset + i."""
    n = int(np.prod(shape))
    idx = np.arange(n, dtype=np.uint64) + np.uint64(index_offset)
    keep = uniform24(seed, idx) >= float(np.float32(p))
    return keep.reshape(shape).astype(np.uint8)


def dropout(x, p: float, seed: int, index_offset: int = 0):
    """Returns (y, mask).  y = x*s where kept, +0 where dropped.  Element i
    of x uses counter index_offset + i (a block of rows of a larger tensor
    passes the flat index of its first element)."""
    X = np.asarray(x, dtype=np.float64)
    mask = dropout_mask(X.shape, p, seed, index_offset)
    s = keep_scale(p)
    return np.where(mask == 1, X * s, 0.0), mask


def dropout_bwd(d, mask, p: float):
    D = np.asarray(d, dtype=np.float64)
    return np.where(np.asarray(mask) == 1, D * keep_scale(p), 0.0)


def site_seed(base_seed: int, layer: int, site: int) -> int:
    """[DO] "每个 dropout 站点的确定性 seed": a block's seed is base XOR
    layer index, and each site XORs its own constant (attention 0xA77, FFN
    0xF70 -- the page's FFN constant is garbled; 0xF70 is the reading)."""
    return (base_seed ^ layer ^ site) & _M64


SITE_ATTN = 0xA77
SITE_FFN = 0xF70
