"""Pins for the oracle's counter-based dropout ([DO] "RNG：counter-based",
"dropout 节点的 backward", "验证方法"): published SplitMix64 outputs, p = 0
identity, keep fraction, expectation preservation, the linear-map gradient
under a fixed mask, and seed/site behaviour."""
import math
import os

import numpy as np

from oracle import fd, rng

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_splitmix64_published_sequence():
    vals = [int(l) for l in open(os.path.join(GOLDEN, "splitmix64_1234567.txt")) if l.strip() and l[0] != "#"]
    assert rng.splitmix64_stream(1234567, len(vals)) == vals


def test_vectorised_hash_equals_scalar_hash():
    seed = 42
    idx = np.array([0, 1, 2, 511, 2 ** 31 + 5, 2 ** 40 + 3], dtype=np.uint64)
    u = rng.uniform24(seed, idx)
    for i, ui in zip(idx.tolist(), u):
        key = seed ^ ((i * rng.GOLDEN_GAMMA) & ((1 << 64) - 1))
        assert ui == (rng.splitmix64(key) >> 40) / 2 ** 24


def test_p_zero_is_bit_identity():
    x = np.random.default_rng(0).standard_normal((8, 64)).astype(np.float32)
    y, mask = rng.dropout(x, 0.0, 42)
    assert np.all(mask == 1)
    np.testing.assert_array_equal(y.astype(np.float32), x)


def test_keep_fraction_and_uniformity():
    p = 0.1
    n = 1 << 22
    mask = rng.dropout_mask((n,), p, 42)
    keep_prob = 1.0 - math.ceil(float(np.float32(p)) * 2 ** 24) / 2 ** 24   # u >= p on a 2^-24 grid
    sigma = math.sqrt(keep_prob * (1 - keep_prob) / n)
    assert abs(mask.mean() - keep_prob) < 5 * sigma
    # chi-square of u over 64 equal buckets
    u = rng.uniform24(7, np.arange(n, dtype=np.uint64))
    counts = np.bincount((u * 64).astype(np.int64), minlength=64)
    chi2 = float(np.sum((counts - n / 64) ** 2 / (n / 64)))
    assert chi2 < 130.0          # 63 dof: P(chi2 > 130) ~ 1e-6


def test_expectation_preserved():
    x = np.linspace(-2.0, 2.0, 16)
    acc = np.zeros_like(x)
    trials = 4000
    for s in range(trials):
        acc += rng.dropout(x, 0.25, 1000 + s)[0]
    # per element: Var(y) = x^2 * p/(1-p); mean of `trials` draws within 5 sigma
    sig = np.abs(x) * math.sqrt(0.25 / 0.75) / math.sqrt(trials)
    assert np.all(np.abs(acc / trials - x) <= 5 * sig + 1e-12)


def test_mask_depends_only_on_seed_and_index_and_fd():
    x = np.random.default_rng(1).standard_normal((4, 6))
    W = np.random.default_rng(2).standard_normal((4, 6))
    y1, m1 = rng.dropout(x, 0.3, 99)
    y2, m2 = rng.dropout(x * 3.0 + 1.0, 0.3, 99)
    np.testing.assert_array_equal(m1, m2)
    dx = rng.dropout_bwd(W, m1, 0.3)
    num = fd.numeric_grad(lambda a: float(np.sum(W * rng.dropout(a, 0.3, 99)[0])), x)
    np.testing.assert_allclose(dx, num, rtol=1e-6, atol=1e-8)
    s = rng.keep_scale(0.3)
    np.testing.assert_array_equal(y1, np.where(m1 == 1, x * s, 0.0))


def test_scale_is_f32_reciprocal_and_seeds_differ():
    assert rng.keep_scale(0.1) == float(np.float32(1.1111112))
    assert rng.keep_scale(0.0) == 1.0
    a = rng.dropout_mask((4096,), 0.1, rng.site_seed(42, 0, rng.SITE_ATTN))
    b = rng.dropout_mask((4096,), 0.1, rng.site_seed(42, 0, rng.SITE_FFN))
    c = rng.dropout_mask((4096,), 0.1, rng.site_seed(42, 1, rng.SITE_ATTN))
    assert (a != b).sum() > 100 and (a != c).sum() > 100
    assert rng.site_seed(42, 0, rng.SITE_ATTN) == 42 ^ 0xA77
    assert rng.site_seed(42, 3, rng.SITE_FFN) == 42 ^ 3 ^ 0xF70


def test_index_offset_shards_reproduce_whole_mask():
    whole = rng.dropout_mask((6, 10), 0.2, 5)
    top = rng.dropout_mask((2, 10), 0.2, 5)
    bottom = rng.dropout_mask((4, 10), 0.2, 5, index_offset=20)
    np.testing.assert_array_equal(np.vstack([top, bottom]), whole)
