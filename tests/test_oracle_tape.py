"""Pins for the oracle tape: the dual-number worked example of [AD] section 2,
the fan-out identity of [AE] "梯度累加（扇出求和）" (y = x*x + x*x gives
dL/dx = 4x), finite differences through the composed attention of
[AE] "Attention 用组合", and through a small pre-norm transformer block."""
import os

import numpy as np

from oracle import fd
from oracle.tape import Tape
from oracle_block import block_loss

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_dual_worked_example():
    row = [l.split() for l in open(os.path.join(GOLDEN, "dual_worked_example.txt")) if l.strip() and l[0] != "#"][0]
    x0, val, der = map(float, row)
    t = Tape()
    x = t.leaf([[x0]])
    f = t.add(t.mul(x, x), t.scale(x, 3.0))
    t.backward(f)
    assert t.value(f)[0, 0] == val and t.grad(x)[0, 0] == der


def test_fanout_four_x_exact():
    x0 = np.random.default_rng(3).standard_normal((8, 64))
    t = Tape()
    x = t.leaf(x0)
    y = t.add(t.mul(x, x), t.mul(x, x))
    t.backward(t.sum(y))
    np.testing.assert_array_equal(t.grad(x), 4.0 * x0)
    # with an upstream weight W: dL/dx = 4 * (W*x), exactly
    W = np.random.default_rng(4).standard_normal((8, 64))
    t2 = Tape()
    x = t2.leaf(x0)
    w = t2.leaf(W)
    y = t2.add(t2.mul(x, x), t2.mul(x, x))
    t2.backward(t2.sum(t2.mul(w, y)))
    np.testing.assert_array_equal(t2.grad(x), 4.0 * (W * x0))


def test_repeated_backward_accumulates_and_zero_grad():
    t = Tape()
    x = t.leaf([[1.5, -2.0]])
    L = t.sum(t.scale(x, 3.0))
    t.backward(L)
    t.backward(L)
    np.testing.assert_array_equal(t.grad(x), [[6.0, 6.0]])
    t.zero_grad()
    assert t.grad(x) is None


def test_dropout_p0_records_nothing():
    t = Tape()
    x = t.leaf(np.ones((2, 3)))
    assert t.dropout(x, 0.0, 7) == x


def _attention(t, q, k, v, S, Dh):
    scores = t.matmul(q, k, 1.0, False, True)
    probs = t.softmax(t.scale(scores, 1.0 / np.sqrt(Dh)), 1.0, True, S)
    return t.matmul(probs, v)


def test_composed_attention_fd():
    S, Dh = 5, 4
    g = np.random.default_rng(5)
    Q, K, V, W = (g.standard_normal((S, Dh)) for _ in range(4))

    def loss(q0, k0, v0):
        t = Tape()
        q, k, v = t.leaf(q0), t.leaf(k0), t.leaf(v0)
        out = _attention(t, q, k, v, S, Dh)
        return t, (q, k, v), out, t.sum(t.mul(t.leaf(W), out))

    t, (q, k, v), out, L = loss(Q, K, V)
    t.backward(L)
    for i, ref in enumerate([Q, K, V]):
        def f(a, i=i):
            args = [Q, K, V]
            args[i] = a
            tt, _, _, LL = loss(*args)
            return float(tt.value(LL)[0])
        num = fd.numeric_grad(f, ref)
        np.testing.assert_allclose(t.grad([q, k, v][i]), num, rtol=1e-6, atol=1e-8)
    # and the forward equals the explicit formula with a lower-triangular mask
    s = Q @ K.T / np.sqrt(Dh)
    s = np.where(np.tril(np.ones((S, S))) == 1, s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(t.value(out), p @ V, rtol=1e-13)


def test_block_fd_on_sampled_entries():
    B, S, H, Dh, V, hidden = 2, 4, 2, 4, 11, 6
    D = H * Dh
    g = np.random.default_rng(6)
    params = {k: 0.3 * g.standard_normal(s) for k, s in
              dict(wq=(D, D), wk=(D, D), wv=(D, D), wo=(D, D), wg=(D, hidden), wu=(D, hidden),
                   wd=(hidden, D), wout=(D, V)).items()}
    for k in ("g1", "g2", "g3"):
        params[k] = 1.0 + 0.1 * g.standard_normal(D)
    x0 = g.standard_normal((B * S, D))
    targets = g.integers(0, V, size=B * S)
    for p_drop in (0.0, 0.2):
        t, P, x, L = block_loss(params, x0, targets, B, S, H, Dh, p_drop, 11)
        t.backward(L)
        for name in ("wq", "wk", "wo", "wd", "g1", "wout"):
            for idx in [(0,) * params[name].ndim, tuple(s - 1 for s in params[name].shape)]:
                def f(eps):
                    pp = {k: v.copy() for k, v in params.items()}
                    pp[name][idx] += eps
                    tt, _, _, LL = block_loss(pp, x0, targets, B, S, H, Dh, p_drop, 11)
                    return float(tt.value(LL)[0])
                num = (f(1e-6) - f(-1e-6)) / 2e-6
                assert abs(t.grad(P[name])[idx] - num) <= 1e-6 * max(1.0, abs(num)), (name, idx)
        # input gradient too
        idx = (3, 5)
        def fx(eps):
            xx = x0.copy()
            xx[idx] += eps
            tt, _, _, LL = block_loss(params, xx, targets, B, S, H, Dh, p_drop, 11)
            return float(tt.value(LL)[0])
        num = (fx(1e-6) - fx(-1e-6)) / 2e-6
        assert abs(t.grad(x)[idx] - num) <= 1e-6 * max(1.0, abs(num))
