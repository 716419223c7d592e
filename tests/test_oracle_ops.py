"""Pins for the oracle's ops: each is checked against something other than its
own formula -- f64 central differences for every backward, closed forms,
invariants, hand-worked values, brute-force loops and library/table values.
"""
import math
import os

import numpy as np
import pytest

from oracle import fd, ops
from oracle.numerics import round_bf16, bf16_to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def rnd(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def check_fd(f_out, bwd_grads, inputs, W, tol=1e-6):
    """For each input k, compare bwd_grads[k] with the central difference of
    L = sum(W * f_out(*inputs)) w.r.t. inputs[k]."""
    L = fd.weighted_loss(W)
    for k, x in enumerate(inputs):
        def f(xk, k=k):
            args = list(inputs)
            args[k] = xk
            return L(f_out(*args))
        num = fd.numeric_grad(f, x)
        ana = np.asarray(bwd_grads[k], dtype=np.float64)
        scale = max(1.0, float(np.max(np.abs(num))))
        assert np.max(np.abs(ana - num)) <= tol * scale, (k, np.max(np.abs(ana - num)))


# ------------------------------------------------------------------ matmul
@pytest.mark.parametrize("ta,tb", [(False, False), (False, True), (True, False), (True, True)])
def test_matmul_brute_force_and_fd(ta, tb):
    M, K, N = 3, 4, 5
    A = rnd(K, M) if ta else rnd(M, K)
    B = rnd(N, K) if tb else rnd(K, N)
    alpha = 0.75
    C = ops.matmul(A, B, alpha, ta, tb)
    for i in range(M):
        for j in range(N):
            s = 0.0
            for k in range(K):
                a = A[k][i] if ta else A[i][k]
                b = B[j][k] if tb else B[k][j]
                s += a * b
            assert abs(C[i, j] - alpha * s) < 1e-12
    W = rnd(M, N)
    dA, dB = ops.matmul_bwd(W, A, B, alpha, ta, tb)
    check_fd(lambda a, b: ops.matmul(a, b, alpha, ta, tb), [dA, dB], [A, B], W)


def test_matmul_batched_matches_per_batch_loop():
    A, B = rnd(2, 3, 4, 5), rnd(2, 3, 5, 6)
    C = ops.matmul(A, B, 2.0, False, False)
    for i in range(2):
        for j in range(3):
            ref = [[2.0 * sum(A[i, j, r, k] * B[i, j, k, c] for k in range(5)) for c in range(6)]
                   for r in range(4)]
            np.testing.assert_allclose(C[i, j], ref, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------- add / mul / scale
def test_add_mul_scale_fd():
    a, b, W = rnd(3, 4), rnd(3, 4), rnd(3, 4)
    check_fd(ops.add, ops.add_bwd(W), [a, b], W)
    check_fd(ops.mul, ops.mul_bwd(W, a, b), [a, b], W)
    check_fd(lambda x: ops.scale(x, -1.7), [ops.scale_bwd(W, -1.7)], [a], W)
    assert ops.mul([[2.0]], [[3.0]])[0, 0] == 6.0
    assert ops.add([[2.0]], [[3.0]])[0, 0] == 5.0


def test_add_bias_fd_and_loop():
    x, bias, W = rnd(5, 3), rnd(3), rnd(5, 3)
    dx, db = ops.add_bias_bwd(W)
    check_fd(ops.add_bias, [dx, db], [x, bias], W)
    for c in range(3):
        assert abs(db[c] - sum(W[r][c] for r in range(5))) < 1e-12
        for r in range(5):
            assert ops.add_bias(x, bias)[r, c] == x[r, c] + bias[c]


# ------------------------------------------------------------- rms_norm
def test_rms_norm_worked_value():
    y, ir = ops.rms_norm([[3.0, 4.0]], [1.0, 2.0], 0.0)
    # mean(x^2) = 12.5
    assert abs(ir[0] - 1.0 / math.sqrt(12.5)) < 1e-15
    np.testing.assert_allclose(y[0], [3.0 / math.sqrt(12.5), 8.0 / math.sqrt(12.5)], rtol=1e-15)


@pytest.mark.parametrize("eps", [1e-5, 0.3])
def test_rms_norm_fd_and_invariants(eps):
    x, gamma, W = rnd(4, 6), 1.0 + 0.1 * rnd(6), rnd(4, 6)
    y, ir = ops.rms_norm(x, gamma, eps)
    dx, dg = ops.rms_norm_bwd(W, x, gamma, ir)
    check_fd(lambda a, g: ops.rms_norm(a, g, eps)[0], [dx, dg], [x, gamma], W)
    ms = np.mean(x * x, axis=1)
    rms_of_normed = np.sqrt(np.mean((y / gamma) ** 2, axis=1))
    np.testing.assert_allclose(rms_of_normed, np.sqrt(ms / (ms + eps)), rtol=1e-13)


def test_rms_norm_scale_invariance_gives_orthogonal_grad():
    # eps = 0: y(c*x) = y(x)  =>  sum_c x*dx = 0 on every row
    x, gamma, W = rnd(5, 7), rnd(7), rnd(5, 7)
    _, ir = ops.rms_norm(x, gamma, 0.0)
    dx, _ = ops.rms_norm_bwd(W, x, gamma, ir)
    assert np.max(np.abs(np.sum(x * dx, axis=1))) < 1e-12


# ----------------------------------------------------------- layer_norm
def test_layer_norm_worked_value():
    y, mu, rstd = ops.layer_norm([[1.0, 2.0, 3.0, 4.0]], [1.0] * 4, [0.0] * 4, 0.0)
    assert mu[0] == 2.5 and abs(rstd[0] - 1.0 / math.sqrt(1.25)) < 1e-15
    np.testing.assert_allclose(y[0], np.array([-1.5, -0.5, 0.5, 1.5]) / math.sqrt(1.25), rtol=1e-14)


@pytest.mark.parametrize("eps", [1e-5, 0.5])
def test_layer_norm_fd_and_invariants(eps):
    x, g, b, W = rnd(4, 6), 1 + 0.1 * rnd(6), 0.1 * rnd(6), rnd(4, 6)
    y, mu, rs = ops.layer_norm(x, g, b, eps)
    dx, dg, db = ops.layer_norm_bwd(W, x, g, mu, rs)
    check_fd(lambda a, gg, bb: ops.layer_norm(a, gg, bb, eps)[0], [dx, dg, db], [x, g, b], W)
    xhat = (y - b) / g
    assert np.max(np.abs(np.mean(xhat, axis=1))) < 1e-13
    var = np.var(x, axis=1)
    np.testing.assert_allclose(np.mean(xhat ** 2, axis=1), var / (var + eps), rtol=1e-12)
    # shift invariance: the gradient rows sum to zero, even with eps
    assert np.max(np.abs(np.sum(dx, axis=1))) < 1e-12
    np.testing.assert_allclose(db, W.sum(axis=0), rtol=1e-14)


# --------------------------------------------------------------- softmax
def test_softmax_worked_values():
    y = ops.softmax([[0.0, math.log(2.0), math.log(3.0)]])
    np.testing.assert_allclose(y[0], [1 / 6, 2 / 6, 3 / 6], rtol=1e-14)
    y = ops.softmax([[0.0, math.log(4.0)]], alpha=0.5)       # softmax([0, ln 2])
    np.testing.assert_allclose(y[0], [1 / 3, 2 / 3], rtol=1e-14)
    np.testing.assert_allclose(ops.softmax(np.full((2, 5), 3.3)), np.full((2, 5), 0.2), rtol=1e-15)


@pytest.mark.parametrize("alpha,causal", [(1.0, False), (0.125, False), (1.0, True), (0.5, True)])
def test_softmax_fd_and_invariants(alpha, causal):
    R, C, S = 6, 4, 4
    x, W = rnd(R, C, scale=2.0), rnd(R, C)
    y = ops.softmax(x, alpha, causal, S)
    np.testing.assert_allclose(y.sum(axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(ops.softmax(x + 7.0, alpha, causal, S), y, rtol=1e-12)
    dx = ops.softmax_bwd(W, y, alpha)
    assert np.max(np.abs(dx.sum(axis=1))) < 1e-13
    check_fd(lambda a: ops.softmax(a, alpha, causal, S), [dx], [x], W)
    if causal:
        for r in range(R):
            q = r % S
            assert np.all(y[r, q + 1:] == 0.0) and np.all(dx[r, q + 1:] == 0.0)
            np.testing.assert_allclose(y[r, :q + 1], ops.softmax(x[r:r + 1, :q + 1], alpha)[0], rtol=1e-14)
        np.testing.assert_array_equal(y[0], [1.0, 0.0, 0.0, 0.0])


# --------------------------------------------------------- cross_entropy
def test_cross_entropy_worked_value():
    L, lse, loss_row = ops.cross_entropy([[0.0, math.log(2.0), math.log(3.0)]], [2])
    assert abs(lse[0] - math.log(6.0)) < 1e-15
    assert abs(L - math.log(2.0)) < 1e-15          # -log(3/6)
    d = ops.cross_entropy_bwd(1.0, [[0.0, math.log(2.0), math.log(3.0)]], [2], lse)
    np.testing.assert_allclose(d[0], [1 / 6, 2 / 6, 3 / 6 - 1], rtol=1e-14)


@pytest.mark.parametrize("V", [64, 4096, 50257, 128256])
def test_cross_entropy_constant_logits_is_log_vocab(V):
    # every class equally likely: L = ln V (math.log as the library routine)
    L, _, _ = ops.cross_entropy(np.full((2, V), -1.25), [0, V - 1])
    assert abs(L - math.log(V)) < 1e-12


def test_cross_entropy_fd_and_invariants():
    R, V = 4, 7
    x, t = rnd(R, V, scale=2.0), np.array([0, 6, 3, 3])
    L, lse, loss_row = ops.cross_entropy(x, t)
    assert L >= 0 and np.all(loss_row >= 0)
    g = -0.6
    dx = ops.cross_entropy_bwd(g, x, t, lse)
    assert np.max(np.abs(dx.sum(axis=1))) < 1e-14
    num = fd.numeric_grad(lambda a: g * ops.cross_entropy(a, t)[0], x)
    assert np.max(np.abs(num - dx)) < 1e-8


def test_cross_entropy_bad_target_is_nan_row():
    x = rnd(3, 5)
    L, lse, loss_row = ops.cross_entropy(x, [1, 5, -1])
    assert math.isnan(L) and not math.isnan(loss_row[0]) and math.isnan(loss_row[1]) and math.isnan(loss_row[2])
    dx = ops.cross_entropy_bwd(1.0, x, [1, 5, -1], lse)
    assert np.all(np.isfinite(dx[0])) and np.all(np.isnan(dx[1])) and np.all(np.isnan(dx[2]))


# ------------------------------------------------------ silu / swiglu / gelu
def test_silu_gelu_values():
    assert ops.silu([0.0])[0] == 0.0 and ops.silu_bwd([1.0], [0.0])[0] == 0.5
    assert abs(ops.silu([1.0])[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert ops.gelu([0.0])[0] == 0.0 and ops.gelu_bwd([1.0], [0.0])[0] == 0.5
    rows = [l.split() for l in open(os.path.join(GOLDEN, "normal_cdf_table.txt")) if l.strip() and l[0] != "#"]
    for xs, phis in rows:
        xv, phi = float(xs), float(phis)
        assert abs(ops.normal_cdf([xv])[0] - phi) < 1e-14
        assert abs(ops.gelu([xv])[0] - xv * phi) < 1e-14
    from scipy.stats import norm
    xs = np.linspace(-6, 6, 101)
    np.testing.assert_allclose(ops.normal_cdf(xs), norm.cdf(xs), rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(ops.normal_pdf(xs), norm.pdf(xs), rtol=1e-13)


def test_gelu_tanh_form():
    """The tanh form is an approximation of x*Phi(x): it must stay within
    5e-4 of the exact GELU everywhere (its largest gap, near |x| = 2.7, is
    4.7e-4; a dropped cubic term gives 3.4e-2, a cubic coefficient off by
    ten percent about 3e-3), match its slope and curvature at 0 (which
    fixes the sqrt(2/pi) factor), and g(x) - g(-x) = x holds exactly for
    any odd inner function."""
    xs = np.linspace(-12.0, 12.0, 240001)
    assert np.max(np.abs(ops.gelu_tanh(xs) - ops.gelu(xs))) < 5e-4
    np.testing.assert_allclose(ops.gelu_tanh(xs) - ops.gelu_tanh(-xs), xs, rtol=0, atol=1e-14)
    assert ops.gelu_tanh([0.0])[0] == 0.0 and ops.gelu_tanh_bwd([1.0], [0.0])[0] == 0.5
    # second derivative at 0 equals the exact GELU's, 2 phi(0) = sqrt(2/pi)
    h = 1e-4
    curv = (ops.gelu_tanh_bwd([1.0], [h])[0] - ops.gelu_tanh_bwd([1.0], [-h])[0]) / (2 * h)
    assert abs(curv - math.sqrt(2.0 / math.pi)) < 1e-7
    # tails: x for large positive x, 0 for large negative x
    assert ops.gelu_tanh([30.0])[0] == 30.0 and abs(ops.gelu_tanh([-30.0])[0]) < 1e-300
    x, W = rnd(4, 7, scale=2.5), rnd(4, 7)
    check_fd(ops.gelu_tanh, [ops.gelu_tanh_bwd(W, x)], [x], W)


def test_silu_swiglu_gelu_fd():
    x, g, u, W = rnd(3, 5, scale=2.0), rnd(3, 5, scale=2.0), rnd(3, 5), rnd(3, 5)
    check_fd(ops.silu, [ops.silu_bwd(W, x)], [x], W)
    check_fd(ops.gelu, [ops.gelu_bwd(W, x)], [x], W)
    check_fd(ops.swiglu, list(ops.swiglu_bwd(W, g, u)), [g, u], W)
    np.testing.assert_allclose(ops.swiglu(g, np.ones_like(g)), ops.silu(g), rtol=1e-15)


# ------------------------------------------------------------------ rope
def test_rope_pairing_direction_and_angles():
    # head_dim 4, base 4: theta_{pos,0} = pos, theta_{pos,1} = pos/2
    x = np.zeros((3, 4)); x[:, 0] = 1.0
    y = ops.rope(x, 4, 4.0, 3)
    for pos in range(3):
        np.testing.assert_allclose(y[pos], [math.cos(pos), 0.0, math.sin(pos), 0.0], atol=1e-15)
    x = np.zeros((3, 4)); x[:, 1] = 1.0
    y = ops.rope(x, 4, 4.0, 3)
    for pos in range(3):
        np.testing.assert_allclose(y[pos], [0.0, math.cos(pos / 2), 0.0, math.sin(pos / 2)], atol=1e-15)
    # the page's backward formula on d = e_{i+h}: dx_i = sin, dx_{i+h} = cos
    d = np.zeros((3, 4)); d[:, 2] = 1.0
    dx = ops.rope_bwd(d, 4, 4.0, 3)
    for pos in range(3):
        np.testing.assert_allclose(dx[pos], [math.sin(pos), 0.0, math.cos(pos), 0.0], atol=1e-15)


def test_rope_is_complex_rotation_for_head_dim_2():
    R = 7
    x = rnd(R, 6)                          # three heads of width 2
    y = ops.rope(x, 2, 10000.0, R)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * np.arange(R))[:, None]
    np.testing.assert_allclose(y[:, 0::2], z.real, atol=1e-14)
    np.testing.assert_allclose(y[:, 1::2], z.imag, atol=1e-14)


def test_rope_orthogonal_identity_at_zero_and_fd():
    Dh, R, S = 8, 6, 4
    x, W = rnd(R, 2 * Dh), rnd(R, 2 * Dh)
    y = ops.rope(x, Dh, 10000.0, S)
    np.testing.assert_array_equal(y[0], x[0])                  # pos 0
    np.testing.assert_array_equal(y[S], x[S])                  # pos wraps to 0
    h = Dh // 2
    for hd in range(2):
        a = x[:, hd * Dh:hd * Dh + h] ** 2 + x[:, hd * Dh + h:(hd + 1) * Dh] ** 2
        b = y[:, hd * Dh:hd * Dh + h] ** 2 + y[:, hd * Dh + h:(hd + 1) * Dh] ** 2
        np.testing.assert_allclose(a, b, rtol=1e-13)
    np.testing.assert_allclose(ops.rope_bwd(y, Dh, 10000.0, S), x, atol=1e-14)
    # explicit positions select the same rotation as the row index would
    rows = np.array([5, 2, 3])
    np.testing.assert_array_equal(ops.rope(x[rows], Dh, 10000.0, S, positions=rows % S), y[rows])
    check_fd(lambda a: ops.rope(a, Dh, 10000.0, S), [ops.rope_bwd(W, Dh, 10000.0, S)], [x], W)


# ----------------------------------------------------------- accumulate
def test_grad_accumulate_and_bf16_rounding():
    a, b = rnd(3, 3), rnd(3, 3)
    np.testing.assert_array_equal(ops.grad_accumulate(a, b), a + b)
    # bf16 rounding: 1 + 2^-8 is a tie between 1 and 1+2^-7 -> even (1.0)
    np.testing.assert_array_equal(round_bf16([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9]),
                                  [1.0, 1.0 + 2 ** -6, 1.0])
    np.testing.assert_array_equal(bf16_to_f64(np.array([0x3F80, 0xC000], dtype=np.uint16)), [1.0, -2.0])


# ------------------------------------------------------- gradient buffers
def test_grad_norm_closed_forms():
    # 3-4-5 across two tensors; 100 ones in four tensors -> 10
    assert ops.grad_norm([np.array([[3.0]]), np.array([[4.0]])]) == 5.0
    assert ops.grad_norm([np.ones((5, 5)) for _ in range(4)]) == 10.0
    assert ops.grad_norm([]) == 0.0
    assert ops.grad_norm([np.zeros((0, 7)), np.array([[0.0, -2.0]])]) == 2.0


def test_grad_norm_against_library_norm_and_scaling():
    gs = [rnd(3, 5), rnd(1, 17, scale=3.0), rnd(40, 2)]
    flat = np.concatenate([g.ravel() for g in gs])
    n = ops.grad_norm(gs)
    assert abs(n - np.linalg.norm(flat)) <= 1e-13 * n
    # power-of-two scaling is exact
    assert ops.grad_norm([2.0 * g for g in gs]) == 2.0 * n


def test_clip_coefficient_rule():
    assert ops.clip_coefficient(5.0, 1.0) == 0.2
    assert ops.clip_coefficient(0.5, 1.0) == 1.0
    assert ops.clip_coefficient(1.0, 1.0) == 1.0      # not above the threshold
    assert ops.clip_coefficient(5.0, 0.0) == 1.0      # no threshold
    # after clipping, the global norm is the threshold
    gs = [rnd(4, 6, scale=5.0), rnd(2, 3, scale=5.0)]
    c = ops.clip_coefficient(ops.grad_norm(gs), 1.5)
    assert c < 1.0 and abs(ops.grad_norm([c * g for g in gs]) - 1.5) < 1e-12


def test_scale_grad_rounding():
    x = rnd(6, 9, scale=4.0).astype(np.float32).astype(np.float64)
    assert np.array_equal(ops.scale_grad(x, 1.0), x)
    assert np.array_equal(ops.scale_grad(x, 2.0), 2.0 * x)
    assert np.array_equal(ops.scale_grad(x, 0.0), 0.0 * x)
    # f32: the correctly rounded f32 product
    f = np.float32(0.1)
    assert np.array_equal(ops.scale_grad(x, f), (x.astype(np.float32) * f).astype(np.float64))
    # bf16 storage: values stay on the bf16 grid; a power of two keeps them exact
    from oracle.numerics import round_bf16
    xb = round_bf16(x)
    yb = ops.scale_grad(xb, 0.3, "bf16")
    assert np.array_equal(round_bf16(yb), yb)
    assert np.array_equal(ops.scale_grad(xb, 0.25, "bf16"), 0.25 * xb)


# ------------------------------------------------------------ embedding
def test_embed_is_a_one_hot_product():
    V, D, R = 7, 5, 23
    E = rnd(V, D)
    ids = RNG.integers(0, V, size=R)
    onehot = np.zeros((R, V))
    onehot[np.arange(R), ids] = 1.0
    np.testing.assert_array_equal(ops.embed(E, ids), onehot @ E)           # exact: one nonzero per row
    d = rnd(R, D)
    np.testing.assert_allclose(ops.embed_bwd(d, ids, V), onehot.T @ d, rtol=1e-14, atol=1e-14)
    # counts: with d = 1 every dE row holds the number of uses of its id
    cnt = ops.embed_bwd(np.ones((R, 1)), ids, V)[:, 0]
    np.testing.assert_array_equal(cnt, np.bincount(ids, minlength=V))
    check_fd(lambda e: ops.embed(e, ids), [ops.embed_bwd(d, ids, V)], [E], d)


def test_embed_out_of_range_ids():
    E = rnd(4, 3)
    y = ops.embed(E, [0, 4, -1, 3])
    assert np.all(np.isnan(y[1])) and np.all(np.isnan(y[2]))
    np.testing.assert_array_equal(y[[0, 3]], E[[0, 3]])
    dE = ops.embed_bwd(np.ones((4, 3)), [0, 4, -1, 0], 4)
    np.testing.assert_array_equal(dE, [[2, 2, 2], [0, 0, 0], [0, 0, 0], [0, 0, 0]])


# --------------------------------------------------------- fused attention
def _compose_attention(q, k, v, S, H, Dh, alpha):
    """The [AE] composition with the separately pinned ops, per (b, h)."""
    B = q.shape[0] // S
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            rs, cs = slice(b * S, (b + 1) * S), slice(h * Dh, (h + 1) * Dh)
            P = ops.softmax(ops.matmul(q[rs, cs], k[rs, cs], trans_b=True), alpha, True, S)
            out[rs, cs] = ops.matmul(P, v[rs, cs])
    return out


def test_attention_equals_the_composition_and_closed_forms():
    S, H, Dh, B = 7, 2, 4, 3
    q, k, v = rnd(B * S, H * Dh), rnd(B * S, H * Dh), rnd(B * S, H * Dh)
    o, lse = ops.attention(q, k, v, S, H, Dh, 0.5)
    np.testing.assert_allclose(o, _compose_attention(q, k, v, S, H, Dh, 0.5), rtol=1e-13, atol=1e-13)
    # the first token attends to itself only: out = v there
    for b in range(B):
        np.testing.assert_allclose(o[b * S], v[b * S], rtol=1e-14)
    # q = 0: uniform over the causal prefix, lse = log(s + 1)
    o0, l0 = ops.attention(np.zeros_like(q), k, v, S, H, Dh, 0.5)
    for b in range(B):
        for s in range(S):
            np.testing.assert_allclose(o0[b * S + s], v[b * S: b * S + s + 1].mean(axis=0), rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(l0[b * S + s], math.log(s + 1), rtol=1e-14)
    # lse by its definition on one (b, h, s)
    b, h, s = 1, 1, 5
    z = 0.5 * k[b * S: b * S + s + 1, h * Dh:(h + 1) * Dh] @ q[b * S + s, h * Dh:(h + 1) * Dh]
    assert abs(lse[b * S + s, h] - math.log(np.sum(np.exp(z)))) < 1e-13


def test_attention_bwd_fd():
    S, H, Dh, B = 5, 2, 3, 2
    q, k, v = rnd(B * S, H * Dh), rnd(B * S, H * Dh), rnd(B * S, H * Dh)
    W = rnd(B * S, H * Dh)
    f = lambda q_, k_, v_: ops.attention(q_, k_, v_, S, H, Dh, 0.7)[0]  # noqa: E731
    check_fd(f, list(ops.attention_bwd(W, q, k, v, S, H, Dh, 0.7)), [q, k, v], W)


def test_attention_bwd_from_the_stored_output():
    """rowsum(dP * P) = rowsum(dO * O): fed the exact output, the backward that
    reads the stored output equals the one that forms the row term from P;
    the row term does not enter dV."""
    S, H, Dh, B = 6, 2, 4, 2
    q, k, v, d = (rnd(B * S, H * Dh) for _ in range(4))
    for causal in (True, False):
        o, _ = ops.attention(q, k, v, S, H, Dh, 0.6, causal)
        ref = ops.attention_bwd(d, q, k, v, S, H, Dh, 0.6, causal)
        got = ops.attention_bwd(d, q, k, v, S, H, Dh, 0.6, causal, out=o)
        for a, b in zip(got, ref):
            np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
        moved = ops.attention_bwd(d, q, k, v, S, H, Dh, 0.6, causal, out=o + 0.01)
        np.testing.assert_array_equal(moved[2], ref[2])
        assert np.max(np.abs(moved[0] - ref[0])) > 1e-4


def test_attention_term_magnitudes():
    """Each magnitude bounds its sum (triangle inequality) and equals it when
    every term is nonnegative: v >= 0 for the output, dO >= 0 for dV."""
    S, H, Dh, B = 7, 2, 4, 2
    q, k, v, d = (rnd(B * S, H * Dh) for _ in range(4))
    o, _ = ops.attention(q, k, v, S, H, Dh, 0.5)
    dq, dk, dv = ops.attention_bwd(d, q, k, v, S, H, Dh, 0.5)
    A = ops.attention_term_magnitudes(d, q, k, v, S, H, Dh, 0.5)
    for got, mag in zip((o, dq, dk, dv), A):
        assert np.all(np.abs(got) <= mag * (1 + 1e-12) + 1e-15)
    o_pos, _ = ops.attention(q, k, np.abs(v), S, H, Dh, 0.5)
    np.testing.assert_allclose(ops.attention_term_magnitudes(d, q, k, np.abs(v), S, H, Dh, 0.5)[0], o_pos,
                               rtol=1e-13)
    dv_pos = ops.attention_bwd(np.abs(d), q, k, v, S, H, Dh, 0.5)[2]
    np.testing.assert_allclose(ops.attention_term_magnitudes(np.abs(d), q, k, v, S, H, Dh, 0.5)[3], dv_pos,
                               rtol=1e-13)
