"""GPU parity: every op's forward and backward through the C ABI against the
oracle, on seeded inputs, at sizes the oracle finishes quickly that still
span several tiles, a partial 16-byte pack, unaligned rows (generic path)
and the tiny 8 x 64 configuration."""
import math

import numpy as np
import pytest

from oracle import ops, rng
from oracle.numerics import round_bf16
import synth

pytestmark = pytest.mark.gpu

if True:  # GPU-only imports are deferred so CPU collection never loads libxt
    try:
        import torch
        import autograd_row_wise_amd as xt
        from xt_testutil import bwd, close, close_f32, dev, empty, fwd, host, sum_scale
    except Exception:  # pragma: no cover - CPU host without the library
        pass

DTYPES = ["f32", "bf16"]
# (rows, cols, ld): ld None = contiguous
LAYOUTS = [(8, 64, None), (37, 1000, None), (37, 1000, 1008), (37, 1001, None), (37, 1001, 1008),
           (5, 3001, 3008), (3, 20000, None), (130, 256, None), (9, 32768, None),
           # wider than any register-resident row: the streaming kernels, ragged and strided
           (3, 40000, None), (2, 65601, 65608),
           # a vocabulary-wide row: every row starts at another offset modulo 16 bytes
           (9, 50257, None),
           # aligned rows past the register kernels' reach whose parameter partials the
           # streaming backward keeps per thread (f32 up to 4 packs, bf16 up to 2 per thread)
           (33, 16384, None), (20, 12288, None), (17, 16000, 16004),
           # ... with a tail of 3 elements after the last whole f32 pack
           (6, 15999, 16004)]


def put(a_f32: np.ndarray, dtype: str, ld=None):
    """Store host values (f32) on the device in `dtype`, optionally inside a
    wider row pitch; returns (device view tensor, f64 values it holds)."""
    R, C = a_f32.shape
    bits = synth.host_bf16_bits(a_f32) if dtype == "bf16" else a_f32.astype(np.float32)
    vals = synth.bf16_bits_to_f32(bits).astype(np.float64) if dtype == "bf16" else bits.astype(np.float64)
    if ld is None:
        return dev(bits, dtype), vals
    pad = np.zeros((R, ld), dtype=bits.dtype)
    pad[:, :C] = bits
    return dev(pad, dtype)[:, :C], vals


def out_like(R, C, dtype, ld=None):
    if ld is None:
        return empty((R, C), dtype)
    return empty((R, ld), dtype)[:, :C]


def normal(shape, seed, stream, mean=0.0, std=1.0):
    return synth.host_normal(shape, seed, stream, mean, std, "f32")


# ------------------------------------------------------------------ rms_norm
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("R,C,ld", LAYOUTS)
def test_rms_norm(dtype, R, C, ld):
    eps = 1e-5
    x, xv = put(normal((R, C), 0, "x"), dtype, ld)
    g = dev(normal((C,), 0, "gamma", 1.0, 0.1))
    gv = host(g)
    d, dv = put(normal((R, C), 0, "dout"), dtype, ld)
    y, ir = out_like(R, C, dtype, ld), empty((R, 1), "f32")
    prm = xt.params(eps=eps)
    fwd(xt.OP.RMS_NORM, prm, [x, g], [y, ir])
    y_ref, ir_ref = ops.rms_norm(xv, gv, eps)
    close(host(y), y_ref, dtype, what="y")
    close_f32(host(ir)[:, 0], ir_ref, what="inv_rms")
    dx, dg = out_like(R, C, dtype, ld), empty((C,), "f32")
    bwd(xt.OP.RMS_NORM, prm, d, [x, g], [ir], [dx, dg])
    dx_ref, dg_ref = ops.rms_norm_bwd(dv, xv, gv, ir_ref)
    if dtype == "f32":
        # dx = ir*g - x*ir^3/C*sum(g*x): a signed combination of two terms
        gg = dv * gv[None, :]
        terms = ir_ref[:, None] * np.abs(gg) + np.abs(xv) * (ir_ref ** 3 / C * np.sum(np.abs(gg * xv), axis=1))[:, None]
        close_f32(host(dx), dx_ref, sum_scale(terms, 2), what="dx")
    else:
        close(host(dx), dx_ref, dtype, what="dx")
    A = np.sum(np.abs(dv * xv * ir_ref[:, None]), axis=0)
    close_f32(host(dg), dg_ref, sum_scale(A, R), what="dgamma")


# ---------------------------------------------------------------- layer_norm
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("R,C,ld", LAYOUTS)
def test_layer_norm(dtype, R, C, ld):
    eps = 1e-5
    x, xv = put(normal((R, C), 1, "x"), dtype, ld)
    g = dev(normal((C,), 1, "gamma", 1.0, 0.1))
    b = dev(normal((C,), 1, "beta", 0.0, 0.1))
    gv, bv = host(g), host(b)
    d, dv = put(normal((R, C), 1, "dout"), dtype, ld)
    y, mu, rs = out_like(R, C, dtype, ld), empty((R, 1), "f32"), empty((R, 1), "f32")
    prm = xt.params(eps=eps)
    fwd(xt.OP.LAYER_NORM, prm, [x, g, b], [y, mu, rs])
    y_ref, mu_ref, rs_ref = ops.layer_norm(xv, gv, bv, eps)
    close(host(y), y_ref, dtype, what="y")
    close_f32(host(mu)[:, 0], mu_ref, sum_scale(np.sum(np.abs(xv), axis=1) / C, C), what="mean")
    close_f32(host(rs)[:, 0], rs_ref, what="rstd")
    dx, dg, db = out_like(R, C, dtype, ld), empty((C,), "f32"), empty((C,), "f32")
    bwd(xt.OP.LAYER_NORM, prm, d, [x, g, b], [mu, rs], [dx, dg, db])
    dx_ref, dg_ref, db_ref = ops.layer_norm_bwd(dv, xv, gv, mu_ref, rs_ref)
    xhat = (xv - mu_ref[:, None]) * rs_ref[:, None]
    if dtype == "f32":
        # dx = rstd*(g - mean(g) - xhat*mean(g*xhat)) is a difference of
        # row sums: scale its bar by the magnitude of the terms
        gg = dv * gv[None, :]
        scale = rs_ref[:, None] * (np.abs(gg) + np.mean(np.abs(gg), axis=1, keepdims=True)
                                   + np.abs(xhat) * np.mean(np.abs(gg * xhat), axis=1, keepdims=True))
        close_f32(host(dx), dx_ref, sum_scale(scale, 3), what="dx")
    else:
        close(host(dx), dx_ref, dtype, what="dx")
    close_f32(host(dg), dg_ref, sum_scale(np.sum(np.abs(dv * xhat), axis=0), R), what="dgamma")
    close_f32(host(db), db_ref, sum_scale(np.sum(np.abs(dv), axis=0), R), what="dbeta")


# ------------------------------------------------------------------ softmax
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("R,C,ld", LAYOUTS)
@pytest.mark.parametrize("alpha,causal", [(1.0, 0), (0.125, 1)])
def test_softmax(dtype, R, C, ld, alpha, causal):
    S = min(C, 16) if causal else 0
    x, xv = put(normal((R, C), 2, "x", std=2.0), dtype, ld)
    d, dv = put(normal((R, C), 2, "dout"), dtype, ld)
    y = out_like(R, C, dtype, ld)
    prm = xt.params(alpha=alpha, causal=causal, seq_len=S)
    fwd(xt.OP.SOFTMAX, prm, [x], [y])
    y_ref = ops.softmax(xv, alpha, bool(causal), S)
    close(host(y), y_ref, dtype, what="y")
    dx = out_like(R, C, dtype, ld)
    bwd(xt.OP.SOFTMAX, prm, d, [x], [y], [dx])
    y_saved = round_bf16(y_ref) if dtype == "bf16" else y_ref
    dx_ref = ops.softmax_bwd(dv, y_saved, alpha)
    if dtype == "f32":
        dot = np.sum(np.abs(dv * y_saved), axis=1, keepdims=True)
        close_f32(host(dx), dx_ref, sum_scale(alpha * y_saved * (np.abs(dv) + dot), 2), what="dx")
    else:
        close(host(dx), dx_ref, dtype, what="dx")
    if causal:
        q = np.arange(R)[:, None] % S
        masked = np.arange(C)[None, :] > q
        assert np.all(host(y)[masked] == 0.0) and np.all(host(dx)[masked] == 0.0)


# ------------------------------------------------------------ cross entropy
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("R,V,ld", [(8, 64, None), (33, 5003, None), (17, 4096, 4100), (6, 50257, None)])
def test_cross_entropy(dtype, R, V, ld):
    x, xv = put(normal((R, V), 3, "logits", std=2.0), dtype, ld)
    t = synth.host_uniform_int((R,), 0, V, 3, "targets")
    td = dev(t.reshape(R, 1), "i32")
    L, lse, lr = empty((1, 1), "f32"), empty((R, 1), "f32"), empty((R, 1), "f32")
    prm = xt.params()
    fwd(xt.OP.CROSS_ENTROPY, prm, [x, td], [L, lse, lr])
    L_ref, lse_ref, lr_ref = ops.cross_entropy(xv, t)
    close_f32(host(lse)[:, 0], lse_ref, what="lse")
    close_f32(host(lr)[:, 0], lr_ref, what="loss_row")
    close_f32(host(L)[0, 0], L_ref, what="L")
    g = 0.75
    dL = dev(np.array([[g]], dtype=np.float32))
    dx = out_like(R, V, dtype, ld)
    bwd(xt.OP.CROSS_ENTROPY, prm, dL, [x, td], [lse], [dx, None])
    dx_ref = ops.cross_entropy_bwd(g, xv, t, lse_ref)
    close(host(dx), dx_ref, dtype, what="dlogits")


def test_cross_entropy_bad_targets_give_nan_rows():
    R, V = 4, 100
    x, xv = put(normal((R, V), 4, "logits"), "f32")
    t = np.array([3, -1, 100, 99], dtype=np.int32)
    td = dev(t.reshape(R, 1), "i32")
    L, lse, lr = empty((1, 1), "f32"), empty((R, 1), "f32"), empty((R, 1), "f32")
    fwd(xt.OP.CROSS_ENTROPY, xt.params(), [x, td], [L, lse, lr])
    _, _, lr_ref = ops.cross_entropy(xv, t)
    got = host(lr)[:, 0]
    assert np.array_equal(np.isnan(got), np.isnan(lr_ref)) and math.isnan(host(L)[0, 0])
    dx = empty((R, V), "f32")
    bwd(xt.OP.CROSS_ENTROPY, xt.params(), dev(np.ones((1, 1), np.float32)), [x, td], [lse], [dx, None])
    h = host(dx)
    assert np.all(np.isfinite(h[0])) and np.all(np.isfinite(h[3])) and np.all(np.isnan(h[1])) and np.all(np.isnan(h[2]))


# ------------------------------------------------------ silu / gelu / swiglu
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("R,C,ld", [(8, 64, None), (37, 1001, None), (37, 1001, 1008), (64, 688, None)])
@pytest.mark.parametrize("name", ["silu", "gelu", "gelu_tanh"])
def test_silu_gelu(dtype, R, C, ld, name):
    op = xt.OP.SILU if name == "silu" else xt.OP.GELU
    f, fb = {"silu": (ops.silu, ops.silu_bwd), "gelu": (ops.gelu, ops.gelu_bwd),
             "gelu_tanh": (ops.gelu_tanh, ops.gelu_tanh_bwd)}[name]
    prm = xt.params(gelu_tanh=int(name == "gelu_tanh"))
    x, xv = put(normal((R, C), 5, "x", std=3.0), dtype, ld)
    d, dv = put(normal((R, C), 5, "dout"), dtype, ld)
    y, dx = out_like(R, C, dtype, ld), out_like(R, C, dtype, ld)
    fwd(op, prm, [x], [y])
    close(host(y), f(xv), dtype, what="y")
    bwd(op, prm, d, [x], [], [dx])
    close(host(dx), fb(dv, xv), dtype, what="dx")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("R,C,ld", [(8, 64, None), (37, 1001, None), (64, 688, None), (16, 11008, None)])
def test_swiglu(dtype, R, C, ld):
    g, gv = put(normal((R, C), 6, "g", std=2.0), dtype, ld)
    u, uv = put(normal((R, C), 6, "u"), dtype, ld)
    d, dv = put(normal((R, C), 6, "dout"), dtype, ld)
    y = out_like(R, C, dtype, ld)
    fwd(xt.OP.SWIGLU, xt.params(), [g, u], [y])
    close(host(y), ops.swiglu(gv, uv), dtype, what="y")
    dg, du = out_like(R, C, dtype, ld), out_like(R, C, dtype, ld)
    bwd(xt.OP.SWIGLU, xt.params(), d, [g, u], [], [dg, du])
    dg_ref, du_ref = ops.swiglu_bwd(dv, gv, uv)
    close(host(dg), dg_ref, dtype, what="dg")
    close(host(du), du_ref, dtype, what="du")


# --------------------------------------------------------------------- rope
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("R,H,Dh,S", [(8, 4, 16, 8), (300, 4, 64, 256), (33, 2, 128, 4096), (10, 3, 6, 5),
                                     (5, 80, 128, 16),        # rows longer than one pipelined tile
                                     (20000, 8, 64, 1000)])   # more tiles than blocks: pipelined loop
def test_rope(dtype, R, H, Dh, S):
    C = H * Dh
    x, xv = put(normal((R, C), 7, "x"), dtype)
    d, dv = put(normal((R, C), 7, "dout"), dtype)
    prm = xt.params(head_dim=Dh, rope_base=10000.0, seq_len=S)
    y, dx = empty((R, C), dtype), empty((R, C), dtype)
    fwd(xt.OP.ROPE, prm, [x], [y])
    close(host(y), ops.rope(xv, Dh, 10000.0, S), dtype, what="y")
    bwd(xt.OP.ROPE, prm, d, [x], [], [dx])
    close(host(dx), ops.rope_bwd(dv, Dh, 10000.0, S), dtype, what="dx")
    if dtype == "f32":   # position 0 rows are the identity, bit for bit
        for r in range(0, R, S):
            assert np.array_equal(host(y)[r], xv[r])
    # accumulate: dx += rope_bwd(d) onto the previous dx
    prev = host(dx)
    bwd(xt.OP.ROPE, prm, d, [x], [], [dx], acc=1)
    close(host(dx), prev + ops.rope_bwd(dv, Dh, 10000.0, S), dtype, what="dx+=")


# ----------------------------------------------------------------- add_bias
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("R,C,ld", [(8, 64, None), (37, 1001, None), (37, 1001, 1008), (1000, 512, None)])
def test_add_bias(dtype, R, C, ld):
    x, xv = put(normal((R, C), 8, "x"), dtype, ld)
    b = dev(normal((C,), 8, "bias"))
    bv = host(b)
    d, dv = put(normal((R, C), 8, "dout"), dtype, ld)
    y = out_like(R, C, dtype, ld)
    fwd(xt.OP.ADD_BIAS, xt.params(), [x, b], [y])
    close(host(y), ops.add_bias(xv, bv), dtype, what="y")
    dx, db = out_like(R, C, dtype, ld), empty((C,), "f32")
    bwd(xt.OP.ADD_BIAS, xt.params(), d, [x, b], [], [dx, db])
    dx_ref, db_ref = ops.add_bias_bwd(dv)
    close(host(dx), dx_ref, dtype, what="dx")
    close_f32(host(db), db_ref, sum_scale(np.sum(np.abs(dv), axis=0), R), what="dbias")


# ------------------------------------------------------------------ dropout
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("R,C,ld,p,seed", [(8, 64, None, 0.1, 42), (37, 1001, None, 0.3, 7),
                                           (37, 1001, 1008, 0.5, 2 ** 63 + 5), (64, 4096, None, 0.1, 42 ^ 0xA77),
                                           (16, 64, None, 0.0, 1)])
def test_dropout(dtype, R, C, ld, p, seed):
    x, xv = put(normal((R, C), 9, "x"), dtype, ld)
    d, dv = put(normal((R, C), 9, "dout"), dtype, ld)
    y, m = out_like(R, C, dtype, ld), empty((R, C), "u8")
    prm = xt.params(p=p, seed=seed)
    fwd(xt.OP.DROPOUT, prm, [x], [y, m])
    y_ref, m_ref = rng.dropout(xv, p, seed)
    assert np.array_equal(host(m), m_ref), "mask differs from the oracle's"
    close(host(y), y_ref, dtype, what="y")
    if dtype == "f32":     # x*s rounded once to f32: exact
        assert np.array_equal(host(y).astype(np.float32), y_ref.astype(np.float32))
    if p == 0.0:
        assert np.array_equal(host(y), xv)
    dx = out_like(R, C, dtype, ld)
    bwd(xt.OP.DROPOUT, prm, d, [x], [m], [dx])
    close(host(dx), rng.dropout_bwd(dv, m_ref, p), dtype, what="dx")
    m2 = empty((R, C), "u8")
    xt.xt_dropout_mask(xt.view(m2), p, seed)
    torch.cuda.synchronize()
    assert np.array_equal(host(m2), m_ref)


# -------------------------------------------------------- add / mul / scale
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("R,C,ld", [(8, 64, None), (37, 1001, None), (37, 1001, 1008)])
def test_add_mul_scale(dtype, R, C, ld):
    a, av = put(normal((R, C), 10, "a"), dtype, ld)
    b, bv = put(normal((R, C), 10, "b"), dtype, ld)
    d, dv = put(normal((R, C), 10, "dout"), dtype, ld)
    for op, ref in [(xt.OP.ADD, av + bv), (xt.OP.MUL, av * bv)]:
        y = out_like(R, C, dtype, ld)
        fwd(op, xt.params(), [a, b], [y])
        close(host(y), ref, dtype, what=f"op{op}")
    y = out_like(R, C, dtype, ld)
    fwd(xt.OP.SCALE, xt.params(alpha=-0.37), [a], [y])
    close(host(y), -0.37 * av, dtype, what="scale")
    da, db = out_like(R, C, dtype, ld), out_like(R, C, dtype, ld)
    bwd(xt.OP.MUL, xt.params(), d, [a, b], [], [da, db])
    ra, rb = ops.mul_bwd(dv, av, bv)
    close(host(da), ra, dtype, what="da")
    close(host(db), rb, dtype, what="db")
    bwd(xt.OP.ADD, xt.params(), d, [a, b], [], [da, db])
    assert np.array_equal(host(da), dv) and np.array_equal(host(db), dv)
    bwd(xt.OP.SCALE, xt.params(alpha=-0.37), d, [a], [], [da])
    close(host(da), -0.37 * dv, dtype, what="dscale")


@pytest.mark.parametrize("dd,sd", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16"), ("bf16", "f32")])
def test_grad_accumulate_and_accumulate_bits(dd, sd):
    R, C = 37, 1001
    dst, dstv = put(normal((R, C), 11, "a"), dd)
    src, srcv = put(normal((R, C), 11, "b"), sd)
    xt.xt_grad_accumulate(xt.view(dst), xt.view(src))
    torch.cuda.synchronize()
    ref = dstv + srcv
    if dd == "f32":
        assert np.array_equal(host(dst), ref.astype(np.float32).astype(np.float64))
    else:
        assert np.array_equal(host(dst), round_bf16(ref.astype(np.float32)))


def test_fused_accumulate_fanout_is_exact():
    # mul(x, x) pushed twice into one f32 buffer via the accumulate bit, twice:
    # x+x+x+x == 4x exactly (the [AE] fan-out identity), with upstream 1
    R, C = 8, 64
    x, xv = put(normal((R, C), 12, "x"), "f32")
    ones = dev(np.ones((R, C), np.float32))
    gx = empty((R, C), "f32")
    for k in range(2):
        bwd(xt.OP.MUL, xt.params(), ones, [x, x], [], [gx, None], acc=1 if k else 0)
        bwd(xt.OP.MUL, xt.params(), ones, [x, x], [], [None, gx], acc=2)
    assert np.array_equal(host(gx), 4.0 * xv)


# ------------------------------------------------------------------ matmul
MM_CASES = [  # (M, N, K, ta, tb, batch)
    (8, 64, 64, 0, 0, (1, 1)), (200, 130, 70, 0, 0, (1, 1)), (200, 130, 70, 0, 1, (1, 1)),
    (200, 130, 70, 1, 0, (1, 1)), (200, 130, 70, 1, 1, (1, 1)), (256, 256, 64, 0, 1, (2, 3)),
    (129, 257, 300, 0, 0, (1, 1)), (512, 384, 256, 0, 0, (1, 1)),
    # whole-tile shapes: the large-tile kernels (256 x 256 x 32 bf16, 128 x 128 x 32 f32)
    (512, 256, 192, 0, 0, (1, 1)), (512, 256, 192, 0, 1, (1, 1)), (512, 256, 192, 1, 0, (1, 1)),
    (512, 256, 192, 1, 1, (1, 1)), (256, 512, 128, 0, 1, (2, 2)), (256, 256, 64, 1, 0, (1, 3)),
    (256, 256, 32, 1, 1, (1, 1)), (768, 512, 416, 0, 1, (1, 1)),
    # small f32 products on 16-byte chunks: 32 x 32 tiles with edge tiles in
    # both dimensions, and 64 x 64 tiles (more than 128 of them) with edges
    (200, 132, 72, 0, 0, (1, 1)), (196, 132, 72, 1, 1, (1, 1)),
    (1000, 700, 96, 0, 1, (1, 1)), (1000, 700, 96, 1, 0, (1, 1)),
]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N,K,ta,tb,batch", MM_CASES)
def test_matmul(dtype, M, N, K, ta, tb, batch):
    nb = batch[0] * batch[1]
    ash = (K, M) if ta else (M, K)
    bsh = (N, K) if tb else (K, N)
    A3 = normal((nb,) + ash, 13, "a")
    B3 = normal((nb,) + bsh, 13, "b", std=0.5)
    D3 = normal((nb, M, N), 13, "dout")
    def stack(a3):
        return a3.reshape(nb * a3.shape[1], a3.shape[2])
    A, Av = put(stack(A3), dtype)
    B, Bv = put(stack(B3), dtype)
    D, Dv = put(stack(D3), dtype)
    Av, Bv, Dv = (v.reshape((nb,) + s) for v, s in ((Av, ash), (Bv, bsh), (Dv, (M, N))))
    alpha = 0.5
    def bview(t, r, c):
        return xt.view(t, rows=r, cols=c, ld=c, nb=batch, sb=(batch[1] * r * c, r * c))
    Cout = empty((nb * M, N), dtype)
    prm = xt.params(alpha=alpha, trans_a=ta, trans_b=tb)
    xt.xt_op_fwd(xt.OP.MATMUL, prm, [bview(A, *ash), bview(B, *bsh)], [bview(Cout, M, N)])
    torch.cuda.synchronize()
    ref = ops.matmul(Av, Bv, alpha, bool(ta), bool(tb))
    absA = np.abs(Av); absB = np.abs(Bv)
    A_abs = alpha * ops.matmul(absA, absB, 1.0, bool(ta), bool(tb))
    got = host(Cout).reshape(nb, M, N)
    if dtype == "f32":
        close_f32(got, ref, sum_scale(A_abs, K), what="C")
    else:
        close(got, ref, "bf16", what="C")
    dA, dB = empty((nb * ash[0], ash[1]), "f32"), empty((nb * bsh[0], bsh[1]), "f32")
    xt.xt_op_bwd(xt.OP.MATMUL, prm, bview(D, M, N), [bview(A, *ash), bview(B, *bsh)], [],
                 [bview(dA, *ash), bview(dB, *bsh)], 0, None, 0)
    torch.cuda.synchronize()
    dA_ref, dB_ref = ops.matmul_bwd(Dv, Av, Bv, alpha, bool(ta), bool(tb))
    sA, sB = ops.matmul_bwd(np.abs(Dv), absA, absB, alpha, bool(ta), bool(tb))
    close_f32(host(dA).reshape(dA_ref.shape), dA_ref, sum_scale(sA, N), what="dA")
    close_f32(host(dB).reshape(dB_ref.shape), dB_ref, sum_scale(sB, M), what="dB")


# Few output tiles and a long K: the product is split along K into f32
# partials summed in a fixed order (needs the workspace xt_workspace_bytes
# reports; with less it splits less, with none it does not split).
SPLIT_CASES = [  # (M, N, K, ta, tb, batch)
    (128, 128, 2048, 1, 0, (1, 1)),     # one large f32 tile, 16 slices
    (256, 256, 1024, 1, 0, (1, 1)),     # one large bf16 tile
    (200, 130, 1000, 1, 0, (1, 1)),     # ragged: 128 x 128 kernel, ragged last slice
    (256, 128, 640, 0, 1, (2, 2)),      # batched
    (96, 64, 1537, 0, 0, (1, 1)),       # K not a multiple of any tile
]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("M,N,K,ta,tb,batch", SPLIT_CASES)
@pytest.mark.parametrize("ws_frac", [1.0, 0.5])
def test_matmul_split_k(dtype, M, N, K, ta, tb, batch, ws_frac):
    nb = batch[0] * batch[1]
    ash = (K, M) if ta else (M, K)
    bsh = (N, K) if tb else (K, N)
    A3 = normal((nb,) + ash, 17, "a")
    B3 = normal((nb,) + bsh, 17, "b", std=0.5)
    D3 = normal((nb, M, N), 17, "dout")
    def stack(a3):
        return a3.reshape(nb * a3.shape[1], a3.shape[2])
    A, Av = put(stack(A3), dtype)
    B, Bv = put(stack(B3), dtype)
    D, Dv = put(stack(D3), dtype)
    Av, Bv, Dv = (v.reshape((nb,) + s) for v, s in ((Av, ash), (Bv, bsh), (Dv, (M, N))))
    alpha = 0.5
    def bview(t, r, c):
        return xt.view(t, rows=r, cols=c, ld=c, nb=batch, sb=(batch[1] * r * c, r * c))
    prm = xt.params(alpha=alpha, trans_a=ta, trans_b=tb)
    ins = [bview(A, *ash), bview(B, *bsh)]
    wf = xt.xt_workspace_bytes(xt.OP.MATMUL, 0, prm, ins)
    wb = xt.xt_workspace_bytes(xt.OP.MATMUL, 1, prm, ins)
    assert wf > 0 or wb > 0, "this shape is meant to split"
    wsf = torch.empty(max(int(wf * ws_frac), 1), dtype=torch.uint8, device="cuda")
    wsb = torch.empty(max(int(wb * ws_frac), 1), dtype=torch.uint8, device="cuda")
    Cout = empty((nb * M, N), dtype)
    xt.xt_op_fwd(xt.OP.MATMUL, prm, ins, [bview(Cout, M, N)], wsf.data_ptr(), int(wf * ws_frac))
    torch.cuda.synchronize()
    ref = ops.matmul(Av, Bv, alpha, bool(ta), bool(tb))
    absA = np.abs(Av); absB = np.abs(Bv)
    A_abs = alpha * ops.matmul(absA, absB, 1.0, bool(ta), bool(tb))
    got = host(Cout).reshape(nb, M, N)
    if dtype == "f32":
        close_f32(got, ref, sum_scale(A_abs, K), what="C")
    else:
        close(got, ref, "bf16", what="C")
    dA, dB = empty((nb * ash[0], ash[1]), dtype), empty((nb * bsh[0], bsh[1]), "f32")
    dA_ref, dB_ref = ops.matmul_bwd(Dv, Av, Bv, alpha, bool(ta), bool(tb))
    sA, sB = ops.matmul_bwd(np.abs(Dv), absA, absB, alpha, bool(ta), bool(tb))
    # second call accumulates onto the first: the result is the sum of two
    # equal products (one f32 rounding of the add in dB; dA in its dtype)
    for acc in (0, 3):
        xt.xt_op_bwd(xt.OP.MATMUL, prm, bview(D, M, N), ins, [], [bview(dA, *ash), bview(dB, *bsh)], acc,
                     wsb.data_ptr(), int(wb * ws_frac))
        torch.cuda.synchronize()
    k = 2.0
    if dtype == "f32":
        close_f32(host(dA).reshape(dA_ref.shape), k * dA_ref, k * sum_scale(sA, N), what="dA")
    else:
        close(host(dA).reshape(dA_ref.shape), k * dA_ref, "bf16", what="dA")
    close_f32(host(dB).reshape(dB_ref.shape), k * dB_ref, k * sum_scale(sB, M), what="dB")


# ----------------------------------------------- accumulating row backwards
ACC_LAYOUTS = [(130, 256, None), (37, 1001, None), (33, 16384, None), (3, 40000, None), (5, 3001, 3008)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("R,C,ld", ACC_LAYOUTS)
@pytest.mark.parametrize("op", ["rms_norm", "layer_norm", "softmax"])
def test_row_backward_accumulate(op, dtype, R, C, ld):
    """A second backward with every accumulate bit set adds onto the first:
    f32 gradients become exactly twice the first pass (one rounding of g + g),
    bf16 dx twice the oracle within the bf16 bar; register-resident,
    streaming, owned-partial and column-pass layouts."""
    x, xv = put(normal((R, C), 6, "x"), dtype, ld)
    d, dv = put(normal((R, C), 6, "dout"), dtype, ld)
    g = dev(normal((C,), 6, "gamma", 1.0, 0.1))
    b = dev(normal((C,), 6, "beta", 0.0, 0.1))
    if op == "rms_norm":
        opc, prm, ins = xt.OP.RMS_NORM, xt.params(eps=1e-5), [x, g]
        saved = [empty((R, 1), "f32")]
        nparam = 1
    elif op == "layer_norm":
        opc, prm, ins = xt.OP.LAYER_NORM, xt.params(eps=1e-5), [x, g, b]
        saved = [empty((R, 1), "f32"), empty((R, 1), "f32")]
        nparam = 2
    else:
        opc, prm, ins = xt.OP.SOFTMAX, xt.params(), [x]
        saved = []
        nparam = 0
    y = out_like(R, C, dtype, ld)
    fwd(opc, prm, ins, [y] + saved)
    if op == "softmax":
        saved = [y]
    grads = [out_like(R, C, dtype, ld)] + [empty((C,), "f32") for _ in range(nparam)]
    bwd(opc, prm, d, ins, saved, grads)
    first = [host(t) for t in grads]
    bwd(opc, prm, d, ins, saved, grads, acc=(1 << len(grads)) - 1)
    for k, (t, f0) in enumerate(zip(grads, first)):
        if dtype == "f32" or k > 0:
            assert np.array_equal(host(t), 2.0 * f0), (op, k)
    if dtype == "bf16":
        if op == "rms_norm":
            ref = ops.rms_norm_bwd(dv, xv, host(g), ops.rms_norm(xv, host(g), 1e-5)[1])[0]
        elif op == "layer_norm":
            _, mu, rs = ops.layer_norm(xv, host(g), host(b), 1e-5)
            ref = ops.layer_norm_bwd(dv, xv, host(g), mu, rs)[0]
        else:
            ref = ops.softmax_bwd(dv, round_bf16(ops.softmax(xv)))
        close(host(grads[0]), 2.0 * ref, dtype, what="accumulated dx")
