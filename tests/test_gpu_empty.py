"""Degenerate sizes through the C ABI: tensors with zero rows.

Reading of the pages for R = 0 (they are silent): every row-wise and
element-wise op is a no-op; a parameter gradient is a sum over rows, so over
no rows it is zero (stored when not accumulating, left as it was when
accumulating); the cross-entropy mean over no rows is 0/0 = NaN, as numpy's
mean of an empty array; a matmul whose contraction length is zero writes
alpha * 0.  Every case checks the oracle gives the same answer."""
import numpy as np
import pytest

from oracle import ops

pytestmark = pytest.mark.gpu

if True:  # GPU-only imports are deferred so CPU collection never loads libxt
    try:
        import torch
        import autograd_row_wise_amd as xt
        from xt_testutil import bwd, dev, empty, fwd, host
    except Exception:  # pragma: no cover - CPU host without the library
        pass

SENTINEL = 7.0
C = 64


def filled(n, v=SENTINEL):
    return torch.full((n,), v, dtype=torch.float32, device="cuda")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("acc", [0, 2])
def test_rms_norm_zero_rows(dtype, acc):
    x, d, y, dx = (empty((0, C), dtype) for _ in range(4))
    g, ir = dev(np.ones(C)), empty((0, 1), "f32")
    fwd(xt.OP.RMS_NORM, xt.params(eps=1e-5), [x, g], [y, ir])
    dg = filled(C)
    bwd(xt.OP.RMS_NORM, xt.params(eps=1e-5), d, [x, g], [ir], [dx, dg], acc)
    ref = ops.rms_norm_bwd(np.zeros((0, C)), np.zeros((0, C)), np.ones(C), np.zeros(0))[1]
    want = SENTINEL + ref if acc else ref
    assert np.array_equal(host(dg), want), host(dg)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("acc", [0, 6])
def test_layer_norm_zero_rows(dtype, acc):
    x, d, y, dx = (empty((0, C), dtype) for _ in range(4))
    g, b = dev(np.ones(C)), dev(np.zeros(C))
    mu, rs = empty((0, 1), "f32"), empty((0, 1), "f32")
    fwd(xt.OP.LAYER_NORM, xt.params(eps=1e-5), [x, g, b], [y, mu, rs])
    dg, db = filled(C), filled(C)
    bwd(xt.OP.LAYER_NORM, xt.params(eps=1e-5), d, [x, g, b], [mu, rs], [dx, dg, db], acc)
    _, rg, rb = ops.layer_norm_bwd(np.zeros((0, C)), np.zeros((0, C)), np.ones(C), np.zeros(0), np.zeros(0))
    assert np.array_equal(host(dg), SENTINEL + rg if acc else rg)
    assert np.array_equal(host(db), SENTINEL + rb if acc else rb)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_add_bias_zero_rows(dtype):
    x, d, y, dx = (empty((0, C), dtype) for _ in range(4))
    bias = dev(np.arange(C, dtype=np.float32))
    fwd(xt.OP.ADD_BIAS, xt.params(), [x, bias], [y])
    db = filled(C)
    bwd(xt.OP.ADD_BIAS, xt.params(), d, [x, bias], [], [dx, db])
    assert np.array_equal(host(db), ops.add_bias_bwd(np.zeros((0, C)))[1])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_row_and_elementwise_ops_zero_rows(dtype):
    """Softmax, silu, gelu, swiglu, rope, dropout, add, mul, scale and the
    fan-out accumulate accept zero rows and launch nothing that fails."""
    x, u, d, y, dx, du = (empty((0, C), dtype) for _ in range(6))
    P = xt.params
    fwd(xt.OP.SOFTMAX, P(alpha=1.0), [x], [y])
    bwd(xt.OP.SOFTMAX, P(alpha=1.0), d, [x], [y], [dx])
    for op in (xt.OP.SILU, xt.OP.GELU):
        fwd(op, P(), [x], [y])
        bwd(op, P(), d, [x], [], [dx])
    fwd(xt.OP.SWIGLU, P(), [x, u], [y])
    bwd(xt.OP.SWIGLU, P(), d, [x, u], [], [dx, du])
    rp = P(head_dim=16, seq_len=8, rope_base=10000.0)
    fwd(xt.OP.ROPE, rp, [x], [y])
    bwd(xt.OP.ROPE, rp, d, [x], [], [dx])
    m = empty((0, C), "u8")
    fwd(xt.OP.DROPOUT, P(p=0.1, seed=42), [x], [y, m])
    bwd(xt.OP.DROPOUT, P(p=0.1, seed=42), d, [x], [m], [dx])
    xt.xt_dropout_mask(xt.view(m), 0.1, 42)
    for op in (xt.OP.ADD, xt.OP.MUL):
        fwd(op, P(), [x, u], [y])
        bwd(op, P(), d, [x, u], [], [dx, du])
    fwd(xt.OP.SCALE, P(alpha=0.5), [x], [y])
    bwd(xt.OP.SCALE, P(alpha=0.5), d, [x], [], [dx])
    xt.xt_grad_accumulate(xt.view(dx), xt.view(d))
    torch.cuda.synchronize()


def test_cross_entropy_zero_rows_is_nan():
    x, dx = empty((0, 50), "f32"), empty((0, 50), "f32")
    t = empty((0, 1), "i32")
    L, lse, lr = empty((1, 1), "f32"), empty((0, 1), "f32"), empty((0, 1), "f32")
    fwd(xt.OP.CROSS_ENTROPY, xt.params(), [x, t], [L, lse, lr])
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore"):
        ref = ops.cross_entropy(np.zeros((0, 50)), np.zeros(0, dtype=np.int32))[0]
    assert np.isnan(ref) and np.isnan(host(L)[0, 0])
    dL = dev(np.ones((1, 1)))
    bwd(xt.OP.CROSS_ENTROPY, xt.params(), dL, [x, t], [lse], [dx, None])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_matmul_zero_contraction_writes_zero(dtype):
    A, B = empty((5, 0), dtype), empty((0, 7), dtype)
    Cm = dev(np.full((5, 7), SENTINEL, dtype=np.float32))
    fwd(xt.OP.MATMUL, xt.params(), [A, B], [Cm])
    torch.cuda.synchronize()
    assert np.array_equal(host(Cm), ops.matmul(np.zeros((5, 0)), np.zeros((0, 7))))


def test_embedding_zero_tokens_zeroes_the_table_gradient():
    E = dev(np.ones((11, C), dtype=np.float32))
    ids, y, d = empty((0, 1), "i32"), empty((0, C), "f32"), empty((0, C), "f32")
    fwd(xt.OP.EMBED, xt.params(), [E, ids], [y])
    dE = dev(np.full((11, C), SENTINEL, dtype=np.float32))
    bwd(xt.OP.EMBED, xt.params(), d, [E, ids], [], [dE, None])
    assert np.array_equal(host(dE), ops.embed_bwd(np.zeros((0, C)), np.zeros(0, dtype=np.int32), 11))
