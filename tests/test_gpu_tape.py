"""GPU parity of the tape (xt_tape_*): reverse traversal, fan-out sums, the
composed attention and the small transformer block, against the oracle tape."""
import os

import numpy as np
import pytest

import synth
from oracle.tape import Tape as OTape

pytestmark = pytest.mark.gpu

try:
    import torch
    import autograd_row_wise_amd as xt
    from autograd_row_wise_amd import block as xb
    from oracle_block import block_loss
    from xt_testutil import close_chain_f32, dev, host
except Exception:  # pragma: no cover
    pass

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tg(tape, var):
    return host(xt.to_torch(tape.grad(var)))


def tv(tape, var):
    return host(xt.to_torch(tape.value(var)))


def test_dual_worked_example():
    row = [l.split() for l in open(os.path.join(GOLDEN, "dual_worked_example.txt")) if l.strip() and l[0] != "#"][0]
    x0, val, der = map(float, row)
    x = dev(np.array([[x0]], np.float32))
    t = xt.Tape()
    vx = t.leaf(xt.view(x))
    f = t.apply(xt.OP.ADD, xt.params(), t.apply(xt.OP.MUL, xt.params(), vx, vx),
                t.apply(xt.OP.SCALE, xt.params(alpha=3.0), vx))
    t.backward(f)
    torch.cuda.synchronize()
    assert tv(t, f)[0, 0] == val and tg(t, vx)[0, 0] == der


def test_fanout_four_x_exact_and_repeated_backward():
    x0 = synth.host_normal((8, 64), 3, "x")
    W0 = synth.host_normal((8, 64), 3, "w")
    x, W, ones = dev(x0), dev(W0), dev(np.ones((8, 64), np.float32))
    t = xt.Tape()
    vx = t.leaf(xt.view(x))
    y = t.apply(xt.OP.ADD, xt.params(), t.apply(xt.OP.MUL, xt.params(), vx, vx),
                t.apply(xt.OP.MUL, xt.params(), vx, vx))
    t.backward_seeded(y, xt.view(ones))
    torch.cuda.synchronize()
    x64 = x0.astype(np.float64)
    assert np.array_equal(tg(t, vx), 4.0 * x64)
    t.zero_grad()
    assert not t.grad(vx).data
    t.backward_seeded(y, xt.view(W))
    torch.cuda.synchronize()
    a = (W0 * x0).astype(np.float32).astype(np.float64)       # one f32 rounding per push
    assert np.array_equal(tg(t, vx), 4.0 * a)
    # a second pass adds into the leaf gradient ([BP] microbatch += semantics)
    t.backward_seeded(y, xt.view(W))
    torch.cuda.synchronize()
    # the four pushes of the second pass land one at a time, each rounded to f32
    exp = (4.0 * a).astype(np.float32)
    for _ in range(4):
        exp = (exp + a.astype(np.float32)).astype(np.float32)
    assert np.array_equal(tg(t, vx), exp.astype(np.float64)), "second pass did not add push by push"


def test_dropout_p0_records_no_node():
    x = dev(np.ones((2, 8), np.float32))
    t = xt.Tape()
    vx = t.leaf(xt.view(x))
    n = t.num_nodes()
    assert t.apply(xt.OP.DROPOUT, xt.params(p=0.0, seed=5), vx) == vx and t.num_nodes() == n


def test_composed_attention_single_head():
    S, Dh = 37, 16
    Q0, K0, V0, W0 = (synth.host_normal((S, Dh), 5, s) for s in ("q", "k", "v", "w"))
    Q, K, V, W = (dev(a) for a in (Q0, K0, V0, W0))
    t = xt.Tape()
    q, k, v = (t.leaf(xt.view(a)) for a in (Q, K, V))
    out = xb.attention(t, q, k, v, 1, S, 1, Dh, xt.DT.F32)
    t.backward_seeded(out, xt.view(W))
    torch.cuda.synchronize()
    o = OTape()
    oq, ok, ov = o.leaf(Q0), o.leaf(K0), o.leaf(V0)
    sc = o.matmul(oq, ok, 1.0, False, True)
    oo = o.matmul(o.softmax(o.scale(sc, 1 / np.sqrt(Dh)), 1.0, True, S), ov)
    o.backward(o.sum(o.mul(o.leaf(W0), oo)))
    close_chain_f32(tv(t, out), o.value(oo), what="composed attention out")
    for name, gv, ov_ in (("dq", q, oq), ("dk", k, ok), ("dv", v, ov)):
        close_chain_f32(tg(t, gv), o.grad(ov_), what=f"composed attention {name}")


def _block_case(shp, p_drop, seed=0, w_std=0.02, x_std=1.0):
    g = {}
    for k, s in xb.WEIGHT_SHAPES(shp).items():
        if k.startswith("g"):
            g[k] = np.ones(s, np.float32)
        else:
            g[k] = synth.host_normal(s, seed, k, 0.0, w_std)
    x0 = synth.host_normal((shp.B * shp.S, shp.D), seed, "x", 0.0, x_std)
    t0 = synth.host_uniform_int((shp.B * shp.S,), 0, shp.vocab, seed, "targets")
    return g, x0, t0


def _run_block(shp, p_drop, base_seed, seed=0, w_std=0.02):
    g, x0, t0 = _block_case(shp, p_drop, seed, w_std)
    W = {k: dev(v) for k, v in g.items()}
    x = dev(x0)
    tt = dev(t0.reshape(-1, 1), "i32")
    t = xt.Tape()
    w = xb.leaves(t, W)
    vx = t.leaf(xt.view(x))
    loss = xb.block(t, w, vx, t.leaf(xt.view(tt), requires_grad=False), shp, xt.DT.F32, p_drop, base_seed)
    t.backward(loss)
    torch.cuda.synchronize()
    got = {k: tg(t, v) for k, v in w.items()}
    got["x"] = tg(t, vx)
    L = tv(t, loss)[0, 0]
    o, P, ox, ol = block_loss({k: v.astype(np.float64) for k, v in g.items()}, x0.astype(np.float64), t0,
                              shp.B, shp.S, shp.H, shp.Dh, p_drop, base_seed)
    o.backward(ol)
    ref = {k: o.grad(P[k]) for k in P}
    ref["x"] = o.grad(ox)
    t.close()
    return L, float(o.value(ol)[0]), got, ref


def _check_block(L, Lr, got, ref):
    # A full block composes ~40 ops: the loss at the per-op f32 bar, every
    # gradient element at the composed-graph f32 bar (1e-6 + 1e-5 (|ref| +
    # rms(ref))), with the literal-bar pass rate printed beside it.
    assert abs(L - Lr) <= 1e-6 + 1e-5 * abs(Lr), (L, Lr)
    for k in ref:
        close_chain_f32(got[k], ref[k].reshape(got[k].shape), what=f"block d{k}")


@pytest.mark.parametrize("p_drop,base_seed", [(0.0, 0), (0.2, 42)])
def test_tiny_block_matches_oracle(p_drop, base_seed):
    shp = xb.BlockShape(B=2, S=8, H=2, Dh=8, hidden=12, vocab=11)
    _check_block(*_run_block(shp, p_drop, base_seed, w_std=0.3))


def test_config2_block_matches_oracle():
    """batch 4, seq 256, d_model 256, 4 heads x 64, SwiGLU 688, vocab 4096,
    weights N(0, 0.02), activations N(0, 1), causal, f32: the full size."""
    shp = xb.BlockShape(B=4, S=256, H=4, Dh=64, hidden=688, vocab=4096)
    _check_block(*_run_block(shp, 0.0, 0))
