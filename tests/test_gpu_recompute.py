"""GPU: activation recompute on the tape.  A layer recorded as a checkpoint
segment keeps only its output; the backward re-runs the segment and must
reproduce the first forward bit for bit ([DO] "RNG：counter-based": the
counter-based dropout exists so that a re-run draws the same masks).  The
checkpointed tape is compared bitwise with the same graph recorded without
segments (itself checked against the oracle tape in test_gpu_tape) and with
the oracle directly."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

try:
    import torch
    import autograd_row_wise_amd as xt
    from autograd_row_wise_amd import block as xb
    from oracle_block import block_loss
    from xt_testutil import close_chain_f32, dev, host
except Exception:  # pragma: no cover
    pass


def tg(tape, var):
    return host(xt.to_torch(tape.grad(var)))


def mask(tape, var):
    return xt.to_torch(tape.saved(var, 1)).cpu().numpy().copy()


def inputs(shp, seed, w_std):
    g = {}
    for k, s in xb.WEIGHT_SHAPES(shp).items():
        g[k] = np.ones(s, np.float32) if k.startswith("g") else synth.host_normal(s, seed, k, 0.0, w_std)
    x0 = synth.host_normal((shp.B * shp.S, shp.D), seed, "x")
    t0 = synth.host_uniform_int((shp.B * shp.S,), 0, shp.vocab, seed, "targets")
    return g, x0, t0


def run(shp, g, x0, t0, p_drop, base_seed, layers, ckpt, passes=1):
    """`layers` pre-norm layers sharing one weight set, each optionally one
    checkpoint segment, then the loss head.  Returns the loss, the leaf
    gradients after each backward pass, the masks of the first forward and
    the masks present after the last backward."""
    W = {k: dev(v) for k, v in g.items()}
    x = dev(x0)
    tt = dev(t0.reshape(-1, 1), "i32")
    t = xt.Tape()
    w = xb.leaves(t, W)
    vx = t.leaf(xt.view(x))
    h = vx
    taps_all, first_masks = [], []
    for li in range(layers):
        taps = {}
        if ckpt:
            t.checkpoint_begin()
        h2 = xb.block_layer(t, w, h, shp, xt.DT.F32, p_drop, base_seed, li, taps=taps)
        torch.cuda.synchronize()
        first_masks.append([mask(t, taps["drop_attn"]), mask(t, taps["drop_ffn"])])
        if ckpt:
            t.checkpoint_end(h2)
        taps_all.append(taps)
        h = h2
    logits = t.apply(xt.OP.MATMUL, xt.params(), t.apply(xt.OP.RMS_NORM, xt.params(eps=1e-5), h, w["g3"]), w["wout"])
    loss = t.apply(xt.OP.CROSS_ENTROPY, xt.params(), logits, t.leaf(xt.view(tt), requires_grad=False))
    grads = []
    for _ in range(passes):
        t.backward(loss)
        torch.cuda.synchronize()
        gp = {k: tg(t, v) for k, v in w.items()}
        gp["x"] = tg(t, vx)
        grads.append(gp)
    L = host(xt.to_torch(t.value(loss)))[0, 0]
    # the walk recomputes the newest segment first, so the first layer's
    # masks are the ones in the arena after the backward
    after = [[mask(t, tp["drop_attn"]), mask(t, tp["drop_ffn"])] for tp in taps_all[:1]] if ckpt else None
    t.close()
    return L, grads, first_masks, after


@pytest.mark.parametrize("shape", ["tiny", "config2"])
def test_checkpointed_layer_is_bitwise_the_plain_one(shape):
    if shape == "tiny":
        shp, w_std = xb.BlockShape(B=2, S=8, H=2, Dh=8, hidden=12, vocab=11), 0.3
    else:
        shp, w_std = xb.BlockShape(B=4, S=256, H=4, Dh=64, hidden=688, vocab=4096), 0.02
    g, x0, t0 = inputs(shp, 3, w_std)
    Lp, gp, mp, _ = run(shp, g, x0, t0, 0.2, 42, 1, False)
    Lc, gc, mc, after = run(shp, g, x0, t0, 0.2, 42, 1, True)
    assert Lp == Lc
    for k in gp[0]:
        assert np.array_equal(gp[0][k], gc[0][k]), k
    # first-forward masks equal, and the recompute drew the same masks again
    for a, b in zip(mp[0], mc[0]):
        assert np.array_equal(a, b)
    for a, b in zip(mc[0], after[0]):
        assert np.array_equal(a, b)
    assert 0.1 < 1.0 - mc[0][0].mean() < 0.3          # p = 0.2 drops about a fifth
    # and the oracle agrees (same bar as the plain block test)
    o, P, ox, ol = block_loss({k: v.astype(np.float64) for k, v in g.items()}, x0.astype(np.float64), t0,
                              shp.B, shp.S, shp.H, shp.Dh, 0.2, 42)
    o.backward(ol)
    assert abs(Lc - float(o.value(ol)[0])) <= 1e-6 + 1e-5 * abs(Lc)
    for k in P:
        close_chain_f32(gc[0][k], o.grad(P[k]).reshape(gc[0][k].shape), what=f"recompute d{k}")


def test_two_segments_and_repeated_backward():
    """Two checkpointed layers over one weight set (the weight gradients sum
    over both segments); two backward passes accumulate into the leaves and
    recompute both segments each time."""
    shp = xb.BlockShape(B=2, S=16, H=2, Dh=8, hidden=24, vocab=13)
    g, x0, t0 = inputs(shp, 4, 0.3)
    Lp, gp, mp, _ = run(shp, g, x0, t0, 0.1, 7, 2, False, passes=2)
    Lc, gc, mc, after = run(shp, g, x0, t0, 0.1, 7, 2, True, passes=2)
    assert Lp == Lc
    for p in range(2):
        for k in gp[p]:
            assert np.array_equal(gp[p][k], gc[p][k]), (p, k)
    # layer seeds differ (base ^ layer ^ site): the two layers' masks differ
    assert not np.array_equal(mc[0][0], mc[1][0])
    for a, b in zip(mc[0], after[0]):
        assert np.array_equal(a, b)
    for k in gp[0]:
        close_chain_f32(gc[1][k], 2 * gc[0][k], what=f"second pass d{k}")


def test_segment_rules():
    shp = xb.BlockShape(B=1, S=8, H=2, Dh=4, hidden=8, vocab=5)
    g, x0, t0 = inputs(shp, 5, 0.3)
    W = {k: dev(v) for k, v in g.items()}
    x = dev(x0)
    t = xt.Tape()
    w = xb.leaves(t, W)
    vx = t.leaf(xt.view(x))
    with pytest.raises(xt.XtError):
        t.checkpoint_end(vx)                          # no segment open
    t.checkpoint_begin()
    with pytest.raises(xt.XtError):
        t.checkpoint_begin()                          # segments do not nest
    taps = {}
    h2 = xb.block_layer(t, w, vx, shp, xt.DT.F32, 0.1, 1, 0, taps=taps)
    with pytest.raises(xt.XtError):
        t.checkpoint_end(vx)                          # not a node of the segment
    with pytest.raises(xt.XtError):
        t.backward(h2)                                # a segment is open
    t.checkpoint_end(h2)
    with pytest.raises(xt.XtError):                   # a closed segment's inner node
        t.apply(xt.OP.SCALE, xt.params(alpha=2.0), taps["n1"])
    with pytest.raises(xt.XtError):
        t.value(taps["n1"])                           # its buffer was reused
    y = t.apply(xt.OP.SCALE, xt.params(alpha=2.0), h2)  # the output stays usable
    assert host(xt.to_torch(t.value(y))).shape == (shp.B * shp.S, shp.D)
    t.close()
