"""Ops replayed from a captured HIP graph give the eager results bit for bit.

bench.py times the hot path by replaying captured graphs, so the kernels
must hold up under capture: a graph of one call of each op (norms with their
column-sum folds, softmax, cross-entropy with its mean, dbias, dropout, f32
and bf16 matmuls, fused attention, the embedding backward's sort and merge,
the global gradient norm) is replayed three times, with eager work and
synchronisations between the replays and every output overwritten with NaN
before each replay; each replay must reproduce the eager outputs exactly."""
import math

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

if True:  # GPU-only imports are deferred so CPU collection never loads libxt
    try:
        import torch
        import autograd_row_wise_amd as xt
    except Exception:  # pragma: no cover - CPU host without the library
        pass


def _ws(op, prm, ins, keep, is_bwd=1):
    n = xt.xt_workspace_bytes(op, is_bwd, prm, ins)
    if not n:
        return None, 0
    w = torch.empty(n, dtype=torch.uint8, device="cuda")
    keep.append(w)
    return w.data_ptr(), n


def _build():
    V, P = xt.view, xt.params
    keep, outs, fns = [], [], []

    sid = [400]

    def nd(shape, name, dtype="f32", mean=0.0, std=1.0):
        sid[0] += 1                                   # a stream of its own per tensor
        t = synth.device_normal(shape, 21, sid[0], mean, std, dtype=dtype)
        keep.append(t)
        return t

    def out(shape, dtype=torch.float32):
        t = torch.empty(shape, dtype=dtype, device="cuda")
        outs.append(t)
        return t

    bf = torch.bfloat16
    # rms_norm fwd / bwd (dgamma through the partial-column fold), bf16
    R, C = 300, 1000
    x, d = nd((R, C), "x", "bf16"), nd((R, C), "d", "bf16")
    gam = nd((1, C), "g", "f32", 1.0, 0.1)
    y, ir, dx, dg = out((R, C), bf), out((R, 1)), out((R, C), bf), out((1, C))
    pe = P(eps=1e-5)
    fns.append(lambda: xt.xt_op_fwd(xt.OP.RMS_NORM, pe, [V(x), V(gam)], [V(y), V(ir)]))
    w_rms = _ws(xt.OP.RMS_NORM, pe, [V(x), V(gam)], keep)
    fns.append(lambda: xt.xt_op_bwd(xt.OP.RMS_NORM, pe, V(d), [V(x), V(gam)], [V(ir)], [V(dx), V(dg)], 0, *w_rms))
    # layer_norm bwd, f32 (dgamma and dbeta folds)
    xf, df = nd((257, 768), "xf"), nd((257, 768), "df")
    g2, b2 = nd((1, 768), "g2", "f32", 1.0, 0.1), nd((1, 768), "b2", "f32", 0.0, 0.1)
    yl, mu, rs = out((257, 768)), out((257, 1)), out((257, 1))
    dxl, dgl, dbl = out((257, 768)), out((1, 768)), out((1, 768))
    fns.append(lambda: xt.xt_op_fwd(xt.OP.LAYER_NORM, pe, [V(xf), V(g2), V(b2)], [V(yl), V(mu), V(rs)]))
    w_ln = _ws(xt.OP.LAYER_NORM, pe, [V(xf), V(g2), V(b2)], keep)
    fns.append(lambda: xt.xt_op_bwd(xt.OP.LAYER_NORM, pe, V(df), [V(xf), V(g2), V(b2)], [V(mu), V(rs)],
                                    [V(dxl), V(dgl), V(dbl)], 0, *w_ln))
    # causal softmax fwd / bwd, bf16
    ps = P(alpha=0.125, causal=1, seq_len=256)
    sx, sd = nd((512, 256), "sx", "bf16"), nd((512, 256), "sd", "bf16")
    sy, sdx = out((512, 256), bf), out((512, 256), bf)
    fns.append(lambda: xt.xt_op_fwd(xt.OP.SOFTMAX, ps, [V(sx)], [V(sy)]))
    fns.append(lambda: xt.xt_op_bwd(xt.OP.SOFTMAX, ps, V(sd), [V(sx)], [V(sy)], [V(sdx)]))
    # cross-entropy fwd (with the fixed-order mean) / bwd, f32
    cx = nd((64, 5003), "cx", "f32", 0.0, 2.0)
    tg = torch.from_numpy(synth.host_uniform_int((64, 1), 0, 5003, 21, "targets")).cuda()
    one = torch.full((1, 1), 0.5, dtype=torch.float32, device="cuda")
    keep += [tg, one]
    L, lse, lr, cdx = out((1, 1)), out((64, 1)), out((64, 1)), out((64, 5003))
    fns.append(lambda: xt.xt_op_fwd(xt.OP.CROSS_ENTROPY, P(), [V(cx), V(tg)], [V(L), V(lse), V(lr)]))
    tslot = V(tg)
    tslot.data = None
    fns.append(lambda: xt.xt_op_bwd(xt.OP.CROSS_ENTROPY, P(), V(one), [V(cx), V(tg)], [V(lse)], [V(cdx), tslot]))
    # dbias column sum (partials + fold), bf16
    bx, bd = nd((4099, 512), "bx", "bf16"), nd((4099, 512), "bd", "bf16")
    bias = nd((1, 512), "bias")
    bdx, bdb = out((4099, 512), bf), out((1, 512))
    w_b = _ws(xt.OP.ADD_BIAS, P(), [V(bx), V(bias)], keep)
    fns.append(lambda: xt.xt_op_bwd(xt.OP.ADD_BIAS, P(), V(bd), [V(bx), V(bias)], [], [V(bdx), V(bdb)], 0, *w_b))
    # dropout forward (counter-based mask), bf16
    pd = P(p=0.1, seed=42)
    dy, dm = out((300, 1000), bf), out((300, 1000), torch.uint8)
    fns.append(lambda: xt.xt_op_fwd(xt.OP.DROPOUT, pd, [V(x)], [V(dy), V(dm)]))
    # matmuls: f32 (split-k) and bf16 on the matrix cores
    A, B = nd((256, 3000), "A"), nd((3000, 192), "B")
    Cf = out((256, 192))
    w_mf = _ws(xt.OP.MATMUL, P(), [V(A), V(B)], keep, 0)
    fns.append(lambda: xt.xt_op_fwd(xt.OP.MATMUL, P(), [V(A), V(B)], [V(Cf)], *w_mf))
    Ab, Bb = nd((512, 1024), "Ab", "bf16"), nd((1024, 768), "Bb", "bf16")
    Cb = out((512, 768), bf)
    w_mb = _ws(xt.OP.MATMUL, P(), [V(Ab), V(Bb)], keep, 0)
    fns.append(lambda: xt.xt_op_fwd(xt.OP.MATMUL, P(), [V(Ab), V(Bb)], [V(Cb)], *w_mb))
    # fused causal attention fwd / bwd, bf16
    S_, H_, D_ = 256, 4, 64
    q, k, v, do = (nd((2 * S_, H_ * D_), n, "bf16") for n in ("q", "k", "v", "do"))
    pa = P(alpha=1.0 / math.sqrt(D_), causal=1, seq_len=S_, head_dim=D_)
    ao, al = out((2 * S_, H_ * D_), bf), out((2 * S_, H_))
    dq, dk, dv = (out((2 * S_, H_ * D_), bf) for _ in range(3))
    ins_a = [V(q), V(k), V(v)]
    fns.append(lambda: xt.xt_op_fwd(xt.OP.ATTENTION, pa, ins_a, [V(ao), V(al)]))
    w_a = _ws(xt.OP.ATTENTION, pa, ins_a, keep)
    fns.append(lambda: xt.xt_op_bwd(xt.OP.ATTENTION, pa, V(do), ins_a, [V(ao), V(al)], [V(dq), V(dk), V(dv)], 0,
                                    *w_a))
    # embedding backward (sort, merge rounds, run table, segment sums), f32
    E = nd((997, 256), "E")
    ids = torch.from_numpy(synth.host_zipf_int((20000, 1), 997, 1.1, 21, "ids")).cuda()
    ed = nd((20000, 256), "ed")
    keep.append(ids)
    dE = out((997, 256))
    w_e = _ws(xt.OP.EMBED, P(), [V(E), V(ids)], keep)
    islot = V(ids)
    islot.data = None
    fns.append(lambda: xt.xt_op_bwd(xt.OP.EMBED, P(), V(ed), [V(E), V(ids)], [], [V(dE), islot], 0, *w_e))
    # global gradient norm over a list of buffers (f64 partials, fixed order)
    gl = [nd(s, "gr%d" % i, "f32", 0.0, 1e-2) for i, s in enumerate([(768, 768), (1, 768), (3072, 768), (5, 7)])]
    gv = [V(t) for t in gl]
    nb = xt.xt_grad_norm_workspace(gv)
    gw = torch.empty(max(nb, 8), dtype=torch.uint8, device="cuda")
    keep.append(gw)
    gn = out((2,))
    fns.append(lambda: xt.xt_grad_norm(gv, 1.0, gn.data_ptr(), gw.data_ptr(), nb))
    return fns, outs, keep


def test_graph_replays_reproduce_eager_results():
    fns, outs, keep = _build()
    for fn in fns:
        fn()
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for fn in fns:
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in fns:
            fn()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            if t.dtype == torch.uint8:
                t.fill_(7)
            else:
                t.fill_(float("nan"))
        scratch = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, ref) in enumerate(zip(outs, want)):
            assert torch.equal(got.view(torch.uint8) if got.dtype != torch.uint8 else got,
                               ref.view(torch.uint8) if ref.dtype != torch.uint8 else ref), (rep, i)
        del scratch
    del g, keep


@pytest.mark.parametrize("fused", [False, True])
def test_tape_block_replays_from_a_graph(fused):
    """The tiny transformer block (batch 4, seq 256, d 256, 4 x 64 heads, f32)
    recorded and run backward on a tape inside a graph capture: every
    replay (three, with eager work and synchronisations between them and the
    gradients overwritten with NaN before each) reproduces the eager tape's
    loss and weight gradients bit for bit."""
    from autograd_row_wise_amd import block as xb
    shp = xb.BlockShape(B=4, S=256, H=4, Dh=64, hidden=688, vocab=4096)
    W = {}
    for k, s in xb.WEIGHT_SHAPES(shp).items():
        W[k] = torch.ones(s, device="cuda") if k.startswith("g") else synth.device_normal(s, 31, k, 0.0, 0.02)
    x = synth.device_normal((shp.B * shp.S, shp.D), 31, "x")
    tg = synth.device_uniform_int((shp.B * shp.S, 1), 0, shp.vocab, 31, "targets")

    def record():
        t = xt.Tape()
        w = xb.leaves(t, W)
        loss = xb.block(t, w, t.leaf(xt.view(x)), t.leaf(xt.view(tg), requires_grad=False), shp, xt.DT.F32,
                        fused_attention=fused)
        t.backward(loss)
        return t, w, loss

    te, we, le = record()
    torch.cuda.synchronize()
    ref = {k: xt.to_torch(te.grad(v)).clone() for k, v in we.items()}
    ref_loss = xt.to_torch(te.value(le)).clone()
    te.close()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm-up on a side stream, as torch asks before a capture
        tw, _, _ = record()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    tw.close()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tc, wc, lc = record()
    torch.cuda.synchronize()
    grads = {k: xt.to_torch(tc.grad(v)) for k, v in wc.items()}       # copies: re-read after each replay
    for rep in range(3):
        for k, v in wc.items():
            view = tc.grad(v)                                             # overwrite every gradient with NaN
            nb = ((view.rows - 1) * view.ld + view.cols) * 4
            xt._raw_cuda_tensor(view.data, nb).view(torch.float32).fill_(float("nan"))
        junk = torch.randn(1 << 20, device="cuda").sum()                  # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in wc.items():
            got = xt.to_torch(tc.grad(v))
            assert torch.equal(got, ref[k]), (fused, rep, k)
        assert torch.equal(xt.to_torch(tc.value(lc)), ref_loss)
        del junk
    del grads
    tc.close()
    del g
