"""GPU parity of the fused attention (XT_OP_ATTENTION) through the C ABI
against the oracle: output, log-sum-exp and the three gradients, causal and
not, Dh 32 / 64 / 128, sequence lengths that leave ragged tiles (32-row f32
tiles; 128-row blocks and 32 / 64-row tiles of the bf16 kernels), f32 and
bf16 storage, accumulate mode, bitwise reproducibility; the bf16 path on
unaligned rows (the generic kernels); two heads of the 2 x 2048 x 16 x 128
bf16 workload against the oracle; two heads of a 2 x 4096-token causal
product large enough for the paired grid; and the fused op on the tape
inside the tiny block against the composed attention.

Bars, per element: f32 outputs and gradients are sums over up to S keys
(queries) of products, so each is judged at max(|ref|, A/sqrt(S)) with A the
sum of its terms' magnitudes from the oracle; bf16 ones at 2e-2 |ref| +
1e-2 rms(ref).  The oracle's backward reads the stored output for the row
term rowsum(dO * O), as the kernels do; the log-sum-exp is judged at
max(|ref|, 1) (a relative error of its inner sum is an absolute error of the
logarithm)."""
import math

import numpy as np
import pytest

from oracle import ops
import synth

pytestmark = pytest.mark.gpu

if True:  # GPU-only imports are deferred so CPU collection never loads libxt
    try:
        import torch
        import autograd_row_wise_amd as xt
        from xt_testutil import close_bf16, close_chain_f32, close_f32, dev, host, sum_scale
    except Exception:  # pragma: no cover - CPU host without the library
        pass


def put(a, dtype):
    bits = synth.host_bf16_bits(a) if dtype == "bf16" else a.astype(np.float32)
    vals = synth.bf16_bits_to_f32(bits).astype(np.float64) if dtype == "bf16" else bits.astype(np.float64)
    return dev(bits, dtype), vals


def check(got, ref, dtype, mag, n, what):
    """f32: the per-element rule for a sum of n terms whose magnitudes add up
    to `mag`; bf16: the per-element bf16 rule."""
    if dtype == "f32":
        close_f32(got, ref, sum_scale(mag, n), what=what)
    else:
        close_bf16(got, ref, what=what)


def check_lse(got, ref, what="lse"):
    close_f32(got, ref, np.maximum(np.abs(ref), 1.0), what=what)


def check_all(out, lse, grads, qv, kv, vv, dv, S, H, Dh, alpha, causal, dtype, where=""):
    """Output, log-sum-exp and the three gradients against the oracle; the
    oracle's backward reads the output the kernels stored."""
    o_ref, l_ref = ops.attention(qv, kv, vv, S, H, Dh, alpha, bool(causal))
    mags = ops.attention_term_magnitudes(dv, qv, kv, vv, S, H, Dh, alpha, bool(causal))
    check(host(out), o_ref, dtype, mags[0], S, ("out", where))
    check_lse(host(lse), l_ref, ("lse", where))
    refs = ops.attention_bwd(dv, qv, kv, vv, S, H, Dh, alpha, bool(causal), out=host(out))
    for name, g, r, m in zip(("dq", "dk", "dv"), grads, refs, mags[1:]):
        check(g if isinstance(g, np.ndarray) else host(g), r, dtype, m, S, (name, where))
    return refs, mags


CASES = [  # B, S, H, Dh, causal, dtype
    (2, 40, 2, 32, 1, "f32"),
    (1, 256, 4, 64, 1, "f32"),
    (3, 77, 1, 64, 0, "f32"),
    (1, 100, 2, 128, 1, "f32"),
    (2, 130, 2, 64, 1, "bf16"),
    (1, 64, 3, 128, 0, "bf16"),
    (1, 300, 2, 32, 1, "bf16"),
    (3, 200, 8, 64, 0, "bf16"),
    (2, 512, 4, 128, 1, "bf16"),
    (1, 1, 1, 64, 1, "bf16"),
]


@pytest.mark.parametrize("B,S,H,Dh,causal,dtype", CASES)
def test_attention_fwd_bwd(B, S, H, Dh, causal, dtype):
    R, C = B * S, H * Dh
    alpha = 1.0 / math.sqrt(Dh)
    q, qv = put(synth.host_normal((R, C), 11, "q"), dtype)
    k, kv = put(synth.host_normal((R, C), 11, "k"), dtype)
    v, vv = put(synth.host_normal((R, C), 11, "v"), dtype)
    d, dv = put(synth.host_normal((R, C), 11, "dout"), dtype)
    prm = xt.params(alpha=alpha, causal=causal, seq_len=S, head_dim=Dh)
    out = torch.empty((R, C), dtype=q.dtype, device="cuda")
    lse = torch.empty((R, H), dtype=torch.float32, device="cuda")
    ins = [xt.view(q), xt.view(k), xt.view(v)]
    xt.xt_op_fwd(xt.OP.ATTENTION, prm, ins, [xt.view(out), xt.view(lse)])
    torch.cuda.synchronize()
    grads = [torch.empty((R, C), dtype=q.dtype, device="cuda") for _ in range(3)]
    w, wp, wb = xt.workspace(xt.OP.ATTENTION, 1, prm, ins)
    xt.xt_op_bwd(xt.OP.ATTENTION, prm, xt.view(d), ins, [xt.view(out), xt.view(lse)],
                 [xt.view(g) for g in grads], 0, wp, wb)
    torch.cuda.synchronize()
    got = [host(g) for g in grads]
    refs, mags = check_all(out, lse, got, qv, kv, vv, dv, S, H, Dh, alpha, causal, dtype)
    # bitwise reproducible; accumulate adds onto what is there
    again = [torch.zeros_like(g) for g in grads]
    xt.xt_op_bwd(xt.OP.ATTENTION, prm, xt.view(d), ins, [xt.view(out), xt.view(lse)],
                 [xt.view(g) for g in again], 0, wp, wb)
    torch.cuda.synchronize()
    for a, b in zip(again, got):
        assert np.array_equal(host(a), b)
    xt.xt_op_bwd(xt.OP.ATTENTION, prm, xt.view(d), ins, [xt.view(out), xt.view(lse)],
                 [xt.view(g) for g in again], 0b111, wp, wb)
    torch.cuda.synchronize()
    for name, a, r, m in zip(("dq", "dk", "dv"), again, refs, mags[1:]):
        check(host(a), 2 * r, dtype, 2 * m, S, ("accumulated", name))
    del w


def test_attention_validation():
    R, S, Dh = 64, 32, 48
    t = torch.zeros((R, 2 * Dh), dtype=torch.float32, device="cuda")
    lse = torch.zeros((R, 2), dtype=torch.float32, device="cuda")
    with pytest.raises(xt.XtError) as e:
        xt.xt_op_fwd(xt.OP.ATTENTION, xt.params(seq_len=S, head_dim=Dh), [xt.view(t)] * 3,
                     [xt.view(t), xt.view(lse)])
    assert e.value.status == 4                          # head_dim 48 not built
    with pytest.raises(xt.XtError) as e:
        xt.xt_op_fwd(xt.OP.ATTENTION, xt.params(seq_len=30, head_dim=32), [xt.view(t)] * 3,
                     [xt.view(t), xt.view(lse)])
    assert e.value.status == 2                          # rows not a multiple of seq_len


def test_fused_attention_in_the_block_equals_the_composed_one():
    """The tiny block (batch 4, seq 256, d 256, 4 x 64 heads, f32) with the
    fused op instead of the matmul / softmax composition."""
    from autograd_row_wise_amd import block as xb
    from oracle_block import block_loss
    shp = xb.BlockShape(B=4, S=256, H=4, Dh=64, hidden=688, vocab=4096)
    g = {}
    for kname, s in xb.WEIGHT_SHAPES(shp).items():
        g[kname] = np.ones(s, np.float32) if kname.startswith("g") else synth.host_normal(s, 0, kname, 0.0, 0.02)
    x0 = synth.host_normal((shp.B * shp.S, shp.D), 0, "x")
    t0 = synth.host_uniform_int((shp.B * shp.S,), 0, shp.vocab, 0, "targets")
    res = {}
    for fused in (False, True):
        W = {kname: dev(val) for kname, val in g.items()}
        x, tt = dev(x0), dev(t0.reshape(-1, 1), "i32")
        tp = xt.Tape()
        w = xb.leaves(tp, W)
        vx = tp.leaf(xt.view(x))
        loss = xb.block(tp, w, vx, tp.leaf(xt.view(tt), requires_grad=False), shp, xt.DT.F32,
                        fused_attention=fused)
        tp.backward(loss)
        torch.cuda.synchronize()
        res[fused] = (host(xt.to_torch(tp.value(loss)))[0, 0],
                      {kname: host(xt.to_torch(tp.grad(vv))) for kname, vv in w.items()})
        tp.close()
    o, P, ox, ol = block_loss({kname: val.astype(np.float64) for kname, val in g.items()}, x0.astype(np.float64),
                              t0, shp.B, shp.S, shp.H, shp.Dh, 0.0, 0)
    o.backward(ol)
    L = float(o.value(ol)[0])
    for fused in (False, True):
        Lg, grads = res[fused]
        assert abs(Lg - L) <= 1e-6 + 1e-5 * abs(L)
        for kname in P:
            r = o.grad(P[kname]).reshape(grads[kname].shape)
            close_chain_f32(grads[kname], r, what=f"{'fused' if fused else 'composed'} {kname}")


def test_attention_bf16_unaligned_rows():
    """Row stride C + 4 (not a multiple of 8 elements): the bf16 op takes the
    generic kernels; same bar as the aligned cases."""
    B, S, H, Dh = 1, 70, 2, 32
    R, C, ld = B * S, H * Dh, H * Dh + 4
    alpha = 1.0 / math.sqrt(Dh)

    def padded(a):
        bits = synth.host_bf16_bits(a)
        full = np.zeros((R, ld), np.uint16)
        full[:, :C] = bits
        return dev(full, "bf16")[:, :C], synth.bf16_bits_to_f32(bits).astype(np.float64)

    (q, qv), (k, kv), (v, vv), (d, dv) = (padded(synth.host_normal((R, C), 13, n)) for n in ("q", "k", "v", "dout"))
    prm = xt.params(alpha=alpha, causal=1, seq_len=S, head_dim=Dh)
    out = torch.empty((R, ld), dtype=torch.bfloat16, device="cuda")[:, :C]
    lse = torch.empty((R, H), dtype=torch.float32, device="cuda")
    ins = [xt.view(q), xt.view(k), xt.view(v)]
    xt.xt_op_fwd(xt.OP.ATTENTION, prm, ins, [xt.view(out), xt.view(lse)])
    grads = [torch.empty((R, ld), dtype=torch.bfloat16, device="cuda")[:, :C] for _ in range(3)]
    w, wp, wb = xt.workspace(xt.OP.ATTENTION, 1, prm, ins)
    xt.xt_op_bwd(xt.OP.ATTENTION, prm, xt.view(d), ins, [xt.view(out), xt.view(lse)],
                 [xt.view(g) for g in grads], 0, wp, wb)
    torch.cuda.synchronize()
    check_all(out, lse, grads, qv, kv, vv, dv, S, H, Dh, alpha, True, "bf16", "unaligned")
    del w


def test_attention_bench_shape_two_heads():
    """The 2 x 2048 tokens, 16 heads x 128, causal, bf16 workload run whole
    (its 256 (heaviest, lightest) pairs of 128-key blocks fill a 256-CU
    MI355X, so the dK / dV pass runs its paired grid); heads (sequence 0,
    head 3) and (sequence 1, head 12) checked in full against the oracle on
    those heads alone."""
    B, S, H, Dh = 2, 2048, 16, 128
    R, C = B * S, H * Dh
    alpha = 1.0 / math.sqrt(Dh)
    x = {n: synth.device_normal((R, C), 14, n, dtype="bf16") for n in ("q", "k", "v", "dout")}
    prm = xt.params(alpha=alpha, causal=1, seq_len=S, head_dim=Dh)
    out = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((R, H), dtype=torch.float32, device="cuda")
    ins = [xt.view(x["q"]), xt.view(x["k"]), xt.view(x["v"])]
    xt.xt_op_fwd(xt.OP.ATTENTION, prm, ins, [xt.view(out), xt.view(lse)])
    grads = [torch.empty((R, C), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    w, wp, wb = xt.workspace(xt.OP.ATTENTION, 1, prm, ins)
    xt.xt_op_bwd(xt.OP.ATTENTION, prm, xt.view(x["dout"]), ins, [xt.view(out), xt.view(lse)],
                 [xt.view(g) for g in grads], 0, wp, wb)
    torch.cuda.synchronize()
    for b, hd in ((0, 3), (1, 12)):
        rows, cols = slice(b * S, (b + 1) * S), slice(hd * Dh, (hd + 1) * Dh)
        sl = {n: host(t[rows, cols]) for n, t in x.items()}
        check_all(out[rows, cols], lse[rows, hd:hd + 1], [host(g[rows, cols]) for g in grads], sl["q"], sl["k"],
                  sl["v"], sl["dout"], S, 1, Dh, alpha, True, "bf16", (b, hd))
    del w


def test_attention_causal_paired_key_blocks_odd_ragged():
    """2 x 1900 tokens, 16 heads x 128, causal, bf16: 15 key blocks per
    (sequence, head), the last one ragged (108 keys).  Their 8 pairs per
    (sequence, head), 256 in all, fill a 256-CU MI355X, so the dK / dV pass
    runs its paired grid, the middle block of each head on its own; the dQ
    pass keeps its unpaired grid.  Heads (sequence 0, head 2) and
    (sequence 1, head 9) checked in full against the oracle."""
    B, S, H, Dh = 2, 1900, 16, 128
    R, C = B * S, H * Dh
    alpha = 1.0 / math.sqrt(Dh)
    x = {n: synth.device_normal((R, C), 16, n, dtype="bf16") for n in ("q", "k", "v", "dout")}
    prm = xt.params(alpha=alpha, causal=1, seq_len=S, head_dim=Dh)
    out = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((R, H), dtype=torch.float32, device="cuda")
    ins = [xt.view(x["q"]), xt.view(x["k"]), xt.view(x["v"])]
    xt.xt_op_fwd(xt.OP.ATTENTION, prm, ins, [xt.view(out), xt.view(lse)])
    grads = [torch.empty((R, C), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    w, wp, wb = xt.workspace(xt.OP.ATTENTION, 1, prm, ins)
    xt.xt_op_bwd(xt.OP.ATTENTION, prm, xt.view(x["dout"]), ins, [xt.view(out), xt.view(lse)],
                 [xt.view(g) for g in grads], 0, wp, wb)
    torch.cuda.synchronize()
    for b, hd in ((0, 2), (1, 9)):
        rows, cols = slice(b * S, (b + 1) * S), slice(hd * Dh, (hd + 1) * Dh)
        sl = {n: host(t[rows, cols]) for n, t in x.items()}
        check_all(out[rows, cols], lse[rows, hd:hd + 1], [host(g[rows, cols]) for g in grads], sl["q"], sl["k"],
                  sl["v"], sl["dout"], S, 1, Dh, alpha, True, "bf16", (b, hd))
    del w


def test_attention_causal_paired_query_blocks():
    """2 x 4096 tokens, 16 heads x 128, causal, bf16: 512 (heaviest,
    lightest) pairs of 128-query blocks, two per CU on a 256-CU MI355X, so
    the forward, the dQ pass and the dK / dV pass run their paired grids.  Heads (sequence 0,
    head 5) and (sequence 1, head 14) checked in full against the oracle:
    output, log-sum-exp and the three gradients."""
    B, S, H, Dh = 2, 4096, 16, 128
    R, C = B * S, H * Dh
    alpha = 1.0 / math.sqrt(Dh)
    x = {n: synth.device_normal((R, C), 15, n, dtype="bf16") for n in ("q", "k", "v", "dout")}
    prm = xt.params(alpha=alpha, causal=1, seq_len=S, head_dim=Dh)
    out = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((R, H), dtype=torch.float32, device="cuda")
    ins = [xt.view(x["q"]), xt.view(x["k"]), xt.view(x["v"])]
    xt.xt_op_fwd(xt.OP.ATTENTION, prm, ins, [xt.view(out), xt.view(lse)])
    grads = [torch.empty((R, C), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    w, wp, wb = xt.workspace(xt.OP.ATTENTION, 1, prm, ins)
    xt.xt_op_bwd(xt.OP.ATTENTION, prm, xt.view(x["dout"]), ins, [xt.view(out), xt.view(lse)],
                 [xt.view(g) for g in grads], 0, wp, wb)
    torch.cuda.synchronize()
    for b, hd in ((0, 5), (1, 14)):
        rows, cols = slice(b * S, (b + 1) * S), slice(hd * Dh, (hd + 1) * Dh)
        sl = {n: host(t[rows, cols]) for n, t in x.items()}
        check_all(out[rows, cols], lse[rows, hd:hd + 1], [host(g[rows, cols]) for g in grads], sl["q"], sl["k"],
                  sl["v"], sl["dout"], S, 1, Dh, alpha, True, "bf16", (b, hd))
    del w
