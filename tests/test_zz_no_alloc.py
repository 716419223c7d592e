"""xt_op_bwd_noalloc through the C ABI against xt_op_bwd with a caller
workspace: the same kernels on the same plan, so the outputs must agree bit
for bit (which is within every tolerance of the parity tests).  Each case
runs two calls in a row on the shared static array, the second on a smaller
input, so a stale first-call workspace would show; a backward whose
workspace exceeds the array is rejected before any launch."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

try:
    import torch
    import autograd_row_wise_amd as xt
    from xt_testutil import dev, host
except Exception:  # pragma: no cover - CPU host without the library
    pass


def normal(shape, seed, name, dtype="f32", mean=0.0, std=1.0):
    a = synth.host_normal(shape, seed, name, mean, std, "f32")
    return dev(synth.host_bf16_bits(a), "bf16") if dtype == "bf16" else dev(a)


def both(op, prm, dout, ins, saved, make_din, acc=0):
    """Runs the backward through xt_op_bwd (caller workspace) and through
    xt_op_bwd_noalloc; returns the two lists of gradients as host arrays."""
    iv = [xt.view(t) for t in ins]
    sv = [xt.view(t) for t in saved]
    res = []
    for noalloc in (False, True):
        din = make_din()
        dv = [xt.view(t) if t is not None else xt.empty_view(ins[k]) for k, t in enumerate(din)]
        if noalloc:
            xt.xt_op_bwd_noalloc(op, prm, xt.view(dout), iv, sv, dv, acc)
        else:
            w, wp, wb = xt.workspace(op, 1, prm, iv)
            xt.xt_op_bwd(op, prm, xt.view(dout), iv, sv, dv, acc, wp, wb)
        torch.cuda.synchronize()
        res.append([host(t) if t is not None else None for t in din])
        if not noalloc:
            del w
    return res


def same(a, b, what):
    for k, (x, y) in enumerate(zip(a, b)):
        if x is None:
            continue
        assert np.array_equal(x, y), (what, k, float(np.max(np.abs(x - y))))


@pytest.mark.parametrize("shapes", [((300, 1000), (77, 640))])
def test_layer_norm_f32(shapes):
    for i, (R, C) in enumerate(shapes):
        x, d = normal((R, C), 40 + i, "x"), normal((R, C), 40 + i, "dout")
        g, b = normal((C,), 40 + i, "gamma", mean=1.0, std=0.1), normal((C,), 40 + i, "beta", std=0.1)
        y, mu, rs = (torch.empty((R, C), device="cuda"), torch.empty((R, 1), device="cuda"),
                     torch.empty((R, 1), device="cuda"))
        prm = xt.params(eps=1e-5)
        xt.xt_op_fwd(xt.OP.LAYER_NORM, prm, [xt.view(t) for t in (x, g, b)], [xt.view(t) for t in (y, mu, rs)])
        ref, got = both(xt.OP.LAYER_NORM, prm, d, [x, g, b], [mu, rs],
                        lambda: [torch.empty((R, C), device="cuda"), torch.empty((C,), device="cuda"),
                                 torch.empty((C,), device="cuda")])
        same(ref, got, ("layer_norm", R, C))


@pytest.mark.parametrize("shapes", [((512, 4096), (33, 1024))])
def test_rms_norm_bf16(shapes):
    for i, (R, C) in enumerate(shapes):
        x, d = normal((R, C), 50 + i, "x", "bf16"), normal((R, C), 50 + i, "dout", "bf16")
        g = normal((C,), 50 + i, "gamma", mean=1.0, std=0.1)
        y, ir = torch.empty((R, C), dtype=torch.bfloat16, device="cuda"), torch.empty((R, 1), device="cuda")
        prm = xt.params(eps=1e-5)
        xt.xt_op_fwd(xt.OP.RMS_NORM, prm, [xt.view(x), xt.view(g)], [xt.view(y), xt.view(ir)])
        # the second pair accumulates into dx and dgamma
        acc = 0b11 if i else 0
        ref, got = both(xt.OP.RMS_NORM, prm, d, [x, g], [ir],
                        lambda: [torch.ones((R, C), dtype=torch.bfloat16, device="cuda"),
                                 torch.ones((C,), device="cuda")], acc)
        same(ref, got, ("rms_norm", R, C))


def test_add_bias_dbias():
    for i, (R, C) in enumerate(((1000, 768), (10, 96))):
        x, d = normal((R, C), 60 + i, "x"), normal((R, C), 60 + i, "dout")
        bias = normal((C,), 60 + i, "bias")
        ref, got = both(xt.OP.ADD_BIAS, xt.params(), d, [x, bias], [],
                        lambda: [None, torch.empty((C,), device="cuda")])
        same(ref, got, ("add_bias", R, C))


def test_matmul_split_k():
    # few output tiles and a long contraction: the weight gradient is split
    # along K into f32 partials in the workspace
    for i, (M, K, N) in enumerate(((8192, 256, 384), (2048, 96, 128))):
        A, B, D = normal((M, K), 70 + i, "a"), normal((K, N), 70 + i, "b", std=0.02), normal((M, N), 70 + i, "dout")
        prm = xt.params()
        assert xt.xt_workspace_bytes(xt.OP.MATMUL, 1, prm, [xt.view(A), xt.view(B)]) <= 32 << 20
        ref, got = both(xt.OP.MATMUL, prm, D, [A, B], [],
                        lambda: [torch.empty((M, K), device="cuda"), torch.empty((K, N), device="cuda")])
        same(ref, got, ("matmul", M, K, N))


def test_attention_bf16():
    for i, (B, S, H, Dh) in enumerate(((2, 256, 2, 64), (1, 64, 1, 64))):
        R, C = B * S, H * Dh
        q, k, v, d = (normal((R, C), 80 + i, n, "bf16") for n in ("q", "k", "v", "dout"))
        prm = xt.params(alpha=Dh ** -0.5, causal=1, seq_len=S, head_dim=Dh)
        out = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((R, H), device="cuda")
        xt.xt_op_fwd(xt.OP.ATTENTION, prm, [xt.view(t) for t in (q, k, v)], [xt.view(out), xt.view(lse)])
        ref, got = both(xt.OP.ATTENTION, prm, d, [q, k, v], [out, lse],
                        lambda: [torch.empty((R, C), dtype=torch.bfloat16, device="cuda") for _ in range(3)])
        same(ref, got, ("attention", B, S, H, Dh))


def test_oversized_workspace_is_rejected():
    # 512 rows of 32768 f32 on the streaming backward: 256 partial rows of
    # dgamma | dbeta = 64 MiB > 32 MiB
    R, C = 512, 32768
    x, d, dx = (torch.zeros((R, C), device="cuda") for _ in range(3))
    g, b, dg, db = (torch.zeros((C,), device="cuda") for _ in range(4))
    mu, rs = torch.zeros((R, 1), device="cuda"), torch.ones((R, 1), device="cuda")
    prm = xt.params(eps=1e-5)
    ins = [xt.view(t) for t in (x, g, b)]
    assert xt.xt_workspace_bytes(xt.OP.LAYER_NORM, 1, prm, ins) > 32 << 20
    dg.fill_(7.0)
    torch.cuda.synchronize()
    with pytest.raises(xt.XtError) as e:
        xt.xt_op_bwd_noalloc(xt.OP.LAYER_NORM, prm, xt.view(d), ins, [xt.view(mu), xt.view(rs)],
                             [xt.view(dx), xt.view(dg), xt.view(db)])
    assert e.value.status == 5 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(dg == 7.0)                       # nothing was launched
