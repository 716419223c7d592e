"""GPU parity at the full workload sizes, through the same C-ABI calls the
bench times.  Inputs come from the seeded device generator (the same draws
as the bench); the oracle recomputes sampled rows / entries from copies of
those inputs, and properties that hold at any size are checked on whole
tensors (dropout masks bit-exact everywhere, column sums in full, the mean
loss equal to the mean of the per-row losses)."""
import gc

import numpy as np
import pytest

from oracle import ops, rng
from oracle.numerics import round_bf16

pytestmark = pytest.mark.gpu

try:
    import torch
    import autograd_row_wise_amd as xt
    from synth import device_normal, device_uniform_int
    from xt_testutil import close, close_f32, close_bf16, host, sum_scale
except Exception:  # pragma: no cover
    pass

V, P = (lambda *a, **k: xt.view(*a, **k)), (lambda **k: xt.params(**k))


@pytest.fixture(autouse=True)
def _free():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def empty(shape, dt):
    return torch.empty(shape, dtype={"f32": torch.float32, "bf16": torch.bfloat16, "u8": torch.uint8}[dt], device="cuda")


def sample_rows(R, n=24, seed=0):
    g = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, R - 1], g.integers(0, R, n)]))


def bwd(op, prm, dout, ins, saved, din, acc=0):
    iv = [V(t) for t in ins]
    dv = []
    for k, t in enumerate(din):
        v = V(t if t is not None else ins[k])
        if t is None:
            v.data = None
        dv.append(v)
    n = xt.xt_workspace_bytes(op, 1, prm, iv)
    w = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
    xt.xt_op_bwd(op, prm, V(dout), iv, [V(t) for t in saved], dv, acc, w.data_ptr() if n else None, n)
    torch.cuda.synchronize()


def fwd(op, prm, ins, outs):
    xt.xt_op_fwd(op, prm, [V(t) for t in ins], [V(t) for t in outs])
    torch.cuda.synchronize()


# ----------------------------------------------------- GPT-2-small f32 shapes
def test_c3_layer_norm_full():
    R, C = 8192, 768
    x, d = device_normal((R, C), 3, "x"), device_normal((R, C), 3, "dout")
    g, b = device_normal((C,), 3, "gamma", 1.0, 0.1), device_normal((C,), 3, "beta", 0.0, 0.1)
    y, mu, rs = empty((R, C), "f32"), empty((R, 1), "f32"), empty((R, 1), "f32")
    fwd(xt.OP.LAYER_NORM, P(eps=1e-5), [x, g, b], [y, mu, rs])
    dx, dg, db = empty((R, C), "f32"), empty((C,), "f32"), empty((C,), "f32")
    bwd(xt.OP.LAYER_NORM, P(eps=1e-5), d, [x, g, b], [mu, rs], [dx, dg, db])
    xv, dv, gv, bv = host(x), host(d), host(g), host(b)
    y_ref, mu_ref, rs_ref = ops.layer_norm(xv, gv, bv, 1e-5)
    dx_ref, dg_ref, db_ref = ops.layer_norm_bwd(dv, xv, gv, mu_ref, rs_ref)
    close_f32(host(y), y_ref, what="y")
    close_f32(host(rs)[:, 0], rs_ref, what="rstd")
    xhat = (xv - mu_ref[:, None]) * rs_ref[:, None]
    gg = dv * gv[None, :]
    scale = rs_ref[:, None] * (np.abs(gg) + np.mean(np.abs(gg), axis=1, keepdims=True)
                               + np.abs(xhat) * np.mean(np.abs(gg * xhat), axis=1, keepdims=True))
    close_f32(host(dx), dx_ref, sum_scale(scale, 3), what="dx")
    close_f32(host(dg), dg_ref, sum_scale(np.sum(np.abs(dv * xhat), axis=0), R), what="dgamma")
    close_f32(host(db), db_ref, sum_scale(np.sum(np.abs(dv), axis=0), R), what="dbeta")


def test_c3_gelu_and_residual_add_sampled():
    R, H = 8192, 3072
    h, d = device_normal((R, H), 3, "g"), device_normal((R, H), 3, "d2")
    y, dx = empty((R, H), "f32"), empty((R, H), "f32")
    fwd(xt.OP.GELU, P(), [h], [y])
    bwd(xt.OP.GELU, P(), d, [h], [], [dx])
    rows = sample_rows(R)
    hv, dv = host(h[rows]), host(d[rows])
    close_f32(host(y[rows]), ops.gelu(hv), what="gelu")
    close_f32(host(dx[rows]), ops.gelu_bwd(dv, hv), what="dgelu")
    a, b = device_normal((R, 768), 3, "x"), device_normal((R, 768), 3, "dout")
    s = empty((R, 768), "f32")
    fwd(xt.OP.ADD, P(), [a, b], [s])
    assert np.array_equal(host(s[rows]), (host(a[rows]) + host(b[rows])).astype(np.float32))


def test_c3_cross_entropy_sampled():
    R, Vv = 8192, 50257
    lg = device_normal((R, Vv), 3, "logits", 0.0, 2.0)
    tg = device_uniform_int((R, 1), 0, Vv, 3, "targets")
    L, lse, lr = empty((1, 1), "f32"), empty((R, 1), "f32"), empty((R, 1), "f32")
    fwd(xt.OP.CROSS_ENTROPY, P(), [lg, tg], [L, lse, lr])
    dL = torch.ones((1, 1), dtype=torch.float32, device="cuda")
    dx = empty((R, Vv), "f32")
    bwd(xt.OP.CROSS_ENTROPY, P(), dL, [lg, tg], [lse], [dx, None])
    rows = sample_rows(R, 16)
    xv, tv = host(lg[rows]), host(tg[rows])[:, 0]
    L_s, lse_ref, lr_ref = ops.cross_entropy(xv, tv)
    close_f32(host(lse[rows])[:, 0], lse_ref, what="lse")
    close_f32(host(lr[rows])[:, 0], lr_ref, what="loss_row")
    # dlogits of a row of the full batch: (p - onehot) * g / R with R = 8192
    close_f32(host(dx[rows]), ops.cross_entropy_bwd(1.0, xv, tv, lse_ref) * len(rows) / R, what="dlogits")
    # the mean loss is the fixed-order mean of the per-row losses
    close_f32(host(L)[0, 0], float(np.mean(host(lr)[:, 0])), what="L")


@pytest.mark.parametrize("which", ["mlp1", "mlp2"])
def test_c3_mlp_gemms_sampled(which):
    R, D, H = 8192, 768, 3072
    if which == "mlp1":
        A, B, Dg = device_normal((R, D), 3, "x"), device_normal((D, H), 3, "w1", 0.0, 0.02), device_normal((R, H), 3, "d2")
    else:
        A, B, Dg = device_normal((R, H), 3, "g"), device_normal((H, D), 3, "w2", 0.0, 0.02), device_normal((R, D), 3, "dout")
    M, K = A.shape
    N = B.shape[1]
    C = empty((M, N), "f32")
    fwd(xt.OP.MATMUL, P(), [A, B], [C])
    dA, dB = empty((M, K), "f32"), empty((K, N), "f32")
    bwd(xt.OP.MATMUL, P(), Dg, [A, B], [], [dA, dB])
    g = np.random.default_rng(1)
    ri, ci = np.unique(g.integers(0, M, 64)), np.unique(g.integers(0, N, 64))
    Ah, Bh = host(A), host(B)
    Ar, Dr, Dc = Ah[ri], host(Dg[ri]), host(Dg[:, ci])
    # sampled rows of C = A B and of dA = d B^T, sampled columns of dB = A^T d,
    # each from the oracle's matmul / matmul_bwd on the sampled slices
    close_f32(host(C[ri]), ops.matmul(Ar, Bh), sum_scale(ops.matmul(np.abs(Ar), np.abs(Bh)), K), what="C rows")
    dA_ref = ops.matmul_bwd(Dr, Ar, Bh)[0]
    close_f32(host(dA[ri]), dA_ref, sum_scale(ops.matmul(np.abs(Dr), np.abs(Bh), trans_b=True), N), what="dA rows")
    dB_ref = ops.matmul_bwd(Dc, Ah, Bh[:, ci])[1]
    close_f32(host(dB[:, ci]), dB_ref, sum_scale(ops.matmul(np.abs(Ah), np.abs(Dc), trans_a=True), M),
              what="dB columns")


# ----------------------------------------------------- bf16 16384 x 4096
def test_c4_rms_norm_full_dgamma():
    R, C = 16384, 4096
    x, d = device_normal((R, C), 4, "x", dtype="bf16"), device_normal((R, C), 4, "dout", dtype="bf16")
    g = device_normal((C,), 4, "gamma", 1.0, 0.1)
    y, ir = empty((R, C), "bf16"), empty((R, 1), "f32")
    fwd(xt.OP.RMS_NORM, P(eps=1e-5), [x, g], [y, ir])
    dx, dg = empty((R, C), "bf16"), empty((C,), "f32")
    bwd(xt.OP.RMS_NORM, P(eps=1e-5), d, [x, g], [ir], [dx, dg])
    gv = host(g)
    rows = sample_rows(R)
    xv, dv = host(x[rows]), host(d[rows])
    y_ref, ir_ref = ops.rms_norm(xv, gv, 1e-5)
    close_bf16(host(y[rows]), y_ref, what="y")
    close_f32(host(ir[rows])[:, 0], ir_ref, what="inv_rms")
    close_bf16(host(dx[rows]), ops.rms_norm_bwd(dv, xv, gv, ir_ref)[0], what="dx")
    # dgamma over all 16384 rows, oracle in chunks
    acc = np.zeros(C)
    A = np.zeros(C)
    for r0 in range(0, R, 2048):
        xc, dc = host(x[r0:r0 + 2048]), host(d[r0:r0 + 2048])
        _, irc = ops.rms_norm(xc, gv, 1e-5)
        acc += ops.rms_norm_bwd(dc, xc, gv, irc)[1]          # the oracle's dgamma of this chunk
        A += np.abs(dc * xc * irc[:, None]).sum(axis=0)      # magnitude of its terms (tolerance only)
    close_f32(host(dg), acc, sum_scale(A, R), what="dgamma")


def test_c4_swiglu_rope_accumulate_sampled():
    R, D, F = 16384, 4096, 11008
    rows = sample_rows(R)
    gg, u, d = (device_normal((R, F), 4, s, dtype="bf16") for s in ("g", "u", "d2"))
    y, dg, du = empty((R, F), "bf16"), empty((R, F), "bf16"), empty((R, F), "bf16")
    fwd(xt.OP.SWIGLU, P(), [gg, u], [y])
    bwd(xt.OP.SWIGLU, P(), d, [gg, u], [], [dg, du])
    gv, uv, dv = host(gg[rows]), host(u[rows]), host(d[rows])
    close_bf16(host(y[rows]), ops.swiglu(gv, uv), what="swiglu")
    rg, ru = ops.swiglu_bwd(dv, gv, uv)
    close_bf16(host(dg[rows]), rg, what="dg")
    close_bf16(host(du[rows]), ru, what="du")
    del gg, u, d, y, dg, du
    x, d = device_normal((R, D), 4, "x", dtype="bf16"), device_normal((R, D), 4, "dout", dtype="bf16")
    prm = P(head_dim=128, seq_len=4096, rope_base=10000.0)
    ry, rdx = empty((R, D), "bf16"), empty((R, D), "bf16")
    fwd(xt.OP.ROPE, prm, [x], [ry])
    bwd(xt.OP.ROPE, prm, d, [x], [], [rdx])
    xv, dv = host(x[rows]), host(d[rows])
    pos = rows % 4096
    close_bf16(host(ry[rows]), ops.rope(xv, 128, 10000.0, 4096, positions=pos), what="rope")
    close_bf16(host(rdx[rows]), ops.rope_bwd(dv, 128, 10000.0, 4096, positions=pos), what="rope bwd")
    dres = device_normal((R, D), 4, "resid", dtype="bf16")
    before = host(dres[rows])
    xt.xt_grad_accumulate(V(dres), V(d))
    torch.cuda.synchronize()
    assert np.array_equal(host(dres[rows]), round_bf16((before + dv).astype(np.float32)))


@pytest.mark.parametrize("site", [0xA77, 0xF70])
def test_c4_dropout_mask_bit_exact_everywhere(site):
    R, D = 16384, 4096
    seed = 42 ^ 0 ^ site
    x, d = device_normal((R, D), 4, "x", dtype="bf16"), device_normal((R, D), 4, "dout", dtype="bf16")
    y, m, dx = empty((R, D), "bf16"), empty((R, D), "u8"), empty((R, D), "bf16")
    fwd(xt.OP.DROPOUT, P(p=0.1, seed=seed), [x], [y, m])
    bwd(xt.OP.DROPOUT, P(p=0.1, seed=seed), d, [x], [m], [dx])
    got = m.cpu().numpy()
    for r0 in range(0, R, 4096):
        ref = rng.dropout_mask((4096, D), 0.1, seed, index_offset=r0 * D)
        assert np.array_equal(got[r0:r0 + 4096], ref), f"mask differs in rows {r0}..{r0 + 4096}"
    keep = got.mean()
    n = got.size
    kp = 1.0 - np.ceil(np.float32(0.1) * 2 ** 24) / 2 ** 24
    assert abs(keep - kp) < 5 * np.sqrt(kp * (1 - kp) / n)
    rows = sample_rows(R)
    s = rng.keep_scale(0.1)
    close_bf16(host(y[rows]), np.where(got[rows] == 1, host(x[rows]) * s, 0.0), what="y")
    close_bf16(host(dx[rows]), np.where(got[rows] == 1, host(d[rows]) * s, 0.0), what="dx")


# ----------------------------------------------------- bf16 stress shapes
def test_c5_cross_entropy_sampled():
    R, Vv = 32768, 128256
    lg = device_normal((R, Vv), 5, "logits", 0.0, 3.0, dtype="bf16")
    tg = device_uniform_int((R, 1), 0, Vv, 5, "targets")
    L, lse, lr = empty((1, 1), "f32"), empty((R, 1), "f32"), empty((R, 1), "f32")
    fwd(xt.OP.CROSS_ENTROPY, P(), [lg, tg], [L, lse, lr])
    dL = torch.ones((1, 1), dtype=torch.float32, device="cuda")
    dx = empty((R, Vv), "bf16")
    bwd(xt.OP.CROSS_ENTROPY, P(), dL, [lg, tg], [lse], [dx, None])
    rows = sample_rows(R, 8)
    xv, tv = host(lg[rows]), host(tg[rows])[:, 0]
    _, lse_ref, lr_ref = ops.cross_entropy(xv, tv)
    close_f32(host(lse[rows])[:, 0], lse_ref, what="lse")
    close_f32(host(lr[rows])[:, 0], lr_ref, what="loss_row")
    close_bf16(host(dx[rows]), ops.cross_entropy_bwd(1.0, xv, tv, lse_ref) * len(rows) / R, what="dlogits")
    close_f32(host(L)[0, 0], float(np.mean(host(lr)[:, 0])), what="L")


def test_c5_softmax_sampled():
    R = C = 32768
    x, d = device_normal((R, C), 5, "x", dtype="bf16"), device_normal((R, C), 5, "dout", dtype="bf16")
    y, dx = empty((R, C), "bf16"), empty((R, C), "bf16")
    fwd(xt.OP.SOFTMAX, P(), [x], [y])
    bwd(xt.OP.SOFTMAX, P(), d, [x], [y], [dx])
    rows = sample_rows(R, 8)
    xv, dv = host(x[rows]), host(d[rows])
    y_ref = ops.softmax(xv)
    close_bf16(host(y[rows]), y_ref, what="y")
    close_bf16(host(dx[rows]), ops.softmax_bwd(dv, round_bf16(y_ref)), what="dx")


def test_c5_dbias_full():
    R, C = 65536, 4096
    d = device_normal((R, C), 5, "d3", dtype="bf16")
    x = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    bias = torch.zeros((C,), dtype=torch.float32, device="cuda")
    db = empty((C,), "f32")
    bwd(xt.OP.ADD_BIAS, P(), d, [x, bias], [], [None, db])
    acc, A = np.zeros(C), np.zeros(C)
    for r0 in range(0, R, 4096):
        dc = host(d[r0:r0 + 4096])
        acc += ops.add_bias_bwd(dc)[1]
        A += np.abs(dc).sum(axis=0)
    close_f32(host(db), acc, sum_scale(A, R), what="dbias")


def test_c5_gemm_bwd_sampled():
    M, K, N = 8192, 4096, 4096
    A = device_normal((M, K), 5, "a", dtype="bf16")
    B = device_normal((K, N), 5, "b", 0.0, 0.02, dtype="bf16")
    Dg = device_normal((M, N), 5, "dout", dtype="bf16")
    dA, dB = empty((M, K), "bf16"), empty((K, N), "f32")
    bwd(xt.OP.MATMUL, P(), Dg, [A, B], [], [dA, None])
    bwd(xt.OP.MATMUL, P(), Dg, [A, B], [], [None, dB])
    g = np.random.default_rng(2)
    ri, ci = np.unique(g.integers(0, M, 96)), np.unique(g.integers(0, N, 96))
    Ah, Bh = host(A), host(B)
    Dr, Dc = host(Dg[ri]), host(Dg[:, ci])
    # sampled rows of dA = d B^T and sampled columns of dB = A^T d from the
    # oracle's matmul_bwd on the sampled slices
    close_bf16(host(dA[ri]), ops.matmul_bwd(Dr, Ah[ri], Bh)[0], what="dA rows")
    dB_ref = ops.matmul_bwd(Dc, Ah, Bh[:, ci])[1]
    close_f32(host(dB[:, ci]), dB_ref, sum_scale(ops.matmul(np.abs(Ah), np.abs(Dc), trans_a=True), M),
              what="dB columns")
