"""GPU parity of the token embedding (XT_OP_EMBED) through the C ABI against
the oracle: the gather (bit-exact, NaN rows for ids outside the table), the
deterministic scatter-add backward (Zipf-distributed ids with long runs,
uniform ids, several 16384-row chunks, accumulate mode, bf16, strided views,
bitwise reproducibility), the GPT-2-small shape (8192 tokens, 50257 x 768),
and a tied embedding / output projection on the tape."""
import numpy as np
import pytest

from oracle import ops
from oracle.tape import Tape as OTape
import synth

pytestmark = pytest.mark.gpu

if True:  # GPU-only imports are deferred so CPU collection never loads libxt
    try:
        import torch
        import autograd_row_wise_amd as xt
        from xt_testutil import close, close_chain_f32, close_f32, dev, host, sum_scale
    except Exception:  # pragma: no cover - CPU host without the library
        pass


def put(a, dtype, ld=None):
    R, C = a.shape
    bits = synth.host_bf16_bits(a) if dtype == "bf16" else a.astype(np.float32)
    vals = synth.bf16_bits_to_f32(bits).astype(np.float64) if dtype == "bf16" else bits.astype(np.float64)
    if ld is None:
        return dev(bits, dtype), vals
    pad = np.zeros((R, ld), dtype=bits.dtype)
    pad[:, :C] = bits
    return dev(pad, dtype)[:, :C], vals


def run_fwd(E, ids_t, R, D, dtype, ld=None):
    y = (torch.empty((R, ld if ld else D), dtype=E.dtype, device="cuda"))[:, :D]
    xt.xt_op_fwd(xt.OP.EMBED, xt.params(), [xt.view(E), xt.view(ids_t)], [xt.view(y)])
    torch.cuda.synchronize()
    return y


def run_bwd(E, ids_t, d, dE, acc=0):
    ins = [xt.view(E), xt.view(ids_t)]
    w, wp, wb = xt.workspace(xt.OP.EMBED, 1, xt.params(), ins)
    slot = xt.view(ids_t)
    slot.data = None
    xt.xt_op_bwd(xt.OP.EMBED, xt.params(), xt.view(d), ins, [], [xt.view(dE), slot], acc, wp, wb)
    torch.cuda.synchronize()
    del w


def check_dE(got, ref, d_vals, ids, V, dtype):
    """Each dE row is a sum of the d rows with its id: the f32 bar with the
    long-sum floor (A = sum of |terms|, n = the run length)."""
    if dtype == "bf16":
        close(got, ref, "bf16", what="dE")
        return
    A = ops.embed_bwd(np.abs(d_vals), ids, V)
    n = np.maximum(np.bincount(ids[(ids >= 0) & (ids < V)], minlength=V), 1)[:, None]
    close_f32(got, ref, scale=sum_scale(A, 1) / np.sqrt(n), what="dE")


CASES = [  # V, D, R, dtype, ld_E, ids kind
    (11, 13, 40, "f32", None, "uniform"),
    (997, 1001, 3000, "f32", 1008, "zipf"),
    (997, 256, 3000, "bf16", None, "zipf"),
    (50, 8, 40000, "f32", None, "zipf"),          # five merge rounds, runs of thousands of rows
    (4096, 64, 20000, "bf16", 72, "uniform"),
]


@pytest.mark.parametrize("V,D,R,dtype,ld,kind", CASES)
def test_embed_fwd_bwd(V, D, R, dtype, ld, kind):
    E, Ev = put(synth.host_normal((V, D), 0, "emb"), dtype, ld)
    if kind == "zipf":
        ids = synth.host_zipf_int((R,), V, 1.1, 0, "ids")
    else:
        ids = synth.host_uniform_int((R,), 0, V, 0, "ids")
    ids_t = dev(ids.reshape(-1, 1), "i32")
    y = run_fwd(E, ids_t, R, D, dtype)
    assert np.array_equal(host(y), ops.embed(Ev, ids))
    d, dv = put(synth.host_normal((R, D), 0, "dout"), dtype)
    dE = (torch.empty((V, ld if ld else D), dtype=E.dtype, device="cuda"))[:, :D]
    dE.fill_(float("nan"))                   # every row must be written
    run_bwd(E, ids_t, d, dE)
    got = host(dE)
    ref = ops.embed_bwd(dv, ids, V)
    check_dE(got, ref, dv, ids, V, dtype)
    # bitwise reproducible, and accumulate adds onto what is there
    dE2 = torch.zeros_like(dE)
    run_bwd(E, ids_t, d, dE2)
    assert np.array_equal(host(dE2), got)
    run_bwd(E, ids_t, d, dE2, acc=1)
    got2 = host(dE2)
    if dtype == "f32":
        check_dE(got2, 2 * ref, 2 * dv, ids, V, dtype)
    else:
        close(got2, 2 * ref, "bf16", what="dE accumulated")


def test_embed_out_of_range_ids():
    V, D = 6, 5
    E, Ev = put(synth.host_normal((V, D), 1, "emb"), "f32")
    ids = np.array([0, 6, -1, 5, 2, 100], np.int32)
    ids_t = dev(ids.reshape(-1, 1), "i32")
    y = host(run_fwd(E, ids_t, len(ids), D, "f32"))
    assert np.all(np.isnan(y[[1, 2, 5]])) and np.array_equal(y[[0, 3, 4]], Ev[[0, 5, 2]])
    d, dv = put(synth.host_normal((len(ids), D), 1, "dout"), "f32")
    dE = torch.empty((V, D), dtype=torch.float32, device="cuda")
    run_bwd(E, ids_t, d, dE)
    np.testing.assert_array_equal(host(dE), ops.embed_bwd(dv, ids, V))


def test_gpt2_small_embedding():
    """8 x 1024 Zipf-distributed tokens into the 50257 x 768 f32 table."""
    V, D, R = 50257, 768, 8192
    E = synth.device_normal((V, D), 9, "emb", 0.0, 0.02)
    ids = synth.host_zipf_int((R,), V, 1.1, 9, "ids")
    ids_t = dev(ids.reshape(-1, 1), "i32")
    Ev = host(E)
    y = run_fwd(E, ids_t, R, D, "f32")
    assert np.array_equal(host(y), ops.embed(Ev, ids))
    d = synth.device_normal((R, D), 9, "dout")
    dE = torch.empty((V, D), dtype=torch.float32, device="cuda")
    run_bwd(E, ids_t, d, dE)
    dv = host(d)
    check_dE(host(dE), ops.embed_bwd(dv, ids, V), dv, ids, V, "f32")


def test_tied_embedding_on_the_tape():
    """x = embed(E, ids); logits = rms_norm(x) @ E^T; loss = CE: E receives
    the gather's scatter-add and the projection's dB, summed by the tape."""
    V, D, R = 37, 16, 50
    E0 = synth.host_normal((V, D), 3, "emb", 0.0, 0.5)
    g0 = np.ones((D,), np.float32)
    ids = synth.host_zipf_int((R,), V, 1.2, 3, "ids")
    tgt = synth.host_uniform_int((R,), 0, V, 3, "targets")
    E, g = dev(E0), dev(g0)
    ids_t, tg_t = dev(ids.reshape(-1, 1), "i32"), dev(tgt.reshape(-1, 1), "i32")
    t = xt.Tape()
    vE, vg = t.leaf(xt.view(E)), t.leaf(xt.view(g))
    vi, vt = t.leaf(xt.view(ids_t), requires_grad=False), t.leaf(xt.view(tg_t), requires_grad=False)
    x = t.apply(xt.OP.EMBED, xt.params(), vE, vi)
    h = t.apply(xt.OP.RMS_NORM, xt.params(eps=1e-5), x, vg)
    logits = t.apply(xt.OP.MATMUL, xt.params(trans_b=1), h, vE)
    loss = t.apply(xt.OP.CROSS_ENTROPY, xt.params(), logits, vt)
    t.backward(loss)
    torch.cuda.synchronize()
    o = OTape()
    oE, og = o.leaf(E0.astype(np.float64)), o.leaf(g0.astype(np.float64))
    ox = o.embed(oE, ids)
    oh = o.rms_norm(ox, og, 1e-5)
    ol = o.cross_entropy(o.matmul(oh, oE, trans_b=True), tgt)
    o.backward(ol)
    gE = host(xt.to_torch(t.grad(vE)))
    close_chain_f32(gE, o.grad(oE), what="tied embedding dE")
    Lg = host(xt.to_torch(t.value(loss)))[0, 0]
    assert abs(Lg - float(o.value(ol)[0])) <= 1e-5 * abs(Lg)
    t.close()
