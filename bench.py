#!/usr/bin/env python3
"""Throughput of the row-wise autograd hot path on one MI355X.

One step = one forward+backward pass of every op of the hot path over one
batch of synthetic input, each at the shape its workload names:
  * GPT-2-small-shaped f32 (batch 8 x seq 1024, d 768): layer_norm, GELU
    MLP (hidden 3072: both GEMMs fwd+bwd and the GELU), residual add,
    cross-entropy over vocab 50257 (logits ~ N(0, 2));
  * bf16, 16384 rows x d 4096: rms_norm, SwiGLU gate/up 16384 x 11008, rope
    32 heads x 128, residual dropout p=0.1 at the two sites
    (seeds 42^0^0xA77, 42^0^0xF70), fan-out grad accumulate;
  * bf16 stress: cross-entropy 32768 x 128256 (logits ~ N(0, 3)), softmax
    32768 x 32768, dbias column sum over 65536 x 4096, matmul backward of
    8192 x 4096 x 4096;
  * the tiny transformer block (batch 4, seq 256, d 256, 4 x 64 heads,
    SwiGLU 688, vocab 4096, f32) recorded on the tape, fwd+bwd.
The ops that widen the path are timed after the step, in a loop of their
own, and reported under `next_rows` (not in `value`):
  * the global gradient norm and the clip scaling over every gradient
    buffer of a 12-layer model of GPT-2-small width (about 124M f32 in 124
    tensors);
  * the token embedding of the same model: 8 x 1024 Zipf(1.1)-distributed
    tokens into a 50257 x 768 f32 table, gather and scatter-add backward;
  * fused causal attention fwd+bwd: 2 x 2048 tokens, 16 heads x 128, bf16
    storage; and the tiny block with it in place of the composed attention;
  * the tiny block with its layer as one activation-recompute segment.
Inputs are drawn on the GPU before timing (torch's seeded generator).

`value` is the achieved HBM rate of the memory-bound part of the step: the
algorithmic bytes (what the method must read and write, not what the caches
move) of every memory-bound op fwd+bwd, divided by the wall time of one
graph replay of those ops (`ms_per_step`); `frac` = value / 8 TB/s.  The
whole step (with the GEMMs and the tape-driven block) is timed too
(`ms_per_full_step`).  The step's launches are captured once into a HIP
graph and replayed (the tape-driven block runs eagerly after it); each op's
time comes from a graph of that op launched
several times in a row, with HIP events around the replay, so the Python
launch path is not in the per-op figures (--eager times every launch from
Python instead).  An op whose bytes are below 1 GiB cycles through
independent copies of its buffers in that graph, so it never re-reads its
own data from the Infinity Cache; each figure is the median of the timed
replays.  Per-op figures (bytes, time, GB/s or TFLOP/s, fraction of
peak) are in `ops`; `roofline` is for the op with the largest share of step
time.  `c1_latency` is every op of the 8 x 64 f32 workload fwd and bwd in
microseconds per call (the launch floor).  `cpu_baseline` is the CPU oracle
on a bounded sample, on all host cores (at most 16) and on one core.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--only NAME ...] [--eager]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}

# HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE and
# WRITE_SIZE per dispatch, each scaled by the same counter's reading for a
# plain copy of known size).  A figure holds only for the kernel source it was
# measured on: the fingerprint of those files is checked at run time and the
# figure is dropped (traffic = null) once they have changed.
MEASURED_TRAFFIC = {
    "c5.ce.bwd": {"bytes": 16817274163, "sources": ["autograd_row_wise_amd/csrc/ce.hip",
                                                    "autograd_row_wise_amd/csrc/common.h"],
                  "sha256_16": "648fd5858341e740", "profile": "profiles/ce_bwd_bf16_32768x128256.md"},
}


def measured_traffic(op_name):
    import hashlib
    rec = MEASURED_TRAFFIC.get(op_name)
    if rec is None:
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return rec["bytes"] if h.hexdigest()[:16] == rec["sha256_16"] else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", nargs="*", default=None, help="run only ops whose name starts with one of these")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch every op from Python each step instead of replaying captured HIP graphs")
    ap.add_argument("--no-sweep", action="store_true", help="skip the rows/s sweep over d = 768..4096")
    ap.add_argument("--ops-json", default=None, help="also write the per-op table to this file")
    return ap.parse_args()


# --------------------------------------------------------------------------
class Entry:
    def __init__(self, name, workload, dtype, kind, fn, nbytes=0, flops=0, rows=0):
        self.name, self.workload, self.dtype, self.kind = name, workload, dtype, kind
        self.fn, self.bytes, self.flops, self.rows = fn, nbytes, flops, rows
        self.fns = [fn]          # the same op over independent buffer copies (see ROTATE_BYTES)
        self.times_ms = []


# A memory-bound op whose algorithmic bytes are below ROTATE_BYTES would, when
# launched many times in a row, find its own inputs (and absorb its own
# writes) in the 256 MB Infinity Cache and the L2s.  Such ops are built over
# ceil(ROTATE_BYTES / bytes) independent copies of their buffers (at most
# MAX_COPIES; same values), and the repeated launches cycle through the
# copies, so every launch streams from and to HBM as it would in a step.
ROTATE_BYTES = 1 << 30
MAX_COPIES = 8


def build_entries(only):
    import torch
    import autograd_row_wise_amd as xt
    from autograd_row_wise_amd import block as xb
    from synth import device_normal, device_uniform_int

    V, P = xt.view, xt.params
    E = []
    # a name is wanted when it and a requested prefix agree as far as both go
    # ("c4" selects every bf16 16384 x 4096 op; "c4.rope" only rope)
    want = (lambda n: True) if not only else (lambda n: any(n.startswith(o) or o.startswith(n) for o in only))

    def empty(shape, dt):
        return torch.empty(shape, dtype={"f32": torch.float32, "bf16": torch.bfloat16, "u8": torch.uint8}[dt],
                           device="cuda")

    def ws(op, prm, ins, is_bwd=1):
        n = xt.xt_workspace_bytes(op, is_bwd, prm, ins)
        if not n:
            return None, 0
        buf = torch.empty(n, dtype=torch.uint8, device="cuda")
        keep.append(buf)
        return buf.data_ptr(), n

    keep = []
    nullslot = lambda t: (lambda v: (setattr(v, "data", None), v)[1])(V(t))  # noqa: E731

    # Each workload is built in its own function so the op closures bind
    # that workload's tensors.
    def c3(want, E):
        nonlocal keep
        W3 = "gpt2s-f32 8x1024x768"
        R3, D3, H3, V3 = 8192, 768, 3072, 50257
        if any(want(n) for n in ("c3.ln", "c3.gelu", "c3.add", "c3.ce", "c3.mlp")):
            x = device_normal((R3, D3), 3, "x")
            d = device_normal((R3, D3), 3, "dout")
            gam = device_normal((D3,), 3, "gamma", 1.0, 0.1)
            bet = device_normal((D3,), 3, "beta", 0.0, 0.1)
            y, mu, rs = empty((R3, D3), "f32"), empty((R3, 1), "f32"), empty((R3, 1), "f32")
            dx, dg, db = empty((R3, D3), "f32"), empty((D3,), "f32"), empty((D3,), "f32")
            pln = P(eps=1e-5)
            keep += [x, d, gam, bet, y, mu, rs, dx, dg, db]
            N = R3 * D3
            if want("c3.ln"):
                E.append(Entry("c3.ln.fwd", W3, "f32", "hbm", lambda: xt.xt_op_fwd(
                    xt.OP.LAYER_NORM, pln, [V(x), V(gam), V(bet)], [V(y), V(mu), V(rs)]), 2 * 4 * N + 8 * R3, rows=R3))
                wp, wn = ws(xt.OP.LAYER_NORM, pln, [V(x), V(gam), V(bet)])
                E.append(Entry("c3.ln.bwd", W3, "f32", "hbm", lambda: xt.xt_op_bwd(
                    xt.OP.LAYER_NORM, pln, V(d), [V(x), V(gam), V(bet)], [V(mu), V(rs)], [V(dx), V(dg), V(db)], 0, wp, wn),
                    3 * 4 * N + 8 * R3, rows=R3))
            if want("c3.add"):
                r2 = empty((R3, D3), "f32")
                keep.append(r2)
                E.append(Entry("c3.add.fwd", W3, "f32", "hbm", lambda: xt.xt_op_fwd(
                    xt.OP.ADD, P(), [V(x), V(d)], [V(r2)]), 3 * 4 * N, rows=R3))
            if want("c3.gelu") or want("c3.mlp"):
                hpre = device_normal((R3, H3), 3, "g")
                hd = device_normal((R3, H3), 3, "d2")
                hy, hdx = empty((R3, H3), "f32"), empty((R3, H3), "f32")
                keep += [hpre, hd, hy, hdx]
                NH = R3 * H3
                if want("c3.gelu"):
                    E.append(Entry("c3.gelu.fwd", W3, "f32", "hbm", lambda: xt.xt_op_fwd(
                        xt.OP.GELU, P(), [V(hpre)], [V(hy)]), 2 * 4 * NH, rows=R3))
                    E.append(Entry("c3.gelu.bwd", W3, "f32", "hbm", lambda: xt.xt_op_bwd(
                        xt.OP.GELU, P(), V(hd), [V(hpre)], [], [V(hdx)]), 3 * 4 * NH, rows=R3))
                if want("c3.mlp"):
                    w1 = device_normal((D3, H3), 3, "w1", 0.0, 0.02)
                    w2 = device_normal((H3, D3), 3, "w2", 0.0, 0.02)
                    dw1, dw2 = empty((D3, H3), "f32"), empty((H3, D3), "f32")
                    o1, o2, dxa = empty((R3, H3), "f32"), empty((R3, D3), "f32"), empty((R3, D3), "f32")
                    dh = empty((R3, H3), "f32")
                    keep += [w1, w2, dw1, dw2, o1, o2, dxa, dh]
                    f1 = 2 * R3 * D3 * H3
                    b1 = 4 * (R3 * D3 + D3 * H3 + R3 * H3)
                    m1f = ws(xt.OP.MATMUL, P(), [V(x), V(w1)], 0)
                    m1b = ws(xt.OP.MATMUL, P(), [V(x), V(w1)], 1)
                    m2f = ws(xt.OP.MATMUL, P(), [V(hy), V(w2)], 0)
                    m2b = ws(xt.OP.MATMUL, P(), [V(hy), V(w2)], 1)
                    E.append(Entry("c3.mlp1.fwd", W3, "f32", "mfma", lambda: xt.xt_op_fwd(
                        xt.OP.MATMUL, P(), [V(x), V(w1)], [V(o1)], *m1f), b1, f1, R3))
                    E.append(Entry("c3.mlp1.bwd", W3, "f32", "mfma", lambda: xt.xt_op_bwd(
                        xt.OP.MATMUL, P(), V(hd), [V(x), V(w1)], [], [V(dxa), V(dw1)], 0, *m1b), 2 * b1, 2 * f1, R3))
                    E.append(Entry("c3.mlp2.fwd", W3, "f32", "mfma", lambda: xt.xt_op_fwd(
                        xt.OP.MATMUL, P(), [V(hy), V(w2)], [V(o2)], *m2f), b1, f1, R3))
                    E.append(Entry("c3.mlp2.bwd", W3, "f32", "mfma", lambda: xt.xt_op_bwd(
                        xt.OP.MATMUL, P(), V(d), [V(hy), V(w2)], [], [V(dh), V(dw2)], 0, *m2b), 2 * b1, 2 * f1, R3))
            if want("c3.ce"):
                lg = device_normal((R3, V3), 3, "logits", 0.0, 2.0)
                tg = device_uniform_int((R3, 1), 0, V3, 3, "targets")
                L, lse, lr = empty((1, 1), "f32"), empty((R3, 1), "f32"), empty((R3, 1), "f32")
                dL = torch.ones((1, 1), dtype=torch.float32, device="cuda")
                dlg = empty((R3, V3), "f32")
                keep += [lg, tg, L, lse, lr, dL, dlg]
                E.append(Entry("c3.ce.fwd", W3, "f32", "hbm", lambda: xt.xt_op_fwd(
                    xt.OP.CROSS_ENTROPY, P(), [V(lg), V(tg)], [V(L), V(lse), V(lr)]), 4 * R3 * V3 + 16 * R3, rows=R3))
                E.append(Entry("c3.ce.bwd", W3, "f32", "hbm", lambda: xt.xt_op_bwd(
                    xt.OP.CROSS_ENTROPY, P(), V(dL), [V(lg), V(tg)], [V(lse)], [V(dlg), nullslot(tg)]),
                    2 * 4 * R3 * V3 + 8 * R3, rows=R3))

    def c4(want, E):
        nonlocal keep
        W4 = "bf16 16384x4096"
        R4, D4, F4 = 16384, 4096, 11008
        N4 = R4 * D4
        if any(want(n) for n in ("c4.",)):
            x = device_normal((R4, D4), 4, "x", dtype="bf16")
            d = device_normal((R4, D4), 4, "dout", dtype="bf16")
            keep += [x, d]
            if want("c4.rms"):
                gam = device_normal((D4,), 4, "gamma", 1.0, 0.1)
                y, ir, dx, dg = empty((R4, D4), "bf16"), empty((R4, 1), "f32"), empty((R4, D4), "bf16"), empty((D4,), "f32")
                keep += [gam, y, ir, dx, dg]
                prm = P(eps=1e-5)
                E.append(Entry("c4.rms.fwd", W4, "bf16", "hbm", lambda: xt.xt_op_fwd(
                    xt.OP.RMS_NORM, prm, [V(x), V(gam)], [V(y), V(ir)]), 2 * 2 * N4 + 4 * R4, rows=R4))
                wp, wn = ws(xt.OP.RMS_NORM, prm, [V(x), V(gam)])
                E.append(Entry("c4.rms.bwd", W4, "bf16", "hbm", lambda: xt.xt_op_bwd(
                    xt.OP.RMS_NORM, prm, V(d), [V(x), V(gam)], [V(ir)], [V(dx), V(dg)], 0, wp, wn),
                    3 * 2 * N4 + 4 * R4, rows=R4))
            if want("c4.swiglu"):
                g = device_normal((R4, F4), 4, "g", dtype="bf16")
                u = device_normal((R4, F4), 4, "u", dtype="bf16")
                dd = device_normal((R4, F4), 4, "d2", dtype="bf16")
                yy, dgg, duu = empty((R4, F4), "bf16"), empty((R4, F4), "bf16"), empty((R4, F4), "bf16")
                keep += [g, u, dd, yy, dgg, duu]
                NF = R4 * F4
                E.append(Entry("c4.swiglu.fwd", W4, "bf16", "hbm", lambda: xt.xt_op_fwd(
                    xt.OP.SWIGLU, P(), [V(g), V(u)], [V(yy)]), 3 * 2 * NF, rows=R4))
                E.append(Entry("c4.swiglu.bwd", W4, "bf16", "hbm", lambda: xt.xt_op_bwd(
                    xt.OP.SWIGLU, P(), V(dd), [V(g), V(u)], [], [V(dgg), V(duu)]), 5 * 2 * NF, rows=R4))
            if want("c4.rope"):
                ry, rdx = empty((R4, D4), "bf16"), empty((R4, D4), "bf16")
                keep += [ry, rdx]
                prm_r = P(head_dim=128, seq_len=4096, rope_base=10000.0)
                E.append(Entry("c4.rope.fwd", W4, "bf16", "hbm", lambda: xt.xt_op_fwd(
                    xt.OP.ROPE, prm_r, [V(x)], [V(ry)]), 2 * 2 * N4, rows=R4))
                E.append(Entry("c4.rope.bwd", W4, "bf16", "hbm", lambda: xt.xt_op_bwd(
                    xt.OP.ROPE, prm_r, V(d), [V(x)], [], [V(rdx)]), 2 * 2 * N4, rows=R4))
            if want("c4.dropout"):
                for site, const in (("attn", 0xA77), ("ffn", 0xF70)):
                    prm_d = P(p=0.1, seed=42 ^ 0 ^ const)
                    dy, dm, ddx = empty((R4, D4), "bf16"), empty((R4, D4), "u8"), empty((R4, D4), "bf16")
                    keep += [dy, dm, ddx]
                    E.append(Entry(f"c4.dropout.{site}.fwd", W4, "bf16", "hbm",
                                   (lambda prm_d=prm_d, dy=dy, dm=dm: xt.xt_op_fwd(
                                       xt.OP.DROPOUT, prm_d, [V(x)], [V(dy), V(dm)])), 2 * 2 * N4 + N4, rows=R4))
                    E.append(Entry(f"c4.dropout.{site}.bwd", W4, "bf16", "hbm",
                                   (lambda prm_d=prm_d, dm=dm, ddx=ddx: xt.xt_op_bwd(
                                       xt.OP.DROPOUT, prm_d, V(d), [V(x)], [V(dm)], [V(ddx)])), 2 * 2 * N4 + N4, rows=R4))
            if want("c4.accumulate"):
                dres = device_normal((R4, D4), 4, "resid", dtype="bf16")
                keep.append(dres)
                E.append(Entry("c4.accumulate", W4, "bf16", "hbm", lambda: xt.xt_grad_accumulate(V(dres), V(d)),
                               3 * 2 * N4, rows=R4))

    def c5(want, E):
        nonlocal keep
        W5 = "bf16 stress"
        if want("c5.ce"):
            R5, V5 = 32768, 128256
            lg = device_normal((R5, V5), 5, "logits", 0.0, 3.0, dtype="bf16")
            tg = device_uniform_int((R5, 1), 0, V5, 5, "targets")
            L, lse, lr = empty((1, 1), "f32"), empty((R5, 1), "f32"), empty((R5, 1), "f32")
            dL = torch.ones((1, 1), dtype=torch.float32, device="cuda")
            dlg = empty((R5, V5), "bf16")
            keep += [lg, tg, L, lse, lr, dL, dlg]
            E.append(Entry("c5.ce.fwd", W5, "bf16", "hbm", lambda: xt.xt_op_fwd(
                xt.OP.CROSS_ENTROPY, P(), [V(lg), V(tg)], [V(L), V(lse), V(lr)]), 2 * R5 * V5 + 16 * R5, rows=R5))
            E.append(Entry("c5.ce.bwd", W5, "bf16", "hbm", lambda: xt.xt_op_bwd(
                xt.OP.CROSS_ENTROPY, P(), V(dL), [V(lg), V(tg)], [V(lse)], [V(dlg), nullslot(tg)]),
                2 * 2 * R5 * V5 + 8 * R5, rows=R5))
        if want("c5.softmax"):
            R5 = C5 = 32768
            sx = device_normal((R5, C5), 5, "x", dtype="bf16")
            sd = device_normal((R5, C5), 5, "dout", dtype="bf16")
            sy, sdx = empty((R5, C5), "bf16"), empty((R5, C5), "bf16")
            keep += [sx, sd, sy, sdx]
            NS = R5 * C5
            E.append(Entry("c5.softmax.fwd", W5, "bf16", "hbm", lambda: xt.xt_op_fwd(
                xt.OP.SOFTMAX, P(), [V(sx)], [V(sy)]), 2 * 2 * NS, rows=R5))
            E.append(Entry("c5.softmax.bwd", W5, "bf16", "hbm", lambda: xt.xt_op_bwd(
                xt.OP.SOFTMAX, P(), V(sd), [V(sx)], [V(sy)], [V(sdx)]), 3 * 2 * NS, rows=R5))
        if want("c5.dbias"):
            RB, CB = 65536, 4096
            bd = device_normal((RB, CB), 5, "d3", dtype="bf16")
            bx = torch.empty((RB, CB), dtype=torch.bfloat16, device="cuda")   # shape only (not read)
            bias = torch.zeros((CB,), dtype=torch.float32, device="cuda")
            dbias = empty((CB,), "f32")
            keep += [bd, bx, bias, dbias]
            wp, wn = ws(xt.OP.ADD_BIAS, P(), [V(bd), V(bias)])
            E.append(Entry("c5.dbias", W5, "bf16", "hbm", lambda: xt.xt_op_bwd(
                xt.OP.ADD_BIAS, P(), V(bd), [V(bx), V(bias)], [], [nullslot(bx), V(dbias)], 0, wp, wn),
                2 * RB * CB + 4 * CB, rows=RB))
        if want("c5.gemm"):
            M, K, N = 8192, 4096, 4096
            A = device_normal((M, K), 5, "a", dtype="bf16")
            B = device_normal((K, N), 5, "b", 0.0, 0.02, dtype="bf16")
            Dg = device_normal((M, N), 5, "dout", dtype="bf16")
            dA, dB = empty((M, K), "bf16"), empty((K, N), "f32")
            keep += [A, B, Dg, dA, dB]
            fl = 2 * M * N * K
            gw = ws(xt.OP.MATMUL, P(), [V(A), V(B)], 1)
            E.append(Entry("c5.gemm.bwd_dA", W5, "bf16", "mfma", lambda: xt.xt_op_bwd(
                xt.OP.MATMUL, P(), V(Dg), [V(A), V(B)], [], [V(dA), nullslot(B)], 0, *gw),
                2 * (M * N + N * K + M * K), fl, M))
            E.append(Entry("c5.gemm.bwd_dB", W5, "bf16", "mfma", lambda: xt.xt_op_bwd(
                xt.OP.MATMUL, P(), V(Dg), [V(A), V(B)], [], [nullslot(A), V(dB)], 0, *gw),
                2 * (M * K + M * N) + 4 * K * N, fl, M))

    def c2():
        nonlocal keep
        if any(want(n) for n in ("c2.block", "f4.block", "f1.block")):
            shp = xb.BlockShape(B=4, S=256, H=4, Dh=64, hidden=688, vocab=4096)
            Wt = {}
            for k, s in xb.WEIGHT_SHAPES(shp).items():
                Wt[k] = (torch.ones(s, dtype=torch.float32, device="cuda") if k.startswith("g")
                         else device_normal(s, 2, k, 0.0, 0.02))
            bx2 = device_normal((shp.B * shp.S, shp.D), 2, "x")
            bt2 = device_uniform_int((shp.B * shp.S, 1), 0, shp.vocab, 2, "targets")
            keep += list(Wt.values()) + [bx2, bt2]
            holder = {}

            def run_block(ckpt=False, key="tape", fused=False):
                if key in holder:
                    holder[key].close()
                t = xt.Tape()
                w = xb.leaves(t, Wt)
                loss = xb.block(t, w, t.leaf(V(bx2)), t.leaf(V(bt2), requires_grad=False), shp, xt.DT.F32,
                                checkpoint=ckpt, fused_attention=fused)
                t.backward(loss)
                holder[key] = t
            def graph_block(key, fused=False):
                """The block recorded and run backward on a tape inside a HIP
                graph capture (after one eager warm-up on a side stream); the
                returned call replays it.  The tape stays alive with the graph."""
                side = torch.cuda.Stream()
                side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side):
                    run_block(False, key + "_warm", fused)
                torch.cuda.current_stream().wait_stream(side)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    t = xt.Tape()
                    w = xb.leaves(t, Wt)
                    loss = xb.block(t, w, t.leaf(V(bx2)), t.leaf(V(bt2), requires_grad=False), shp, xt.DT.F32,
                                    fused_attention=fused)
                    t.backward(loss)
                torch.cuda.synchronize()
                holder[key] = (t, g)
                return g.replay

            # GEMM flops of one fwd+bwd (for the record; the block is launch/cache bound)
            T, D = shp.B * shp.S, shp.D
            fl = 2 * T * D * D * 4 + 2 * T * D * shp.hidden * 3 + 2 * T * D * shp.vocab \
                + 2 * 2 * shp.B * shp.H * shp.S * shp.S * shp.Dh
            E.append(Entry("c2.block.fwdbwd", "tiny block 4x256x256 f32", "f32", "block", run_block, 0, 3 * fl,
                           shp.B * shp.S))
            # the same fwd+bwd replayed from a captured graph: device time
            # without the tape's host work and Python launch path
            E.append(Entry("c2.block.fwdbwd_graph", "tiny block 4x256x256 f32", "f32", "blockgraph",
                           graph_block("tape_graph"), 0, 3 * fl, shp.B * shp.S))
            # the same block as one recompute segment: the layer's forward runs
            # twice (the GEMM flops of the record count it once)
            E.append(Entry("f4.block.fwdbwd_recompute", "tiny block 4x256x256 f32", "f32", "block",
                           lambda: run_block(True, "tape_ckpt"), 0, 3 * fl, shp.B * shp.S))
            # the same block with the fused attention op
            E.append(Entry("f1.block.fwdbwd_fused_attention", "tiny block 4x256x256 f32", "f32", "block",
                           lambda: run_block(False, "tape_fused", True), 0, 3 * fl, shp.B * shp.S))
            E.append(Entry("f1.block.fwdbwd_fused_attention_graph", "tiny block 4x256x256 f32", "f32", "blockgraph",
                           graph_block("tape_fused_graph", True), 0, 3 * fl, shp.B * shp.S))
    def f3():
        nonlocal keep
        if not want("f3"):
            return
        # every gradient buffer of a 12-layer model of GPT-2-small width
        # (d 768, MLP 3072, vocabulary 50257, 1024 positions), f32
        shapes = []
        for _ in range(12):
            shapes += [(768, 768)] * 4 + [(768, 3072), (3072, 768)] + [(1, 768)] * 4
        shapes += [(50257, 768), (1024, 768), (1, 768), (1, 768)]
        gr = [device_normal(sh, 8, 200 + k, 0.0, 1e-3) for k, sh in enumerate(shapes)]
        keep += gr
        gv = [V(t) for t in gr]
        n = sum(t.numel() for t in gr)
        nb = xt.xt_grad_norm_workspace(gv)
        wsb = torch.empty(max(nb, 8), dtype=torch.uint8, device="cuda")
        out = torch.empty(2, dtype=torch.float32, device="cuda")
        one = torch.ones(1, dtype=torch.float32, device="cuda")
        keep += [wsb, out, one]
        W = "gpt2s-f32 12-layer gradient set"
        E.append(Entry("f3.grad_norm", W, "f32", "hbm",
                       lambda: xt.xt_grad_norm(gv, 1.0, out.data_ptr(), wsb.data_ptr(), nb), 4 * n, rows=len(gr)))
        # the clip step multiplies by a device-side coefficient (here 1.0, so
        # the buffers keep their values from step to step)
        E.append(Entry("f3.grads_scale", W, "f32", "hbm",
                       lambda: xt.xt_grads_scale(gv, 1.0, one.data_ptr()), 8 * n, rows=len(gr)))

    def f2():
        nonlocal keep
        if not want("f2"):
            return
        # token embedding at the GPT-2-small shape: 8 x 1024 Zipf(1.1) tokens
        # into a 50257 x 768 f32 table
        import synth
        Vv, Dd, Rr = 50257, 768, 8192
        tab = device_normal((Vv, Dd), 10, "emb", 0.0, 0.02)
        ids = torch.from_numpy(synth.host_zipf_int((Rr, 1), Vv, 1.1, 10, "ids")).cuda()
        y, d, dE = empty((Rr, Dd), "f32"), device_normal((Rr, Dd), 10, "dout"), empty((Vv, Dd), "f32")
        keep += [tab, ids, y, d, dE]
        ins = [V(tab), V(ids)]
        wsp, wsn = ws(xt.OP.EMBED, P(), ins)
        W = "gpt2s-f32 embedding 8192 tokens x 50257 x 768"
        E.append(Entry("f2.embed.fwd", W, "f32", "hbm", lambda: xt.xt_op_fwd(xt.OP.EMBED, P(), ins, [V(y)]),
                       2 * 4 * Rr * Dd + 4 * Rr, rows=Rr))
        E.append(Entry("f2.embed.bwd", W, "f32", "hbm", lambda: xt.xt_op_bwd(
            xt.OP.EMBED, P(), V(d), ins, [], [V(dE), nullslot(ids)], 0, wsp, wsn),
            4 * Rr * Dd + 4 * Vv * Dd + 4 * Rr, rows=Rr))

    def f1():
        nonlocal keep
        if not want("f1"):
            return
        # fused causal attention: 2 sequences x 2048 tokens, 16 heads x 128,
        # bf16 storage: bf16 matrix-core products with f32 accumulation
        B1, S1, H1, D1 = 2, 2048, 16, 128
        R1, C1 = B1 * S1, H1 * D1
        q = device_normal((R1, C1), 12, "q", dtype="bf16")
        k = device_normal((R1, C1), 12, "k", dtype="bf16")
        v = device_normal((R1, C1), 12, "v", dtype="bf16")
        d = device_normal((R1, C1), 12, "dout", dtype="bf16")
        out, lse = empty((R1, C1), "bf16"), empty((R1, H1), "f32")
        dq, dk, dv = empty((R1, C1), "bf16"), empty((R1, C1), "bf16"), empty((R1, C1), "bf16")
        keep += [q, k, v, d, out, lse, dq, dk, dv]
        prm = P(alpha=1.0 / math.sqrt(D1), causal=1, seq_len=S1, head_dim=D1)
        ins = [V(q), V(k), V(v)]
        wsp, wsn = ws(xt.OP.ATTENTION, prm, ins)
        # causal: half of the S x S scores; two products forward, five backward
        prod = 2.0 * S1 * S1 * D1 * B1 * H1 / 2
        W = "attention 2x2048 tokens, 16 heads x 128, causal, bf16 storage"
        E.append(Entry("f1.attn.fwd", W, "bf16", "mfma", lambda: xt.xt_op_fwd(
            xt.OP.ATTENTION, prm, ins, [V(out), V(lse)]), 4 * 2 * R1 * C1, 2 * prod, R1))
        E.append(Entry("f1.attn.bwd", W, "bf16", "mfma", lambda: xt.xt_op_bwd(
            xt.OP.ATTENTION, prm, V(d), ins, [V(out), V(lse)], [V(dq), V(dk), V(dv)], 0, wsp, wsn),
            2 * 8 * R1 * C1, 5 * prod, R1))

    c3(want, E)
    c4(want, E)
    c5(want, E)
    c2()
    f3()
    f2()
    f1()
    # extra buffer copies of the memory-bound ops that fit in the caches
    for builder, pre in ((c3, "c3."), (c4, "c4."), (c5, "c5.")):
        rot = {e.name: min(MAX_COPIES, -(-ROTATE_BYTES // e.bytes)) for e in E
               if e.name.startswith(pre) and e.kind == "hbm" and 0 < e.bytes < ROTATE_BYTES and want(e.name)}
        for cp in range(1, max(rot.values(), default=1)):
            names = [n for n, k in rot.items() if k > cp]
            extra = []
            builder(lambda n, names=names: any(m.startswith(n) or n.startswith(m) for m in names), extra)
            for x in extra:
                for e in E:
                    if e.name == x.name and x.name in names:
                        e.fns.append(x.fn)
    return [e for e in E if want(e.name)], keep


# --------------------------------------------------------------------------
SWEEP_DIMS = (768, 1024, 2048, 3072, 4096)


def sweep(steps, warmup):
    """rows/s against the row width d for the row-wise ops: every op fwd and
    bwd at d in SWEEP_DIMS with R = 2^30 / (s*d) rows (1 GiB per activation
    tensor), f32 and bf16; timed with HIP events on the launch stream."""
    import torch
    import autograd_row_wise_amd as xt
    from synth import device_normal

    V, P = xt.view, xt.params
    big = 1 << 30
    res = []
    for dt, s_ in (("f32", 4), ("bf16", 2)):
        tdt = torch.float32 if dt == "f32" else torch.bfloat16
        nel = big // s_
        X = device_normal((nel // 4096, 4096), 7, "x", dtype=dt)
        D = device_normal((nel // 4096, 4096), 7, "dout", dtype=dt)
        Y = torch.empty_like(X)
        DX = torch.empty_like(X)
        st1 = torch.empty(big // (s_ * 768), dtype=torch.float32, device="cuda")
        st2 = torch.empty_like(st1)
        gam = torch.ones(4096, dtype=torch.float32, device="cuda")
        bet = torch.zeros(4096, dtype=torch.float32, device="cuda")
        dg = torch.empty(4096, dtype=torch.float32, device="cuda")
        db = torch.empty(4096, dtype=torch.float32, device="cuda")
        for d in SWEEP_DIMS:
            R = big // (s_ * d)
            N = R * d
            x, dd, y, dx = (t.view(-1)[:N].view(R, d) for t in (X, D, Y, DX))
            a, b = st1[:R].view(R, 1), st2[:R].view(R, 1)
            g, bt, gg, gb = gam[:d].view(1, d), bet[:d].view(1, d), dg[:d].view(1, d), db[:d].view(1, d)
            def wsp(op, prm, ins):
                n = xt.xt_workspace_bytes(op, 1, prm, ins)
                w = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
                return w, (w.data_ptr() if n else None), n
            pe = P(eps=1e-5)
            w_rms = wsp(xt.OP.RMS_NORM, pe, [V(x), V(g)])
            w_ln = wsp(xt.OP.LAYER_NORM, pe, [V(x), V(g), V(bt)])
            pr = P(head_dim=128, seq_len=4096, rope_base=10000.0)
            ops = {
                "rms_norm": (lambda: xt.xt_op_fwd(xt.OP.RMS_NORM, pe, [V(x), V(g)], [V(y), V(a)]),
                             lambda: xt.xt_op_bwd(xt.OP.RMS_NORM, pe, V(dd), [V(x), V(g)], [V(a)], [V(dx), V(gg)], 0,
                                                  w_rms[1], w_rms[2]),
                             2 * s_ * N + 4 * R, 3 * s_ * N + 4 * R),
                "layer_norm": (lambda: xt.xt_op_fwd(xt.OP.LAYER_NORM, pe, [V(x), V(g), V(bt)], [V(y), V(a), V(b)]),
                               lambda: xt.xt_op_bwd(xt.OP.LAYER_NORM, pe, V(dd), [V(x), V(g), V(bt)], [V(a), V(b)],
                                                    [V(dx), V(gg), V(gb)], 0, w_ln[1], w_ln[2]),
                               2 * s_ * N + 8 * R, 3 * s_ * N + 8 * R),
                "softmax": (lambda: xt.xt_op_fwd(xt.OP.SOFTMAX, P(), [V(x)], [V(y)]),
                            lambda: xt.xt_op_bwd(xt.OP.SOFTMAX, P(), V(dd), [V(x)], [V(y)], [V(dx)]),
                            2 * s_ * N, 3 * s_ * N),
                "rope": (lambda: xt.xt_op_fwd(xt.OP.ROPE, pr, [V(x)], [V(y)]),
                         lambda: xt.xt_op_bwd(xt.OP.ROPE, pr, V(dd), [V(x)], [], [V(dx)]),
                         2 * s_ * N, 2 * s_ * N),
                "silu": (lambda: xt.xt_op_fwd(xt.OP.SILU, P(), [V(x)], [V(y)]),
                         lambda: xt.xt_op_bwd(xt.OP.SILU, P(), V(dd), [V(x)], [], [V(dx)]),
                         2 * s_ * N, 3 * s_ * N),
            }
            stream = torch.cuda.current_stream()
            for name, (f, bwd, bf, bb) in ops.items():
                ms = []
                for fn in (f, bwd):
                    for _ in range(warmup):
                        fn()
                    ev = []
                    for _ in range(steps):
                        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        e0.record(stream)
                        fn()
                        e1.record(stream)
                        ev.append((e0, e1))
                    torch.cuda.synchronize()
                    ms.append(sum(e0.elapsed_time(e1) for e0, e1 in ev) / steps)
                gbps = (bf + bb) / ((ms[0] + ms[1]) * 1e-3) / 1e9
                res.append({"op": name, "dtype": dt, "d": d, "rows": R, "fwd_ms": round(ms[0], 4),
                            "bwd_ms": round(ms[1], 4), "fwd_rows_per_s": round(R / (ms[0] * 1e-3)),
                            "bwd_rows_per_s": round(R / (ms[1] * 1e-3)), "fwdbwd_GBps": round(gbps, 1),
                            "frac": round(gbps / HBM_PEAK_GBPS, 4)})
        del X, D, Y, DX
        torch.cuda.empty_cache()
    return res


LONG_ROWS = (("softmax", "f32", 32768), ("softmax", "f32", 50257), ("softmax", "bf16", 50257),
             ("layer_norm", "f32", 16384), ("rms_norm", "f32", 16384), ("layer_norm", "bf16", 50257))


def long_rows(steps, warmup):
    """Rows the register-resident kernels do not take (the streaming path):
    each op fwd and bwd at 1 GiB per activation tensor, R = 2^30 / (s*d)
    contiguous rows (a 50257-wide row starts 16-byte aligned only every
    16 / gcd(16, s*50257) rows); timed like the sweep."""
    import torch
    import autograd_row_wise_amd as xt
    from synth import device_normal

    V, P = xt.view, xt.params
    big = 1 << 30
    res = []
    for name, dt, d in LONG_ROWS:
        s_ = 4 if dt == "f32" else 2
        R = big // (s_ * d)
        N = R * d
        x = device_normal((R, d), 8, "x", dtype=dt)
        dd = device_normal((R, d), 8, "dout", dtype=dt)
        y, dx = torch.empty_like(x), torch.empty_like(x)
        a, b = (torch.empty((R, 1), dtype=torch.float32, device="cuda") for _ in range(2))
        g = torch.ones((1, d), dtype=torch.float32, device="cuda")
        bt = torch.zeros((1, d), dtype=torch.float32, device="cuda")
        gg, gb = torch.empty_like(g), torch.empty_like(g)
        pe = P(eps=1e-5)
        if name == "softmax":
            f = lambda: xt.xt_op_fwd(xt.OP.SOFTMAX, P(), [V(x)], [V(y)])  # noqa: E731
            bw = lambda: xt.xt_op_bwd(xt.OP.SOFTMAX, P(), V(dd), [V(x)], [V(y)], [V(dx)])  # noqa: E731
            bf, bb = 2 * s_ * N, 3 * s_ * N
        elif name == "rms_norm":
            n = xt.xt_workspace_bytes(xt.OP.RMS_NORM, 1, pe, [V(x), V(g)])
            w = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
            f = lambda: xt.xt_op_fwd(xt.OP.RMS_NORM, pe, [V(x), V(g)], [V(y), V(a)])  # noqa: E731
            bw = lambda: xt.xt_op_bwd(xt.OP.RMS_NORM, pe, V(dd), [V(x), V(g)], [V(a)], [V(dx), V(gg)], 0,  # noqa: E731
                                      w.data_ptr(), n)
            bf, bb = 2 * s_ * N + 4 * R, 3 * s_ * N + 4 * R
        else:
            n = xt.xt_workspace_bytes(xt.OP.LAYER_NORM, 1, pe, [V(x), V(g), V(bt)])
            w = torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")
            f = lambda: xt.xt_op_fwd(xt.OP.LAYER_NORM, pe, [V(x), V(g), V(bt)], [V(y), V(a), V(b)])  # noqa: E731
            bw = lambda: xt.xt_op_bwd(xt.OP.LAYER_NORM, pe, V(dd), [V(x), V(g), V(bt)], [V(a), V(b)],  # noqa: E731
                                      [V(dx), V(gg), V(gb)], 0, w.data_ptr(), n)
            bf, bb = 2 * s_ * N + 8 * R, 3 * s_ * N + 8 * R
        stream = torch.cuda.current_stream()
        ms = []
        for fn in (f, bw):
            for _ in range(warmup):
                fn()
            ev = []
            for _ in range(steps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                ev.append((e0, e1))
            torch.cuda.synchronize()
            ms.append(med([e0.elapsed_time(e1) for e0, e1 in ev]))
        gbps = (bf + bb) / ((ms[0] + ms[1]) * 1e-3) / 1e9
        res.append({"op": name, "dtype": dt, "d": d, "rows": R, "fwd_ms": round(ms[0], 4), "bwd_ms": round(ms[1], 4),
                    "fwd_GBps": round(bf / (ms[0] * 1e-3) / 1e9, 1), "bwd_GBps": round(bb / (ms[1] * 1e-3) / 1e9, 1),
                    "fwdbwd_GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)})
        del x, dd, y, dx
        torch.cuda.empty_cache()
    return res


# --------------------------------------------------------------------------
def c1_latency(steps, warmup, reps=50):
    """Every op of the 8 x 64 f32 workload, forward and backward, as the
    device time per launch (microseconds): a HIP graph of `reps` launches of
    the op in a row, HIP events around each replay, median over the replays.
    At 2 KB per tensor these figures are the launch floor of each kernel."""
    import torch
    import autograd_row_wise_amd as xt
    import synth

    V, P = xt.view, xt.params
    R, C = 8, 64

    def dev(a):
        return torch.from_numpy(a).cuda()

    x = dev(synth.host_normal((R, C), 0, "x"))
    g = dev(synth.host_normal((C,), 0, "gamma", 1.0, 0.1))
    bias = dev(synth.host_normal((C,), 0, "bias"))
    d = dev(synth.host_normal((R, C), 0, "dout"))
    t = dev(synth.host_uniform_int((R, 1), 0, C, 0, "targets"))
    y, y2, y3, dx = (torch.empty((R, C), device="cuda") for _ in range(4))
    ir, lse, lr, L = (torch.empty((R, 1), device="cuda"), torch.empty((R, 1), device="cuda"),
                      torch.empty((R, 1), device="cuda"), torch.empty((1, 1), device="cuda"))
    dg = torch.empty((C,), device="cuda")
    mask = torch.empty((R, C), dtype=torch.uint8, device="cuda")
    dL = torch.ones((1, 1), device="cuda")
    wsb = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    wp, wn = wsb.data_ptr(), wsb.numel()
    null = lambda tt: (lambda v: (setattr(v, "data", None), v)[1])(V(tt))  # noqa: E731
    pe = P(eps=1e-5)
    pr = P(head_dim=16, seq_len=8, rope_base=10000.0)
    pd = P(p=0.1, seed=42)
    ops = {
        "rms_norm": (lambda: xt.xt_op_fwd(xt.OP.RMS_NORM, pe, [V(x), V(g)], [V(y), V(ir)]),
                     lambda: xt.xt_op_bwd(xt.OP.RMS_NORM, pe, V(d), [V(x), V(g)], [V(ir)], [V(dx), V(dg)], 0, wp, wn)),
        "softmax": (lambda: xt.xt_op_fwd(xt.OP.SOFTMAX, P(), [V(x)], [V(y)]),
                    lambda: xt.xt_op_bwd(xt.OP.SOFTMAX, P(), V(d), [V(x)], [V(y)], [V(dx)])),
        "silu": (lambda: xt.xt_op_fwd(xt.OP.SILU, P(), [V(x)], [V(y)]),
                 lambda: xt.xt_op_bwd(xt.OP.SILU, P(), V(d), [V(x)], [], [V(dx)])),
        "add_bias": (lambda: xt.xt_op_fwd(xt.OP.ADD_BIAS, P(), [V(x), V(bias)], [V(y)]),
                     lambda: xt.xt_op_bwd(xt.OP.ADD_BIAS, P(), V(d), [V(x), V(bias)], [], [V(dx), V(dg)], 0, wp, wn)),
        "cross_entropy": (lambda: xt.xt_op_fwd(xt.OP.CROSS_ENTROPY, P(), [V(x), V(t)], [V(L), V(lse), V(lr)]),
                          lambda: xt.xt_op_bwd(xt.OP.CROSS_ENTROPY, P(), V(dL), [V(x), V(t)], [V(lse)],
                                               [V(dx), null(t)])),
        "rope": (lambda: xt.xt_op_fwd(xt.OP.ROPE, pr, [V(x)], [V(y)]),
                 lambda: xt.xt_op_bwd(xt.OP.ROPE, pr, V(d), [V(x)], [], [V(dx)])),
        "dropout": (lambda: xt.xt_op_fwd(xt.OP.DROPOUT, pd, [V(x)], [V(y), V(mask)]),
                    lambda: xt.xt_op_bwd(xt.OP.DROPOUT, pd, V(d), [V(x)], [V(mask)], [V(dx)])),
        # y = x*x + x*x: two products and a sum forward.  Backward as the tape
        # runs it: the sum passes d through, then each product's backward once
        # per slot of x, the first push storing into dx, the other three
        # accumulating ([AE] fan-out sum)
        "fan_out": (lambda: (xt.xt_op_fwd(xt.OP.MUL, P(), [V(x), V(x)], [V(y2)]),
                             xt.xt_op_fwd(xt.OP.MUL, P(), [V(x), V(x)], [V(y3)]),
                             xt.xt_op_fwd(xt.OP.ADD, P(), [V(y2), V(y3)], [V(y)])),
                    lambda: (xt.xt_op_bwd(xt.OP.MUL, P(), V(d), [V(x), V(x)], [], [V(dx), null(x)], 0),
                             xt.xt_op_bwd(xt.OP.MUL, P(), V(d), [V(x), V(x)], [], [null(x), V(dx)], 0b10),
                             xt.xt_op_bwd(xt.OP.MUL, P(), V(d), [V(x), V(x)], [], [V(dx), null(x)], 0b01),
                             xt.xt_op_bwd(xt.OP.MUL, P(), V(d), [V(x), V(x)], [], [null(x), V(dx)], 0b10))),
    }
    stream = torch.cuda.current_stream()
    out = {}
    for name, (f, b) in ops.items():
        rec = {}
        for tag, fn in (("fwd", f), ("bwd", b)):
            gr = capture([fn], reps)
            for _ in range(warmup):
                gr.replay()
            torch.cuda.synchronize()
            ev = []
            for _ in range(max(steps, 5)):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                gr.replay()
                e1.record(stream)
                ev.append((e0, e1))
            torch.cuda.synchronize()
            rec[tag] = round(med([a.elapsed_time(b_) * 1e3 / reps for a, b_ in ev]), 2)
            del gr
        out[name] = rec
    return {"workload": "8x64 f32 (x ~ N(0,1) seed 0, gamma ~ N(1,0.1), eps 1e-5, bias ~ N(0,1), targets U[0,64), "
                        "rope head_dim 16 base 1e4 positions 0..7, dropout p 0.1 seed 42, fan-out y = x*x + x*x)",
            "unit": "us per op call (device time, graph of %d calls in a row)" % reps, "ops": out}


# --------------------------------------------------------------------------
def host_cores():
    """Threads the CPU baseline may use: the cores this process may run on,
    at most 16 (the host share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(frac_rows=1 / 32, repeats=3):
    """The oracle (numpy f64) fwd+bwd of every memory-bound op of the step on
    the first `frac_rows` of each op's rows, timed on one core and on all
    host cores (rows split into one contiguous block per thread; each thread
    runs the same oracle functions on its block, numpy limited to one thread
    per call); the median of `repeats` passes of each; GB/s over the
    sample's algorithmic bytes."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits

    from oracle import ops, rng
    import synth

    def rows(R):
        return max(1, int(R * frac_rows))

    jobs = []   # (name, algorithmic bytes, rows, fn(lo, hi)) -- fn runs rows [lo, hi)
    R = rows(8192)
    x = synth.host_normal((R, 768), 3, "x").astype(np.float64)
    g = synth.host_normal((768,), 3, "gamma", 1.0, 0.1).astype(np.float64)
    b = synth.host_normal((768,), 3, "beta", 0.0, 0.1).astype(np.float64)
    d = synth.host_normal((R, 768), 3, "dout").astype(np.float64)
    jobs.append(("ln", 5 * 4 * R * 768 + 16 * R, R,
                 lambda lo, hi: ops.layer_norm_bwd(d[lo:hi], x[lo:hi], g, *ops.layer_norm(x[lo:hi], g, b, 1e-5)[1:])))
    h = synth.host_normal((R, 3072), 3, "g").astype(np.float64)
    jobs.append(("gelu", 5 * 4 * R * 3072, R, lambda lo, hi: (ops.gelu(h[lo:hi]), ops.gelu_bwd(h[lo:hi], h[lo:hi]))))
    lg = synth.host_normal((R, 50257), 3, "logits", 0.0, 2.0).astype(np.float64)
    t = synth.host_uniform_int((R,), 0, 50257, 3, "targets")
    jobs.append(("ce3", 3 * 4 * R * 50257, R, lambda lo, hi: ops.cross_entropy_bwd(
        1.0, lg[lo:hi], t[lo:hi], ops.cross_entropy(lg[lo:hi], t[lo:hi])[1])))
    R4 = rows(16384)
    x4 = synth.host_normal((R4, 4096), 4, "x").astype(np.float64)
    g4 = synth.host_normal((4096,), 4, "gamma", 1.0, 0.1).astype(np.float64)
    d4 = synth.host_normal((R4, 4096), 4, "dout").astype(np.float64)
    jobs.append(("rms", 5 * 2 * R4 * 4096, R4, lambda lo, hi: ops.rms_norm_bwd(
        d4[lo:hi], x4[lo:hi], g4, ops.rms_norm(x4[lo:hi], g4, 1e-5)[1])))
    jobs.append(("rope", 4 * 2 * R4 * 4096, R4, lambda lo, hi: (
        ops.rope(x4[lo:hi], 128, 10000.0, 4096, positions=np.arange(lo, hi) % 4096),
        ops.rope_bwd(d4[lo:hi], 128, 10000.0, 4096, positions=np.arange(lo, hi) % 4096))))
    jobs.append(("dropout", 2 * (2 * 2 * R4 * 4096 + R4 * 4096), R4, lambda lo, hi: rng.dropout_bwd(
        d4[lo:hi], rng.dropout(x4[lo:hi], 0.1, 42 ^ 0xA77, index_offset=lo * 4096)[1], 0.1)))
    sg = synth.host_normal((R4, 11008), 4, "g").astype(np.float64)
    jobs.append(("swiglu", 8 * 2 * R4 * 11008, R4, lambda lo, hi: (
        ops.swiglu(sg[lo:hi], sg[lo:hi]), ops.swiglu_bwd(sg[lo:hi], sg[lo:hi], sg[lo:hi]))))
    R5 = rows(32768)
    sx = synth.host_normal((R5, 32768), 5, "x").astype(np.float64)
    jobs.append(("softmax", 5 * 2 * R5 * 32768, R5, lambda lo, hi: ops.softmax_bwd(sx[lo:hi], ops.softmax(sx[lo:hi]))))
    lg5 = synth.host_normal((R5, 128256), 5, "logits", 0.0, 3.0).astype(np.float64)
    t5 = synth.host_uniform_int((R5,), 0, 128256, 5, "targets")
    jobs.append(("ce5", 3 * 2 * R5 * 128256, R5, lambda lo, hi: ops.cross_entropy_bwd(
        1.0, lg5[lo:hi], t5[lo:hi], ops.cross_entropy(lg5[lo:hi], t5[lo:hi])[1])))
    total_b = sum(j[1] for j in jobs)

    def one_pass(pool, n):
        t0 = time.perf_counter()
        for _, _, nr, fn in jobs:
            cuts = [nr * i // n for i in range(n + 1)]
            if n == 1:
                fn(0, nr)
            else:
                list(pool.map(lambda i: fn(cuts[i], cuts[i + 1]), [i for i in range(n) if cuts[i] < cuts[i + 1]]))
        return time.perf_counter() - t0

    res = {}
    ncores = host_cores()
    with threadpool_limits(limits=1):
        for n in sorted({1, ncores}):
            with ThreadPoolExecutor(max_workers=n) as pool:
                ts = sorted(one_pass(pool, n) for _ in range(repeats))
            res[n] = ts[len(ts) // 2]
    sample = (f"numpy f64 oracle, fwd+bwd of layer_norm, gelu, cross_entropy (both vocabularies), rms_norm, rope, "
              f"dropout, swiglu, softmax on the first 1/{int(round(1 / frac_rows))} of each op's rows "
              f"({total_b / 1e9:.2f} GB algorithmic per pass); median of {repeats} passes")
    out = {"value": round(total_b / res[ncores] / 1e9, 4), "unit": "GB/s", "cores": ncores, "kind": "oracle",
           "sample": sample + f"; rows split over {ncores} threads", "pass_s": round(res[ncores], 3),
           "single_core": {"value": round(total_b / res[1] / 1e9, 4), "unit": "GB/s", "cores": 1,
                           "pass_s": round(res[1], 3)}}
    return out


# --------------------------------------------------------------------------
def time_steps(entries, stream, steps, warmup):
    """W untimed passes, then K timed passes over `entries`, each op
    bracketed by HIP events on the launch stream; returns the wall-clock ms
    per pass (synchronised on both sides)."""
    import torch

    def one(record):
        for e in entries:
            if record:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                e.fn()
                b.record(stream)
                e._ev.append((a, b))
            else:
                e.fn()

    for e in entries:
        e._ev = []
    for _ in range(warmup):
        one(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for e in entries:
        e.times_ms = [a.elapsed_time(b) for a, b in e._ev]
    return (t1 - t0) * 1e3 / max(steps, 1)


def capture(fns, reps=1):
    """A HIP graph of `fns` called in order, `reps` times (torch's capture
    stream is current while they launch, so the library's kernels land in
    the graph).  One eager call first, as torch asks before a capture."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for fn in fns:
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            for fn in fns:
                fn()
    torch.cuda.synchronize()
    return g


def time_graphs(entries, stream, steps, warmup, target_ms=0.3):
    """Per-op GPU time without the Python launch path: each op captured
    `reps` times in a row into one graph (enough launches to fill about
    target_ms), replayed with HIP events around each replay; the op's time is
    the replay's / reps."""
    import torch
    for e in entries:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(3):
            e.fn()
        b.record(stream)
        torch.cuda.synchronize()
        est = a.elapsed_time(b) / 3
        k = len(e.fns)
        e.reps = max(1, min(50, math.ceil(target_ms / max(est, 1e-4))))
        e.reps = max(k, -(-e.reps // k) * k)          # whole cycles through the buffer copies
        g = capture([e.fns[i % k] for i in range(e.reps)])
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        ev = []
        for _ in range(steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            g.replay()
            b.record(stream)
            ev.append((a, b))
        torch.cuda.synchronize()
        e.times_ms = [x.elapsed_time(y) / e.reps for x, y in ev]
        del g


def time_step_graph(entries, stream, steps, warmup):
    """The step as one HIP graph of every capturable op (the tape-driven
    block runs eagerly after it): wall-clock ms per step, synchronised on
    both sides of the K timed steps."""
    import torch
    # tape-driven blocks run eagerly after the graph (a block replayed from
    # its own graph cannot be launched inside another capture)
    cap = [e for e in entries if e.kind not in ("block", "blockgraph")]
    eager = [e for e in entries if e.kind in ("block", "blockgraph")]
    g = capture([e.fn for e in cap]) if cap else None
    for _ in range(warmup):
        if g is not None:
            g.replay()
        for e in eager:
            e.fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        if g is not None:
            g.replay()
        for e in eager:
            e.fn()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    del g
    return (t1 - t0) * 1e3 / max(steps, 1)


def copy_floor(ops_out, steps, warmup, below=0.72):
    """For every memory-bound op of the step under `below` of the HBM peak:
    the same algorithmic bytes moved by a plain streaming kernel (the
    library's SCALE by 1: one 16-byte load and one store per pack, nothing
    else), on f32 rows of the op's width, timed the same way as the op (a
    graph of repeated launches over independent buffer copies).  At these
    sizes a launch's ramp-up and drain are a large part of its time; the
    copy's fraction is the floor such a launch reaches."""
    import torch
    import autograd_row_wise_amd as xt
    picked = [o for o in ops_out if "GBps" in o and o["frac"] < below]
    res = []
    for o in picked:
        n = o["bytes"] // 8                                  # f32 elements read (and as many written)
        cols = 768 if n % 768 == 0 else 4096 if n % 4096 == 0 else 1
        rows = n // cols
        k = min(MAX_COPIES, max(1, -(-ROTATE_BYTES // o["bytes"])))
        bufs = [(torch.ones((rows, cols), dtype=torch.float32, device="cuda"),
                 torch.empty((rows, cols), dtype=torch.float32, device="cuda")) for _ in range(k)]
        prm = xt.params(alpha=1.0)
        e = Entry("floor." + o["op"], "copy of the same bytes", "f32", "hbm",
                  lambda a=bufs[0]: xt.xt_op_fwd(xt.OP.SCALE, prm, [xt.view(a[0])], [xt.view(a[1])]), 8 * n, rows=rows)
        e.fns = [(lambda a=a: xt.xt_op_fwd(xt.OP.SCALE, prm, [xt.view(a[0])], [xt.view(a[1])])) for a in bufs]
        time_graphs([e], torch.cuda.current_stream(), steps, warmup)
        ms = med(e.times_ms)
        gbps = e.bytes / (ms * 1e-3) / 1e9
        res.append({"op": o["op"], "op_frac": o["frac"], "bytes": e.bytes, "copy_ms": round(ms, 5),
                    "copy_GBps": round(gbps, 1), "copy_frac": round(gbps / HBM_PEAK_GBPS, 4),
                    "op_vs_copy": round(o["GBps"] / gbps, 4)})
        del bufs
    return res


def med(xs):
    """Median of the timed repetitions (robust to a stray slow launch)."""
    v = sorted(xs)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def op_record(e):
    ms = med(e.times_ms)
    rec = {"op": e.name, "workload": e.workload, "dtype": e.dtype, "ms": round(ms, 5)}
    if getattr(e, "reps", None):
        rec["launches_per_replay"] = e.reps
    if e.kind == "hbm":
        gbps = e.bytes / (ms * 1e-3) / 1e9
        rec.update(bytes=e.bytes, GBps=round(gbps, 1), frac=round(gbps / HBM_PEAK_GBPS, 4),
                   rows_per_s=round(e.rows / (ms * 1e-3), 1))
    elif e.kind == "mfma":
        tf = e.flops / (ms * 1e-3) / 1e12
        rec.update(flops=e.flops, TFLOPs=round(tf, 2), frac=round(tf / MFMA_PEAK_TFLOPS[e.dtype], 4),
                   bytes=e.bytes)
    else:
        rec.update(flops=e.flops, TFLOPs=round(e.flops / (ms * 1e-3) / 1e12, 3),
                   note="tape-driven, cache-resident" + (", replayed from a captured HIP graph (device time)"
                                                         if e.kind == "blockgraph" else ", eager (host tape work and "
                                                         "Python launch path included)"))
    return rec


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (collectives are out of scope); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    entries, keep = build_entries(args.only)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    # The step is every op of the hot path (names c2..c5); the ops that
    # widen it (names f1..f4) are timed after it, in a loop of their own.
    main = [e for e in entries if not e.name.startswith("f")]
    extra = [e for e in entries if e.name.startswith("f")]
    if args.eager:
        wall_ms = time_steps(main, stream, args.steps, args.warmup)
        hbm_wall_ms = sum(med(e.times_ms) for e in main if e.kind == "hbm")
        if extra:
            time_steps(extra, stream, args.steps, args.warmup)
    else:
        # the step replays one graph; per-op times come from graphs of each
        # op alone (the tape-driven block is timed eagerly in both)
        wall_ms = time_step_graph(main, stream, args.steps, args.warmup)
        hbm_wall_ms = time_step_graph([e for e in main if e.kind == "hbm"], stream, args.steps, args.warmup)
        for group in (main, extra):
            time_graphs([e for e in group if e.kind not in ("block", "blockgraph")], stream, args.steps, args.warmup)
            time_steps([e for e in group if e.kind in ("block", "blockgraph")], stream, args.steps, args.warmup)

    ops_out = [op_record(e) for e in main]
    extra_out = [op_record(e) for e in extra]
    total_bytes = sum(e.bytes for e in main)
    # the roofline is that of the kernel-level op with the largest share of
    # step time (the tape-driven block is a composite of many kernels)
    kern = [e for e in main if e.kind in ("hbm", "mfma")]
    dom = max(kern, key=lambda e: med(e.times_ms)) if kern else None
    roof = None
    if dom is not None:
        ms = med(dom.times_ms)
        if dom.kind == "mfma":
            ach = dom.flops / (ms * 1e-3) / 1e12
            peak = MFMA_PEAK_TFLOPS[dom.dtype]
            roof = {"bound": "mfma", "kernel": dom.name, "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(ach / peak, 4), "traffic": None}
        else:
            ach = dom.bytes / (ms * 1e-3) / 1e9
            roof = {"bound": "hbm", "kernel": dom.name, "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(dom.name),
                    "algorithmic_bytes": dom.bytes}
    entries = main
    hbm_entries = [e for e in entries if e.kind == "hbm"]
    hbm_ms = sum(med(e.times_ms) for e in hbm_entries)
    hbm_bytes = sum(e.bytes for e in hbm_entries)
    out = {
        "metric": "fwd+bwd achieved HBM GB/s (fraction of peak) per op; rows/s at d=768..4096",
        "value": round(hbm_bytes / (hbm_wall_ms * 1e-3) / 1e9, 2) if hbm_wall_ms else None,
        "unit": "GB/s",
        "value_is": ("achieved HBM GB/s of the memory-bound part of the step: the algorithmic bytes of every "
                     "memory-bound op fwd+bwd / the wall time of one graph replay of those ops; frac = value / "
                     "8000 GB/s.  The GEMMs (TFLOP/s) and the tape-driven block (us) are in ops"),
        "frac": round(hbm_bytes / (hbm_wall_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4) if hbm_wall_ms else None,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(hbm_wall_ms, 3) if hbm_wall_ms else None,
        "ms_per_full_step": round(wall_ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32+bf16", "data": "synthetic",
        "config": {"workload": "hot-path suite: every op fwd+bwd at the gpt2s-f32 8x1024x768, bf16 16384x4096 and "
                               "bf16-stress shapes, and the tiny transformer block on the tape",
                   "parallelism": "none (1 GPU)"},
        "memory_bound_sum_of_ops_GBps": round(hbm_bytes / (hbm_ms * 1e-3) / 1e9, 1) if hbm_ms else None,
        "full_step_bytes_GBps": round(total_bytes / (wall_ms * 1e-3) / 1e9, 2),
        "roofline": roof,
        "cpu_baseline": None,
        "ops": ops_out,
        "next_rows": extra_out,
        "timing": ("eager: every op launched from Python, HIP events around each launch" if args.eager else
                   "HIP graphs: the step is one graph replay (the tape-driven block eager after it); each op's "
                   "time is a graph of that op launched reps times in a row (cycling through independent buffer "
                   "copies when its bytes would fit in the caches), HIP events around the replay / reps, median of "
                   "the timed replays"),
    }
    if args.ops_json:
        with open(args.ops_json, "w") as f:
            json.dump(ops_out + extra_out, f, indent=1)
    if not args.no_sweep and not args.only:
        out["sweep"] = {"what": "fwd and bwd of each row-wise op at 1 GiB per activation tensor, R = 2^30/(s*d)",
                        "entries": sweep(args.steps, args.warmup)}
    if not args.no_sweep and (not args.only or "long" in args.only):
        out["long_rows"] = {"what": "rows the register-resident kernels do not take (streaming kernels), "
                                    "1 GiB per activation tensor", "entries": long_rows(args.steps, args.warmup)}
    if not args.only:
        out["c1_latency"] = c1_latency(args.steps, args.warmup)
    if not args.only or "floor" in args.only:
        out["copy_floor"] = {"what": "each memory-bound op under 72% of HBM peak beside a plain streaming copy "
                                     "(SCALE by 1, f32) of the same algorithmic bytes, timed the same way",
                             "entries": copy_floor(ops_out, args.steps, args.warmup)}
    if not args.no_cpu_baseline:
        try:
            out["cpu_baseline"] = cpu_baseline()
        except Exception as ex:  # the baseline is reported, never required
            out["cpu_baseline"] = {"error": repr(ex)}
    del keep
    print(json.dumps(out))


if __name__ == "__main__":
    main()
