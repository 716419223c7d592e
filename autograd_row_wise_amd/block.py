"""Composed attention and a small pre-norm transformer block recorded on the
libxt tape (Python only marshals: every step runs in libxt's kernels).

[AE] "Attention 用组合": attention is the composition
softmax(scale(Q K^T, 1/sqrt(Dh))) V of matmul / softmax nodes, so its backward
comes from the tape; no fused attention backward exists.  Here the scale is
the softmax pre-scale and K^T is the matmul's transposed-operand flag, so no
transpose node is needed.  Heads are strided views of the [B*S, H*Dh]
projections (no copies); the P.V product writes straight into a [B*S, H*Dh]
matrix.

The block follows the pre-norm wiring of "Phase T18: Dropout" ("dropout 接在哪"):
    h  = x + dropout(attn(rms_norm(x)))          site 0xA77
    h2 = h + dropout(swiglu_mlp(rms_norm(h)))    site 0xF70
    loss = cross_entropy(rms_norm(h2) @ W_out, targets)
with per-site seeds base_seed ^ layer ^ site ("每个 dropout 站点的确定性 seed").
"""
from __future__ import annotations

import math
from dataclasses import dataclass

from . import OP, DT, Tape, Tensor, params, view

SITE_ATTN = 0xA77
SITE_FFN = 0xF70


@dataclass
class BlockShape:
    B: int
    S: int
    H: int
    Dh: int
    hidden: int
    vocab: int

    @property
    def D(self) -> int:
        return self.H * self.Dh


def layout(rows, cols, ld, dtype, nb=(1, 1), sb=(0, 0), offset=0) -> Tensor:
    v = Tensor()
    v.data = offset
    v.dtype = dtype
    v.rows, v.cols, v.ld = rows, cols, ld
    v.nb[0], v.nb[1] = nb
    v.sb[0], v.sb[1] = sb
    return v


def attention(tape: Tape, q: int, k: int, v: int, B: int, S: int, H: int, Dh: int, dtype: int,
              causal: bool = True) -> int:
    """Causal multi-head attention over [B*S, H*Dh] projections; returns the
    [B*S, H*Dh] output var."""
    D = H * Dh
    heads = layout(S, Dh, D, dtype, (B, H), (S * D, Dh))
    qh, kh, vh = (tape.view(t, heads) for t in (q, k, v))
    scores = tape.apply(OP.MATMUL, params(trans_b=1), qh, kh)                 # [B, H, S, S]
    flat = tape.view(scores, layout(B * H * S, S, S, dtype))
    probs = tape.apply(OP.SOFTMAX, params(alpha=1.0 / math.sqrt(Dh), causal=int(causal), seq_len=S), flat)
    ph = tape.view(probs, layout(S, S, S, dtype, (B, H), (H * S * S, S * S)))
    out = tape.apply(OP.MATMUL, params(), ph, vh, layout=layout(S, Dh, D, dtype, (B, H), (S * D, Dh)))
    return tape.view(out, layout(B * S, D, D, dtype))


def fused_attention(tape: Tape, q: int, k: int, v: int, S: int, Dh: int, causal: bool = True) -> int:
    """The same attention as one fused op (no [S, S] probabilities stored)."""
    return tape.apply(OP.ATTENTION, params(alpha=1.0 / math.sqrt(Dh), causal=int(causal), seq_len=S, head_dim=Dh),
                      q, k, v)


def block_layer(tape: Tape, w: dict, x: int, shp: BlockShape, dtype: int, p_drop: float = 0.0,
                base_seed: int = 0, layer_index: int = 0, eps: float = 1e-5, checkpoint: bool = False,
                taps: dict | None = None, fused_attention_op: bool = False) -> int:
    """Records the two residual halves of one layer; returns h2.  With
    `checkpoint`, the layer is one recompute segment whose output is h2.
    `taps` (optional) receives the vars of n1 and of the two dropout nodes."""
    if checkpoint:
        tape.checkpoint_begin()
    mm = params()
    n1 = tape.apply(OP.RMS_NORM, params(eps=eps), x, w["g1"])
    rope = params(head_dim=shp.Dh, seq_len=shp.S, rope_base=10000.0)
    q = tape.apply(OP.ROPE, rope, tape.apply(OP.MATMUL, mm, n1, w["wq"]))
    k = tape.apply(OP.ROPE, rope, tape.apply(OP.MATMUL, mm, n1, w["wk"]))
    v = tape.apply(OP.MATMUL, mm, n1, w["wv"])
    att = (fused_attention(tape, q, k, v, shp.S, shp.Dh) if fused_attention_op
           else attention(tape, q, k, v, shp.B, shp.S, shp.H, shp.Dh, dtype))
    a = tape.apply(OP.MATMUL, mm, att, w["wo"])
    a = tape.apply(OP.DROPOUT, params(p=p_drop, seed=base_seed ^ layer_index ^ SITE_ATTN), a)
    h = tape.apply(OP.ADD, params(), x, a)
    n2 = tape.apply(OP.RMS_NORM, params(eps=eps), h, w["g2"])
    m = tape.apply(OP.SWIGLU, params(), tape.apply(OP.MATMUL, mm, n2, w["wg"]),
                   tape.apply(OP.MATMUL, mm, n2, w["wu"]))
    m = tape.apply(OP.MATMUL, mm, m, w["wd"])
    m = tape.apply(OP.DROPOUT, params(p=p_drop, seed=base_seed ^ layer_index ^ SITE_FFN), m)
    h2 = tape.apply(OP.ADD, params(), h, m)
    if taps is not None:
        taps.update(n1=n1, drop_attn=a, drop_ffn=m)
    if checkpoint:
        tape.checkpoint_end(h2)
    return h2


def block(tape: Tape, w: dict, x: int, targets: int, shp: BlockShape, dtype: int,
          p_drop: float = 0.0, base_seed: int = 0, layer: int = 0, eps: float = 1e-5,
          checkpoint: bool = False, fused_attention: bool = False) -> int:
    """Records the block; `w` maps g1 g2 g3 wq wk wv wo wg wu wd wout to leaf vars.
    Returns the loss var."""
    h2 = block_layer(tape, w, x, shp, dtype, p_drop, base_seed, layer, eps, checkpoint,
                     fused_attention_op=fused_attention)
    logits = tape.apply(OP.MATMUL, params(), tape.apply(OP.RMS_NORM, params(eps=eps), h2, w["g3"]), w["wout"])
    return tape.apply(OP.CROSS_ENTROPY, params(), logits, targets)


WEIGHT_SHAPES = lambda s: {  # noqa: E731
    "g1": (s.D,), "g2": (s.D,), "g3": (s.D,),
    "wq": (s.D, s.D), "wk": (s.D, s.D), "wv": (s.D, s.D), "wo": (s.D, s.D),
    "wg": (s.D, s.hidden), "wu": (s.D, s.hidden), "wd": (s.hidden, s.D), "wout": (s.D, s.vocab),
}


def leaves(tape: Tape, tensors: dict) -> dict:
    """Leaf vars (requires grad) over torch tensors."""
    return {k: tape.leaf(view(t)) for k, t in tensors.items()}
