"""The small pre-norm transformer block on the oracle tape (test-side
composition of oracle ops only).  Heads are handled by explicit per-(batch,
head) slices -- a different construction from the library's strided views.

  h  = x + dropout(attn(rms_norm(x))),   seed base ^ layer ^ 0xA77
  h2 = h + dropout(swiglu_mlp(rms_norm(h))), seed base ^ layer ^ 0xF70
  loss = cross_entropy(rms_norm(h2) @ W_out, targets)
(wiring of "Phase T18: Dropout", "dropout 接在哪"; seeds of
"每个 dropout 站点的确定性 seed"; attention of [AE] "Attention 用组合").
"""
import numpy as np

from oracle.tape import Tape


def _attention(t, q, k, v, S, Dh):
    scores = t.matmul(q, k, 1.0, False, True)
    probs = t.softmax(t.scale(scores, 1.0 / np.sqrt(Dh)), 1.0, True, S)
    return t.matmul(probs, v)


def _slice(t, z, sl):
    shape = t.value(z).shape

    def back(d):
        g = np.zeros(shape)
        g[sl] = d
        return [g]
    return t._push(t.value(z)[sl], [z], back)


def _concat(t, heads, shape):
    val = np.zeros(shape)
    for sl, node in heads:
        val[sl] = t.value(node)
    sls = [sl for sl, _ in heads]
    return t._push(val, [n for _, n in heads], lambda d: [d[sl] for sl in sls])


def block_loss(params, x0, targets, B, S, H, Dh, p_drop=0.0, base_seed=0, layer=0, eps=1e-5):
    """Returns (tape, param leaf ids, x leaf id, loss id)."""
    t = Tape()
    P = {k: t.leaf(v) for k, v in params.items()}
    x = t.leaf(x0)
    D = H * Dh
    n1 = t.rms_norm(x, P["g1"], eps)
    q = t.rope(t.matmul(n1, P["wq"]), Dh, 10000.0, S)
    k = t.rope(t.matmul(n1, P["wk"]), Dh, 10000.0, S)
    v = t.matmul(n1, P["wv"])
    heads = []
    for b in range(B):
        for hh in range(H):
            sl = (slice(b * S, (b + 1) * S), slice(hh * Dh, (hh + 1) * Dh))
            heads.append((sl, _attention(t, _slice(t, q, sl), _slice(t, k, sl), _slice(t, v, sl), S, Dh)))
    cat = _concat(t, heads, (B * S, D))
    h = t.add(x, t.dropout(t.matmul(cat, P["wo"]), p_drop, base_seed ^ layer ^ 0xA77))
    n2 = t.rms_norm(h, P["g2"], eps)
    m = t.matmul(t.swiglu(t.matmul(n2, P["wg"]), t.matmul(n2, P["wu"])), P["wd"])
    h2 = t.add(h, t.dropout(m, p_drop, base_seed ^ layer ^ 0xF70))
    logits = t.matmul(t.rms_norm(h2, P["g3"], eps), P["wout"])
    return t, P, x, t.cross_entropy(logits, targets)
