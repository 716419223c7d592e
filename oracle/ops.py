"""Forward ops and their hand-derived backward passes, in float64.

Conventions: every tensor is a numpy array; row-wise ops act on the last axis
(rows = everything before it).  ``d`` is the upstream gradient (the gradient
of the loss with respect to the op's output).  Each backward returns the
gradient of every differentiable input, in input order.

Tags [AE], [BP], [DO] name the pages; see the package docstring.
"""
from __future__ import annotations

import math

import numpy as np


def _f(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _t(a: np.ndarray) -> np.ndarray:
    return np.swapaxes(a, -1, -2)


# --------------------------------------------------------------------------
# matmul  -- [AE] op-backward table, row "matmul": C = A@B, dA = d@B^T,
# dB = A^T@d.  ``alpha`` scales the product (the attention scale folded in),
# ``trans_*`` read an operand transposed; leading axes are batch axes.
# --------------------------------------------------------------------------
def matmul(a, b, alpha: float = 1.0, trans_a: bool = False, trans_b: bool = False):
    A, B = _f(a), _f(b)
    opA = _t(A) if trans_a else A
    opB = _t(B) if trans_b else B
    return alpha * np.matmul(opA, opB)


def matmul_bwd(d, a, b, alpha: float = 1.0, trans_a: bool = False, trans_b: bool = False):
    D, A, B = _f(d), _f(a), _f(b)
    opA = _t(A) if trans_a else A
    opB = _t(B) if trans_b else B
    d_opA = alpha * np.matmul(D, _t(opB))
    d_opB = alpha * np.matmul(_t(opA), D)
    dA = _t(d_opA) if trans_a else d_opA
    dB = _t(d_opB) if trans_b else d_opB
    return dA, dB


# --------------------------------------------------------------------------
# add / mul / scale / add_bias -- [AE] op-backward table rows of the same
# names.  add_bias broadcasts bias over rows; its gradient sums d over the
# broadcast (row) axis.  Residual add is [BP]'s k_residual_add pair.
# --------------------------------------------------------------------------
def add(a, b):
    return _f(a) + _f(b)


def add_bwd(d):
    D = _f(d)
    return D.copy(), D.copy()


def mul(a, b):
    return _f(a) * _f(b)


def mul_bwd(d, a, b):
    D = _f(d)
    return D * _f(b), D * _f(a)


def scale(x, alpha: float):
    return alpha * _f(x)


def scale_bwd(d, alpha: float):
    return alpha * _f(d)


def add_bias(x, bias):
    return _f(x) + _f(bias)[None, :]


def add_bias_bwd(d):
    D = _f(d)
    return D.copy(), D.sum(axis=0)


# --------------------------------------------------------------------------
# rms_norm -- [AE] "RMSNorm" paragraph: ir = 1/sqrt(mean_c x^2 + eps),
# y = x * ir * gamma; with g = d*gamma and n = cols,
# dx = ir*g - x*ir^3/n * sum_c(g*x),  dgamma = sum_r d*x*ir.
# The forward keeps ir per row so the backward reuses it.
# --------------------------------------------------------------------------
def rms_norm(x, gamma, eps: float):
    X, G = _f(x), _f(gamma)
    ms = np.mean(X * X, axis=1)
    ir = 1.0 / np.sqrt(ms + eps)
    return X * ir[:, None] * G[None, :], ir


def rms_norm_bwd(d, x, gamma, inv_rms):
    D, X, G, ir = _f(d), _f(x), _f(gamma), _f(inv_rms)
    n = X.shape[1]
    g = D * G[None, :]
    dot = np.sum(g * X, axis=1)
    dx = ir[:, None] * g - X * (ir ** 3 / n * dot)[:, None]
    dgamma = np.sum(D * X * ir[:, None], axis=0)
    return dx, dgamma


# --------------------------------------------------------------------------
# layer_norm -- [BP] kernel pair k_layernorm_fwd/k_layernorm_bwd and
# "Sparade tensorer" (the backward needs the mean and variance of the
# forward).  Reading: textbook LayerNorm with the biased variance (divide by
# cols), eps inside the square root, mean and rstd = 1/sqrt(var+eps) saved.
#   xhat = (x-mu)*rstd, y = xhat*gamma + beta
#   g = d*gamma, dx = rstd*(g - mean(g) - xhat*mean(g*xhat)),
#   dgamma = sum_r d*xhat, dbeta = sum_r d.
# --------------------------------------------------------------------------
def layer_norm(x, gamma, beta, eps: float):
    X, G, B = _f(x), _f(gamma), _f(beta)
    mu = np.mean(X, axis=1)
    var = np.mean((X - mu[:, None]) ** 2, axis=1)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (X - mu[:, None]) * rstd[:, None]
    return xhat * G[None, :] + B[None, :], mu, rstd


def layer_norm_bwd(d, x, gamma, mean, rstd):
    D, X, G = _f(d), _f(x), _f(gamma)
    mu, rs = _f(mean), _f(rstd)
    xhat = (X - mu[:, None]) * rs[:, None]
    g = D * G[None, :]
    dx = rs[:, None] * (g - np.mean(g, axis=1)[:, None]
                        - xhat * np.mean(g * xhat, axis=1)[:, None])
    return dx, np.sum(D * xhat, axis=0), np.sum(D, axis=0)


# --------------------------------------------------------------------------
# softmax -- [AE] op-backward table row "softmax" and the "Softmax 反向推导"
# derivation: y = row-wise safe softmax, dx = y*(d - sum_c d*y).
# Readings: ``alpha`` pre-scales the logits (softmax(alpha*x), whose
# gradient gains the factor alpha); ``causal`` excludes columns past the
# query index (row mod seq_len) from the max and the sum and gives them y=0.
# --------------------------------------------------------------------------
def causal_keep(rows: int, cols: int, seq_len: int) -> np.ndarray:
    q = np.arange(rows) % seq_len
    return np.arange(cols)[None, :] <= q[:, None]


def softmax(x, alpha: float = 1.0, causal: bool = False, seq_len: int = 0):
    Z = alpha * _f(x)
    if causal:
        keep = causal_keep(Z.shape[0], Z.shape[1], seq_len)
        Z = np.where(keep, Z, -np.inf)
    m = np.max(Z, axis=1, keepdims=True)
    e = np.exp(Z - m)
    return e / np.sum(e, axis=1, keepdims=True)


def softmax_bwd(d, y, alpha: float = 1.0):
    D, Y = _f(d), _f(y)
    return alpha * Y * (D - np.sum(D * Y, axis=1, keepdims=True))


# --------------------------------------------------------------------------
# cross_entropy -- [AE] op-backward table row "cross_entropy" and the
# "Cross-entropy 反向推导": L = mean over rows of -log softmax(x_r)[t_r];
# dx = (softmax(x) - onehot(t)) / rows, times the upstream scalar.
# Readings: the forward returns lse_r = log sum_c exp(x_rc) (the backward
# rebuilds softmax as exp(x - lse)), the per-row losses and their mean; a
# target outside [0, cols) makes that row's loss and gradient NaN.
# --------------------------------------------------------------------------
def cross_entropy(x, targets):
    X = _f(x)
    t = np.asarray(targets, dtype=np.int64)
    R, V = X.shape
    m = np.max(X, axis=1)
    lse = m + np.log(np.sum(np.exp(X - m[:, None]), axis=1))
    ok = (t >= 0) & (t < V)
    picked = np.where(ok, X[np.arange(R), np.clip(t, 0, V - 1)], np.nan)
    loss_row = lse - picked
    return float(np.mean(loss_row)) if R else float("nan"), lse, loss_row


def cross_entropy_bwd(g: float, x, targets, lse):
    X = _f(x)
    t = np.asarray(targets, dtype=np.int64)
    R, V = X.shape
    p = np.exp(X - _f(lse)[:, None])
    ok = (t >= 0) & (t < V)
    p[np.arange(R)[ok], t[ok]] -= 1.0
    p[~ok, :] = np.nan
    return p * (float(g) / R)


# --------------------------------------------------------------------------
# silu / swiglu -- [AE] op-backward table rows "silu" (y = x*s(x),
# dx = d*(s + x*s*(1-s))) and "swiglu" (silu(g)*u, whose gradient is what
# the silu and mul rows give when composed).
# --------------------------------------------------------------------------
def sigmoid(x):
    X = _f(x)
    return 1.0 / (1.0 + np.exp(-X))


def silu(x):
    X = _f(x)
    return X * sigmoid(X)


def silu_bwd(d, x):
    X = _f(x)
    s = sigmoid(X)
    return _f(d) * (s + X * s * (1.0 - s))


def swiglu(g, u):
    return silu(g) * _f(u)


def swiglu_bwd(d, g, u):
    D = _f(d)
    dg = silu_bwd(D * _f(u), g)     # chain through mul then silu
    du = D * silu(g)
    return dg, du


# --------------------------------------------------------------------------
# gelu -- [BP] kernel pair k_mlp_fwd/k_mlp_bwd ("MLP (med GELU)"), whose
# backward needs the pre-activation.  Reading: the exact form
# y = x*Phi(x), Phi the standard normal CDF, dx = d*(Phi(x) + x*phi(x)).
# --------------------------------------------------------------------------
_erfc = np.vectorize(math.erfc, otypes=[np.float64])


def normal_cdf(x):
    # Phi(x) = erfc(-x/sqrt 2)/2 (no cancellation in the lower tail)
    return 0.5 * _erfc(-_f(x) / math.sqrt(2.0))


def normal_pdf(x):
    X = _f(x)
    return np.exp(-0.5 * X * X) / math.sqrt(2.0 * math.pi)


def gelu(x):
    X = _f(x)
    return X * normal_cdf(X)


def gelu_bwd(d, x):
    X = _f(x)
    return _f(d) * (normal_cdf(X) + X * normal_pdf(X))


# Reading: the op's optional tanh form (Hendrycks & Gimpel's approximation
# of x*Phi(x)), g(x) = x (1 + tanh u)/2 with u = sqrt(2/pi) (x + 0.044715 x^3),
# and its derivative by the product and chain rules.
_GELU_K = math.sqrt(2.0 / math.pi)


def gelu_tanh(x):
    X = _f(x)
    return 0.5 * X * (1.0 + np.tanh(_GELU_K * (X + 0.044715 * X ** 3)))


def gelu_tanh_bwd(d, x):
    X = _f(x)
    t = np.tanh(_GELU_K * (X + 0.044715 * X ** 3))
    du = _GELU_K * (1.0 + 3.0 * 0.044715 * X * X)
    return _f(d) * (0.5 * (1.0 + t) + 0.5 * X * (1.0 - t * t) * du)


# --------------------------------------------------------------------------
# rope -- [AE] op-backward table row "rope" and "RoPE 反向推导": each pair is
# rotated by the 2x2 rotation R(theta); R is orthogonal, so the backward
# applies R(-theta):  dx_i = d_i cos + d_{i+h} sin,
# dx_{i+h} = d_{i+h} cos - d_i sin; position 0 is the identity.
# Readings: rotate-half pairing (i, i+Dh/2) inside each head of width Dh;
# theta_{pos,i} = pos * base^(-2i/Dh), i in [0, Dh/2); pos = row mod seq_len.
# --------------------------------------------------------------------------
def rope_angles(positions, head_dim: int, base: float) -> np.ndarray:
    half = head_dim // 2
    inv_freq = np.power(float(base), -2.0 * np.arange(half, dtype=np.float64) / head_dim)
    return np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]


def _rope(x, head_dim, base, seq_len, sign, positions=None):
    X = _f(x)
    R, C = X.shape
    half = head_dim // 2
    pos = np.arange(R) % seq_len if positions is None else np.asarray(positions)
    th = rope_angles(pos, head_dim, base)                          # [R, half]
    c, s = np.cos(th), sign * np.sin(th)
    Xh = X.reshape(R, C // head_dim, head_dim)
    a, b = Xh[:, :, :half], Xh[:, :, half:]
    ya = a * c[:, None, :] - b * s[:, None, :]
    yb = a * s[:, None, :] + b * c[:, None, :]
    return np.concatenate([ya, yb], axis=2).reshape(R, C)


def rope(x, head_dim: int, base: float, seq_len: int, positions=None):
    """``positions`` (one per row) overrides row mod seq_len, e.g. for a
    sample of rows taken out of a longer batch."""
    return _rope(x, head_dim, base, seq_len, +1.0, positions)


def rope_bwd(d, head_dim: int, base: float, seq_len: int, positions=None):
    return _rope(d, head_dim, base, seq_len, -1.0, positions)


# --------------------------------------------------------------------------
# grad accumulate -- [AE] "梯度累加（扇出求和）": a second gradient reaching
# a tensor is added to the first; [BP] "Ackumulation över mikrobatcher":
# backward adds into the buffer instead of overwriting it.
# --------------------------------------------------------------------------
def grad_accumulate(dst, src):
    return _f(dst) + _f(src)


# --------------------------------------------------------------------------
# Gradient buffers after the backward -- [BP] kernel-pair table (the helper
# kernels k_grad_norm_partial, k_grad_norm_final and k_grad_scale, named for
# gradient clipping) and "Ackumulation över mikrobatcher" (scale_grads(1/n)
# averages the microbatch sum, zero_grads() clears the buffers).
# Readings (the pages name the kernels only):
#   * the norm is the global L2 norm over every element of every gradient
#     tensor, sqrt(sum g^2);
#   * clipping follows Pascanu, Mikolov & Bengio, "On the difficulty of
#     training recurrent neural networks" (2013), section 3.2: when the norm
#     exceeds the threshold, every gradient is multiplied by threshold/norm;
#     otherwise (or with no threshold, max_norm <= 0) the factor is 1;
#   * a scaled element is the f32 product of the stored value and the f32
#     factor, rounded once into the storage type (for bf16: the f32 product
#     rounded to bf16).
# --------------------------------------------------------------------------
def grad_norm(grads):
    """sqrt of the sum of squares of every element of every tensor in the
    list (an empty list has norm 0)."""
    total = 0.0
    for g in grads:
        G = _f(g)
        total += float(np.sum(G * G))
    return math.sqrt(total)


def clip_coefficient(norm: float, max_norm: float) -> float:
    if max_norm > 0 and norm > max_norm:
        return max_norm / norm
    return 1.0


def scale_grad(g, factor: float, dtype: str = "f32"):
    """One gradient tensor times ``factor`` (an f32 value), as stored."""
    from .numerics import round_bf16, round_f32
    prod = _f(g) * float(np.float32(factor))
    return round_bf16(prod) if dtype == "bf16" else round_f32(prod)


# --------------------------------------------------------------------------
# Token embedding -- [BP] kernel-pair table (k_embed_fwd / k_embed_bwd,
# "token-inbäddningsuppslag") and the forward of "Framåtgåendet"
# (x = embed(token_ids), and the tied output projection LN(x) @ embed^T,
# whose gradient reaches the same table as a second contribution).
#   y[r, :] = E[ids[r], :];   dE[v, :] = sum over r with ids[r] = v of d[r, :]
# Readings: ids are int32; an id outside [0, V) gives a NaN output row and
# contributes nothing to dE; the sum runs over r in increasing order.
# --------------------------------------------------------------------------
def embed(table, ids):
    E = _f(table)
    ids = np.asarray(ids).reshape(-1)
    V, D = E.shape
    y = np.full((ids.size, D), np.nan)
    for r, v in enumerate(ids):
        if 0 <= v < V:
            y[r] = E[v]
    return y


def embed_bwd(d, ids, vocab: int):
    D_ = _f(d)
    ids = np.asarray(ids).reshape(-1)
    dE = np.zeros((vocab, D_.shape[1]))
    for r, v in enumerate(ids):
        if 0 <= v < vocab:
            dE[v] += D_[r]
    return dE


# --------------------------------------------------------------------------
# Fused attention -- [AE] "Attention 用组合": attention is
# softmax(scale(Q K^T, alpha) [+ causal]) V, whose backward the tape derives
# from the matmul and softmax rows of the op-backward table.  The fused form
# computes the same thing per (sequence, head) without materialising the
# probabilities; its saved row statistic is the log-sum-exp of the scaled,
# masked scores (the softmax normaliser), from which the backward rebuilds
# the probabilities.
# Layout (a reading): q, k, v and the output are [B*S, H*Dh] matrices, row
# b*S + s holding token s of sequence b, columns h*Dh .. h*Dh+Dh-1 head h;
# the log-sum-exp is [B*S, H].  Causal: key t is visible to query s iff
# t <= s.
# --------------------------------------------------------------------------
def _heads(x, S, H, Dh):
    X = _f(x)
    B = X.shape[0] // S
    return X.reshape(B, S, H, Dh).transpose(0, 2, 1, 3)          # [B, H, S, Dh]


def _unheads(x):
    B, H, S, Dh = x.shape
    return x.transpose(0, 2, 1, 3).reshape(B * S, H * Dh)


def _probs(Q, K, seq_len, alpha, causal):
    """P = softmax(alpha Q K^T) over keys, masked keys (t > s) at probability 0."""
    Z = alpha * np.matmul(Q, np.swapaxes(K, -1, -2))
    if causal:
        keep = np.arange(seq_len)[None, :] <= np.arange(seq_len)[:, None]
        Z = np.where(keep, Z, -np.inf)
    e = np.exp(Z - np.max(Z, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def attention(q, k, v, seq_len: int, heads: int, head_dim: int, alpha: float, causal: bool = True):
    """Returns (out [B*S, H*Dh], lse [B*S, H])."""
    Q, K, Vv = (_heads(t, seq_len, heads, head_dim) for t in (q, k, v))
    Z = alpha * np.matmul(Q, np.swapaxes(K, -1, -2))               # [B, H, S, S]
    if causal:
        keep = np.arange(seq_len)[None, :] <= np.arange(seq_len)[:, None]
        Z = np.where(keep, Z, -np.inf)
    m = np.max(Z, axis=-1, keepdims=True)
    e = np.exp(Z - m)
    s = np.sum(e, axis=-1, keepdims=True)
    P = e / s
    lse = (m + np.log(s))[..., 0]                                  # [B, H, S]
    out = _unheads(np.matmul(P, Vv))
    return out, lse.transpose(0, 2, 1).reshape(-1, heads)


def attention_bwd(d, q, k, v, seq_len: int, heads: int, head_dim: int, alpha: float, causal: bool = True,
                  out=None):
    """(dq, dk, dv) by the composition's chain rule: P = softmax(alpha Q K^T),
    dV = P^T dO, dP = dO V^T, dZ = P (dP - rowsum(dP P)), dQ = alpha dZ K,
    dK = alpha dZ^T Q.

    rowsum(dP P) = rowsum(dO (P V)) = rowsum(dO O): given ``out`` (the
    forward output as it was stored, e.g. rounded to bf16), the row term is
    formed from it, as a backward that reads the saved output does; without
    it, from the exact P."""
    Q, K, Vv = (_heads(t, seq_len, heads, head_dim) for t in (q, k, v))
    dO = _heads(d, seq_len, heads, head_dim)
    P = _probs(Q, K, seq_len, alpha, causal)
    dV = np.matmul(np.swapaxes(P, -1, -2), dO)
    dP = np.matmul(dO, np.swapaxes(Vv, -1, -2))
    if out is None:
        Drow = np.sum(dP * P, axis=-1, keepdims=True)
    else:
        Drow = np.sum(dO * _heads(out, seq_len, heads, head_dim), axis=-1, keepdims=True)
    dZ = P * (dP - Drow)
    dQ = alpha * np.matmul(dZ, K)
    dK = alpha * np.matmul(np.swapaxes(dZ, -1, -2), Q)
    return _unheads(dQ), _unheads(dK), _unheads(dV)


def attention_term_magnitudes(d, q, k, v, seq_len: int, heads: int, head_dim: int, alpha: float,
                              causal: bool = True):
    """For each output of the attention forward and backward, the sum of the
    magnitudes of the terms it adds up: out = sum_t P V_t, dv = sum_s P dO_s,
    and dq = alpha sum_t dZ K_t, dk = alpha sum_s dZ Q_s with each dZ = P dP -
    P D itself two terms (D = rowsum(dP P)).  Returns (|P| |V|, alpha |Z'|
    |K|, alpha |Z'|^T |Q|, |P|^T |dO|) with Z' = P (|dP| + |D|), in the
    [B*S, H*Dh] layout: the size of a long sum, against which its rounding
    error is judged (a sum near zero is still judged at the size of its
    terms)."""
    Q, K, Vv = (_heads(t, seq_len, heads, head_dim) for t in (q, k, v))
    dO = _heads(d, seq_len, heads, head_dim)
    P = _probs(Q, K, seq_len, alpha, causal)
    dP = np.matmul(dO, np.swapaxes(Vv, -1, -2))
    dZ = P * (np.abs(dP) + np.abs(np.sum(dP * P, axis=-1, keepdims=True)))
    return (_unheads(np.matmul(P, np.abs(Vv))), _unheads(alpha * np.matmul(dZ, np.abs(K))),
            _unheads(alpha * np.matmul(np.swapaxes(dZ, -1, -2), np.abs(Q))),
            _unheads(np.matmul(np.swapaxes(P, -1, -2), np.abs(dO))))
