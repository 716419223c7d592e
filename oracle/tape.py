"""A tiny reverse-mode tape for the oracle, in float64.

[AE] "Tape 设计" and "梯度累加（扇出求和）": each op records a node (its
parents and how to push its gradient back); backward seeds the scalar loss
with 1 and visits nodes so that every node is finished before its parents;
a gradient reaching a node from several consumers is summed, and a node
used twice by the same op (mul(x, x)) receives both contributions.

This tape is deliberately built differently from the library's: nodes live
in an index arena in creation order and the backward walks that order in
reverse ([AD] section 3.3: a node is always created after its inputs, so
reverse creation order is a valid reverse topological order).  Every
contribution is added with one f64 rounding, in push order.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, List, Optional

import numpy as np

from . import ops, rng


@dataclass
class _Node:
    value: np.ndarray
    parents: List[int] = field(default_factory=list)
    backward: Optional[Callable] = None      # d -> list of parent grads (None = no grad)
    grad: Optional[np.ndarray] = None


class Tape:
    def __init__(self):
        self.nodes: List[_Node] = []

    # -- recording --------------------------------------------------------
    def _push(self, value, parents=(), backward=None) -> int:
        self.nodes.append(_Node(np.asarray(value, dtype=np.float64), list(parents), backward))
        return len(self.nodes) - 1

    def leaf(self, value) -> int:
        return self._push(np.array(value, dtype=np.float64, copy=True))

    def value(self, i: int) -> np.ndarray:
        return self.nodes[i].value

    def grad(self, i: int) -> Optional[np.ndarray]:
        return self.nodes[i].grad

    def _v(self, i):
        return self.nodes[i].value

    def matmul(self, a, b, alpha=1.0, trans_a=False, trans_b=False):
        A, B = self._v(a), self._v(b)
        return self._push(ops.matmul(A, B, alpha, trans_a, trans_b), [a, b],
                          lambda d: list(ops.matmul_bwd(d, A, B, alpha, trans_a, trans_b)))

    def add(self, a, b):
        return self._push(ops.add(self._v(a), self._v(b)), [a, b],
                          lambda d: list(ops.add_bwd(d)))

    def mul(self, a, b):
        A, B = self._v(a), self._v(b)
        return self._push(ops.mul(A, B), [a, b], lambda d: list(ops.mul_bwd(d, A, B)))

    def scale(self, x, alpha):
        return self._push(ops.scale(self._v(x), alpha), [x],
                          lambda d: [ops.scale_bwd(d, alpha)])

    def add_bias(self, x, bias):
        return self._push(ops.add_bias(self._v(x), self._v(bias)), [x, bias],
                          lambda d: list(ops.add_bias_bwd(d)))

    def rms_norm(self, x, gamma, eps):
        X, G = self._v(x), self._v(gamma)
        y, ir = ops.rms_norm(X, G, eps)
        return self._push(y, [x, gamma], lambda d: list(ops.rms_norm_bwd(d, X, G, ir)))

    def layer_norm(self, x, gamma, beta, eps):
        X, G, B = self._v(x), self._v(gamma), self._v(beta)
        y, mu, rs = ops.layer_norm(X, G, B, eps)
        return self._push(y, [x, gamma, beta],
                          lambda d: list(ops.layer_norm_bwd(d, X, G, mu, rs)))

    def softmax(self, x, alpha=1.0, causal=False, seq_len=0):
        y = ops.softmax(self._v(x), alpha, causal, seq_len)
        return self._push(y, [x], lambda d: [ops.softmax_bwd(d, y, alpha)])

    def cross_entropy(self, x, targets):
        X = self._v(x)
        t = np.asarray(targets)
        L, lse, _ = ops.cross_entropy(X, t)
        return self._push(np.array([L]), [x],
                          lambda d: [ops.cross_entropy_bwd(float(np.asarray(d).reshape(-1)[0]), X, t, lse)])

    def silu(self, x):
        X = self._v(x)
        return self._push(ops.silu(X), [x], lambda d: [ops.silu_bwd(d, X)])

    def gelu(self, x):
        X = self._v(x)
        return self._push(ops.gelu(X), [x], lambda d: [ops.gelu_bwd(d, X)])

    def swiglu(self, g, u):
        G, U = self._v(g), self._v(u)
        return self._push(ops.swiglu(G, U), [g, u], lambda d: list(ops.swiglu_bwd(d, G, U)))

    def rope(self, x, head_dim, base, seq_len):
        return self._push(ops.rope(self._v(x), head_dim, base, seq_len), [x],
                          lambda d: [ops.rope_bwd(d, head_dim, base, seq_len)])

    def embed(self, table, ids):
        """Token embedding ([BP] k_embed_fwd / k_embed_bwd); ids are data,
        not a node."""
        E = self._v(table)
        t = np.asarray(ids).reshape(-1)
        return self._push(ops.embed(E, t), [table], lambda d: [ops.embed_bwd(d, t, E.shape[0])])

    def dropout(self, x, p, seed):
        if p == 0.0:                     # [DO]: p == 0 records nothing
            return x
        y, mask = rng.dropout(self._v(x), p, seed)
        return self._push(y, [x], lambda d: [rng.dropout_bwd(d, mask, p)])

    def sum(self, x):
        """Scalar sum of all elements (used to build test losses)."""
        X = self._v(x)
        return self._push(np.array([X.sum()]), [x],
                          lambda d: [np.full(X.shape, float(np.asarray(d).reshape(-1)[0]))])

    # -- reverse pass ---------------------------------------------------------
    def backward(self, loss: int):
        if self.nodes[loss].value.size != 1:
            raise ValueError("loss must hold exactly one element")
        # Intermediate gradients belong to one pass; leaf gradients keep
        # accumulating across passes until zero_grad ([BP] "Ackumulation
        # över mikrobatcher": backward adds into the buffers).
        for n in self.nodes:
            if n.backward is not None:
                n.grad = None
        seed = np.ones_like(self.nodes[loss].value)
        self._accumulate(loss, seed)
        for i in range(loss, -1, -1):
            node = self.nodes[i]
            if node.backward is None or node.grad is None:
                continue
            contribs = node.backward(node.grad)
            for p, g in zip(node.parents, contribs):
                self._accumulate(p, g)

    def _accumulate(self, i: int, g):
        node = self.nodes[i]
        g = np.asarray(g, dtype=np.float64).reshape(node.value.shape)
        node.grad = g.copy() if node.grad is None else node.grad + g

    def zero_grad(self):
        for n in self.nodes:
            n.grad = None
