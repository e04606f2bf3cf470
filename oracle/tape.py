"""A small reverse-mode autodiff tape over fp64 NumPy arrays.

TEST INFRASTRUCTURE (see the package header).  It exists to check the
hand-derived adjoints in ``oracle.ssm`` and ``oracle.layer`` by an independent
derivation: the forward is rebuilt from primitive ops, unrolled over time, and
differentiated mechanically.

Rules follow luma-tensor 0.0.1 ``src/grad/backprop.rs``: ``Tensor::backward``
(seed the output, walk nodes in reverse topological order, accumulate into a
gradient store), ``sorted_nodes`` (depth-first topological order of the nodes
that reach a leaf; written iteratively here, since a graph unrolled over time
is deeper than Python's recursion limit), ``backward_op`` (Add, Sub, Mul, Div,
scalar-operand forms, Neg, Affine, Matmul, Broadcast, Reshape, Transpose,
Narrow, Cat) and ``backward_unary`` / ``backward_reduce`` (Exp, Ln, Sqr, Sqrt,
Recip, Sigmoid, Silu; Sum, Mean).  Where the page seeds the output with ones,
``backward`` takes the cotangent, so that one call gives the vector-Jacobian
product that the oracle computes.
"""
from __future__ import annotations

import numpy as np


class Node:
    __slots__ = ("value", "op", "args", "meta", "__weakref__")

    def __init__(self, value, op=None, args=(), meta=None):
        self.value = np.asarray(value, dtype=np.float64)
        self.op = op
        self.args = tuple(args)
        self.meta = meta

    @property
    def shape(self):
        return self.value.shape


def leaf(x) -> Node:
    return Node(np.array(x, dtype=np.float64, copy=True))


def _same(a: Node, b: Node):
    if a.shape != b.shape:
        raise ValueError(f"shape mismatch {a.shape} vs {b.shape}; broadcast explicitly")


# ---- binary tensor-tensor -------------------------------------------------
def add(a, b):
    _same(a, b)
    return Node(a.value + b.value, "add", (a, b))


def sub(a, b):
    _same(a, b)
    return Node(a.value - b.value, "sub", (a, b))


def mul(a, b):
    _same(a, b)
    return Node(a.value * b.value, "mul", (a, b))


def div(a, b):
    _same(a, b)
    return Node(a.value / b.value, "div", (a, b))


# ---- scalar operand --------------------------------------------------------
def add_scalar(a, c: float):
    return Node(a.value + c, "add_s", (a,), c)


def mul_scalar(a, c: float):
    return Node(a.value * c, "mul_s", (a,), c)


def neg(a):
    return Node(-a.value, "neg", (a,))


def affine(a, m: float, c: float):
    return Node(a.value * m + c, "affine", (a,), (m, c))


# ---- unary -----------------------------------------------------------------
def exp(a):
    return Node(np.exp(a.value), "exp", (a,))


def ln(a):
    return Node(np.log(a.value), "ln", (a,))


def sqr(a):
    return Node(a.value * a.value, "sqr", (a,))


def sqrt(a):
    return Node(np.sqrt(a.value), "sqrt", (a,))


def recip(a):
    return Node(1.0 / a.value, "recip", (a,))


def _sig(x):
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def sigmoid(a):
    return Node(_sig(a.value), "sigmoid", (a,))


def silu(a):
    return Node(a.value * _sig(a.value), "silu", (a,))


# ---- reductions ------------------------------------------------------------
def _axes(a, axes):
    if isinstance(axes, int):
        axes = (axes,)
    return tuple(sorted(ax % a.value.ndim for ax in axes))


def sum_(a, axes):
    ax = _axes(a, axes)
    return Node(np.sum(a.value, axis=ax), "sum", (a,), ax)


def mean(a, axes):
    ax = _axes(a, axes)
    return Node(np.mean(a.value, axis=ax), "mean", (a,), ax)


# ---- shapes ----------------------------------------------------------------
def broadcast_as(a, shape):
    shape = tuple(shape)
    return Node(np.broadcast_to(a.value, shape).copy(), "bcast", (a,), shape)


def reshape(a, shape):
    return Node(a.value.reshape(shape), "reshape", (a,))


def transpose_last(a):
    return Node(np.swapaxes(a.value, -1, -2).copy(), "transpose", (a,))


def narrow(a, dim: int, start: int, length: int):
    dim = dim % a.value.ndim
    sl = [slice(None)] * a.value.ndim
    sl[dim] = slice(start, start + length)
    return Node(a.value[tuple(sl)].copy(), "narrow", (a,), (dim, start, length))


def cat(args, dim: int):
    dim = dim % args[0].value.ndim
    return Node(np.concatenate([x.value for x in args], axis=dim), "cat", tuple(args), dim)


def matmul(a, b):
    return Node(np.matmul(a.value, b.value), "matmul", (a, b))


# ---- reverse pass ----------------------------------------------------------
def sorted_nodes(root: Node):
    """Nodes reachable from ``root`` in reverse topological order (root first)."""
    order, seen = [], set()
    stack = [(root, False)]
    while stack:
        node, expanded = stack.pop()
        if expanded:
            order.append(node)
            continue
        if id(node) in seen:
            continue
        seen.add(id(node))
        stack.append((node, True))
        for arg in node.args:
            if id(arg) not in seen:
                stack.append((arg, False))
    order.reverse()
    return order


def _unbroadcast(grad: np.ndarray, shape) -> np.ndarray:
    """Broadcast rule: sum the gradient over the dims that were broadcast."""
    left = grad.ndim - len(shape)
    g = grad.sum(axis=tuple(range(left))) if left else grad
    keep = tuple(i for i, (gs, s) in enumerate(zip(g.shape, shape)) if s == 1 and gs != 1)
    if keep:
        g = g.sum(axis=keep, keepdims=True)
    return g.reshape(shape)


def backward(root: Node, seed=None) -> dict:
    """Vector-Jacobian product of ``root`` with ``seed`` (ones if None).

    Returns {id(node): gradient} for every node reachable from ``root``.
    """
    grads = {id(root): np.ones_like(root.value) if seed is None
             else np.asarray(seed, dtype=np.float64).reshape(root.shape).copy()}

    def acc(node, g):
        k = id(node)
        if k in grads:
            grads[k] = grads[k] + g
        else:
            grads[k] = np.array(g, dtype=np.float64, copy=True)

    for node in sorted_nodes(root):
        if node.op is None:
            continue
        g = grads.get(id(node))
        if g is None:
            continue
        op, args = node.op, node.args
        if op == "add":
            acc(args[0], g)
            acc(args[1], g)
        elif op == "sub":
            acc(args[0], g)
            acc(args[1], -g)
        elif op == "mul":
            acc(args[0], g * args[1].value)
            acc(args[1], g * args[0].value)
        elif op == "div":
            acc(args[0], g / args[1].value)
            acc(args[1], -g * args[0].value / (args[1].value ** 2))
        elif op == "add_s":
            acc(args[0], g)
        elif op == "mul_s":
            acc(args[0], g * node.meta)
        elif op == "neg":
            acc(args[0], -g)
        elif op == "affine":
            acc(args[0], g * node.meta[0])
        elif op == "exp":
            acc(args[0], g * node.value)
        elif op == "ln":
            acc(args[0], g / args[0].value)
        elif op == "sqr":
            acc(args[0], 2.0 * g * args[0].value)
        elif op == "sqrt":
            acc(args[0], 0.5 * g / node.value)
        elif op == "recip":
            acc(args[0], -g * node.value ** 2)
        elif op == "sigmoid":
            acc(args[0], g * node.value * (1.0 - node.value))
        elif op == "silu":
            s = _sig(args[0].value)
            si = args[0].value * s
            acc(args[0], g * (s * (1.0 - si) + si))
        elif op in ("sum", "mean"):
            keep = list(args[0].shape)
            n = 1
            for ax in node.meta:
                n *= keep[ax]
                keep[ax] = 1
            gg = np.broadcast_to(g.reshape(keep), args[0].shape)
            acc(args[0], gg / n if op == "mean" else gg)
        elif op == "bcast":
            acc(args[0], _unbroadcast(g, args[0].shape))
        elif op == "reshape":
            acc(args[0], g.reshape(args[0].shape))
        elif op == "transpose":
            acc(args[0], np.swapaxes(g, -1, -2))
        elif op == "narrow":
            dim, start, length = node.meta
            full = np.zeros(args[0].shape)
            sl = [slice(None)] * full.ndim
            sl[dim] = slice(start, start + length)
            full[tuple(sl)] = g
            acc(args[0], full)
        elif op == "cat":
            dim = node.meta
            start = 0
            for x in args:
                ln_ = x.shape[dim]
                sl = [slice(None)] * g.ndim
                sl[dim] = slice(start, start + ln_)
                acc(x, g[tuple(sl)])
                start += ln_
        elif op == "matmul":
            a, b = args
            acc(a, _unbroadcast(np.matmul(g, np.swapaxes(b.value, -1, -2)), a.shape))
            acc(b, _unbroadcast(np.matmul(np.swapaxes(a.value, -1, -2), g), b.shape))
        else:  # pragma: no cover
            raise NotImplementedError(op)
    return grads
