"""Reverse linear recurrence and the cumsum backward it generalises, plain fp64 NumPy.

TEST INFRASTRUCTURE (see the package header): nothing outside the tests, the
smoke check and the bench's CPU-baseline leg may use this module.

rlx-cpu 0.2.17 ``training_bwd.rs``, ``cumsum_backward_row``: the gradient of a
cumulative sum along a row is the suffix sum of the incoming gradient, taken
from the end of the row backwards; the inclusive form includes the element
itself, the exclusive form only the later ones.

The same sweep with a decay per step is the adjoint recurrence of mamba-rs
0.5.1 ``cpu/backward.rs`` Phase B3 for one state (its d_h propagation,
d_h <- da * d_h after each step): with a_t the decay of the forward step
h_t = a_t h_{t-1} + ..., the adjoint is

    x_t = b_t + a_{t+1} x_{t+1},   x_T = 0            (inclusive)
    e_t = a_{t+1} x_{t+1}  ( = x_t - b_t )            (exclusive)

along t for every (batch, channel) of a time-major [B, T, C] tensor; a = None
means a = 1, the cumsum backward.
"""
from __future__ import annotations

import numpy as np


def cumsum_backward_row(dy, exclusive: bool):
    """One row, walked from its end as the page walks it: a running suffix sum."""
    dy = np.asarray(dy, dtype=np.float64)
    dx = np.zeros_like(dy)
    suffix = 0.0
    for i in range(dy.shape[0] - 1, -1, -1):
        if exclusive:
            dx[i] = suffix
            suffix += dy[i]
        else:
            suffix += dy[i]
            dx[i] = suffix
    return dx


def reverse_linear_scan(a, b, exclusive: bool = False):
    """x for a [B, T, C] time-major b (and a, or None for a = 1), sequential over t."""
    b = np.asarray(b, dtype=np.float64)
    a = None if a is None else np.asarray(a, dtype=np.float64)
    nb, T, C = b.shape
    x = np.zeros_like(b)
    carry = np.zeros((nb, C))          # a_{t+1} x_{t+1}, the part coming from later steps
    for t in range(T - 1, -1, -1):
        full = b[:, t] + carry         # inclusive x_t
        x[:, t] = carry if exclusive else full
        carry = full if a is None else a[:, t] * full
    return x
