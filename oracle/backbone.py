"""The Mamba backbone around the layer, plain fp64 NumPy.

TEST INFRASTRUCTURE (see the package header): nothing outside the tests, the
smoke check and the bench's CPU-baseline leg may use this module.

mamba-rs 0.5.1 ``cpu/backward.rs``, ``backward_mamba_backbone_batched``: the
backward takes the final RMSNorm (norm_f) backward on the incoming gradient
first, then every layer's backward in reverse order, each handing its input
gradient to the layer before it, and ends with one backward of the input
projection (weight and bias; its input gradient is discarded there because the
embedding is detached).  The forward it implies:

    x_0 = inp W_ip^T + b_ip,   x_{l+1} = layer_l(x_l)  (each layer adds its input),
    out = RMSNorm(x_L; norm_f_w)

with the layer of ``oracle.layer`` (Phases B1-B8 and the forward read back from
them).  Here the input gradient d_inp is returned as well (the caller may drop it).
"""
from __future__ import annotations

import numpy as np

from oracle.layer import layer_bwd_saved, layer_forward, linear_bwd, linear_fwd, rmsnorm_bwd, rmsnorm_fwd


def backbone_forward(bp: dict, layers: list, d_state: int, dt_rank: int, eps: float = 1e-5) -> dict:
    """bp: inp [B, T, mid], W_ip [d_model, mid], b_ip [d_model], norm_f_w [d_model];
    layers: one parameter dict per layer (oracle.layer names, no "x").
    Returns xs (the n_layers + 1 inputs of the layers and of norm_f), each layer's
    activations and out."""
    xs = [linear_fwd(bp["inp"], bp["W_ip"], bp["b_ip"])]
    acts = []
    for p in layers:
        act = layer_forward(dict(p, x=xs[-1]), d_state, dt_rank, eps)
        acts.append(act)
        xs.append(act["out"])
    return {"xs": xs, "acts": acts, "out": rmsnorm_fwd(xs[-1], bp["norm_f_w"], eps)}


def backbone_bwd_saved(bp: dict, layers: list, xs: list, saved: list, d_out, d_state: int, dt_rank: int,
                       eps: float = 1e-5) -> dict:
    """The backward from the kept activations: xs (layer inputs and the norm_f input)
    and each layer's saved xz, xdbl, delta, y."""
    d, d_norm_f_w = rmsnorm_bwd(xs[-1], bp["norm_f_w"], np.asarray(d_out, dtype=np.float64), eps)
    grads = [None] * len(layers)
    for l in range(len(layers) - 1, -1, -1):
        g = layer_bwd_saved(dict(layers[l], x=xs[l]), saved[l], d, d_state, dt_rank, eps)
        grads[l] = g
        d = g["d_x"]
    d_inp, d_W_ip, d_b_ip = linear_bwd(bp["inp"], bp["W_ip"], d)
    return {"d_inp": d_inp, "d_W_ip": d_W_ip, "d_b_ip": d_b_ip, "d_norm_f_w": d_norm_f_w, "layers": grads}


def backbone_bwd(bp: dict, layers: list, d_out, d_state: int, dt_rank: int, eps: float = 1e-5) -> dict:
    """The backbone's gradient at (bp, layers): the fp64 forward, then the backward from its activations."""
    f = backbone_forward(bp, layers, d_state, dt_rank, eps)
    return backbone_bwd_saved(bp, layers, f["xs"], f["acts"], d_out, d_state, dt_rank, eps)
