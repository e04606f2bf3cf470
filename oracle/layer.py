"""Full Mamba-layer forward and backward around the scan, plain fp64 NumPy.

TEST INFRASTRUCTURE (see the package header).

The layer is the one whose backward mamba-rs 0.5.1 ``cpu/backward.rs`` walks in
``backward_mamba_layer_batched``; the forward is not on the pages and is read
back from the backward's phases (the plainest reading the phases support):

    xn    = RMSNorm(x; norm_w, eps)                  (Phase B8)
    xz    = xn @ W_in^T,  [x_b | z] = split(xz)      (Phase B7: concat [d_x_branch | d_gate])
    c     = causal depthwise conv(x_b; conv_w, conv_b), left zero padding
    u     = SiLU(c)                                   (Phase B6 / note O4)
    xdbl  = u @ W_x^T,  [dt_in | B | C] = split(xdbl) (Phase B5; B, C offsets in Phase B3)
    raw   = dt_in @ W_dt^T + b_dt                     (Phase B4, with bias)
    delta = softplus(raw), raw > 20 passes through    ("Softplus backward" in Phase B3)
    y     = scan(u, delta, A_log, B, C, D)            (Phase B3)
    gated = y * SiLU(z)                               (Phase B2)
    out   = gated @ W_out^T + x                       (Phase B1, residual in Phase B8)

Matrices are [out_features, in_features]; the conv weight is [d_inner, d_conv]
with tap d_conv-1 on the current step (Phase B6's carry multiplies the current
gradient by w[d_conv-2-k] for the k-th older position and by w[0] for the
oldest).  RMSNorm has a weight and no shift, as Phase B8 passes only the norm
weight and the saved rms.
"""
from __future__ import annotations

import numpy as np

from .ssm import _sigmoid, ssm_forward, ssm_scan_bwd


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# ---- RMSNorm ---------------------------------------------------------------
def rmsnorm_fwd(x, w, eps):
    x, w = _f64(x), _f64(w)
    inv_r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * inv_r * w


def rmsnorm_bwd(x, w, dy, eps):
    """rlx-cpu 0.2.17 ``rms_norm_backward_row``, over every row.

    inv_r = 1/sqrt(mean(x^2) + eps);  dx = inv_r * w * dy - inv_r^3 * x * mean(dy * w * x);
    dw = sum over rows of dy * x * inv_r.  (The page's shift term beta is absent here.)
    """
    x, w, dy = _f64(x), _f64(w), _f64(dy)
    inv_r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    dot = np.mean(dy * w * x, axis=-1, keepdims=True)
    dx = inv_r * w * dy - inv_r ** 3 * x * dot
    dw = np.sum((dy * x * inv_r).reshape(-1, x.shape[-1]), axis=0)
    return dx, dw


# ---- linear ----------------------------------------------------------------
def linear_fwd(x, W, b=None):
    y = _f64(x) @ _f64(W).T
    return y if b is None else y + _f64(b)


def linear_bwd(x, W, dy):
    """``sgemm_backward`` as used in Phases B1, B4, B5, B7: y = x W^T (+ b).

    dx = dy W;  dW = sum over rows of dy^T x;  db = sum over rows of dy.
    """
    x, W, dy = _f64(x), _f64(W), _f64(dy)
    x2 = x.reshape(-1, x.shape[-1])
    dy2 = dy.reshape(-1, dy.shape[-1])
    return dy @ W, dy2.T @ x2, dy2.sum(axis=0)


# ---- causal depthwise conv -------------------------------------------------
def conv1d_fwd(x, w, bias):
    """c[t, d] = bias[d] + sum_k w[d, k] * x[t - (K - 1) + k, d], zero before t = 0."""
    x, w, bias = _f64(x), _f64(w), _f64(bias)
    K = w.shape[1]
    T = x.shape[-2]
    c = np.broadcast_to(bias, x.shape).copy()
    for k in range(K):
        s = K - 1 - k          # how far back tap k looks
        if s >= T:
            continue
        c[..., s:, :] += w[:, k] * x[..., : T - s, :]
    return c


def conv1d_bwd(x, w, dc):
    """Adjoint of ``conv1d_fwd`` (Phase B6's reverse loop with its carry, as a stencil).

    dx[t, d] = sum_k dc[t + (K - 1) - k, d] * w[d, k];  dw[d, k] = sum dc[t] x[t - (K-1) + k];
    dbias[d] = sum dc.
    """
    x, w, dc = _f64(x), _f64(w), _f64(dc)
    K = w.shape[1]
    T = x.shape[-2]
    dx = np.zeros_like(x)
    dw = np.zeros_like(w)
    for k in range(K):
        s = K - 1 - k
        if s >= T:
            continue
        dx[..., : T - s, :] += dc[..., s:, :] * w[:, k]
        dw[:, k] = np.sum((dc[..., s:, :] * x[..., : T - s, :]).reshape(-1, x.shape[-1]), axis=0)
    db = np.sum(dc.reshape(-1, dc.shape[-1]), axis=0)
    return dx, dw, db


# ---- pointwise ---------------------------------------------------------------
def silu(x):
    x = _f64(x)
    return x * _sigmoid(x)


def silu_grad(x):
    """d SiLU / dx = s * (1 + x * (1 - s)), as in Phases B2 and B6."""
    x = _f64(x)
    s = _sigmoid(x)
    return s * (1.0 + x * (1.0 - s))


def softplus_fwd(raw, threshold: float = 20.0):
    raw = _f64(raw)
    return np.where(raw > threshold, raw, np.logaddexp(0.0, np.minimum(raw, threshold)))


def softplus_bwd(raw, d_delta, threshold: float = 20.0):
    """"Softplus backward" step of Phase B3: d_raw = d_delta * sigmoid(raw), or d_delta above 20."""
    raw, d_delta = _f64(raw), _f64(d_delta)
    return np.where(raw > threshold, d_delta, d_delta * _sigmoid(raw))


# ---- the layer -------------------------------------------------------------
def layer_forward(p: dict, d_state: int, dt_rank: int, eps: float = 1e-5) -> dict:
    """All activations of the layer forward (see the module docstring)."""
    x = _f64(p["x"])
    di = p["D"].shape[0]
    xn = rmsnorm_fwd(x, p["norm_w"], eps)
    xz = linear_fwd(xn, p["W_in"])
    x_b, z = xz[..., :di], xz[..., di:]
    c = conv1d_fwd(x_b, p["conv_w"], p["conv_b"])
    u = silu(c)
    xdbl = linear_fwd(u, p["W_x"])
    dt_in = xdbl[..., :dt_rank]
    Bm = xdbl[..., dt_rank:dt_rank + d_state]
    Cm = xdbl[..., dt_rank + d_state:dt_rank + 2 * d_state]
    raw = linear_fwd(dt_in, p["W_dt"], p["b_dt"])
    delta = softplus_fwd(raw)
    y, gated = ssm_forward(u, delta, p["A_log"], Bm, Cm, p["D"], z)
    out = linear_fwd(gated, p["W_out"]) + x
    return dict(x=x, xn=xn, xz=xz, x_b=x_b, z=z, c=c, u=u, xdbl=xdbl, dt_in=dt_in,
                B=Bm, C=Cm, raw=raw, delta=delta, y=y, gated=gated, out=out)


def softplus_inv(delta, threshold: float = 20.0):
    """The raw dt_proj output that ``softplus_fwd`` maps to ``delta``: log(e^delta - 1),
    and delta itself above the threshold (where the forward passed raw through)."""
    delta = _f64(delta)
    with np.errstate(divide="ignore"):
        return np.where(delta > threshold, delta, np.log(np.expm1(np.minimum(delta, threshold))))


def layer_bwd_saved(p: dict, saved: dict, d_out, d_state: int, dt_rank: int, eps: float = 1e-5) -> dict:
    """Phases B1-B8 in order, all in fp64, from the activations a forward keeps:
    x (in ``p``), xz, xdbl, delta and y (in ``saved``).  Everything else the
    phases read (xn, x_b, z, the conv output c, u, dt_in, B, C, raw, gated) is
    rebuilt from those, as the layer's forward defines it; raw comes back from
    delta through the softplus inverse.  Returns d_x and every parameter gradient."""
    x = _f64(p["x"])
    di = p["D"].shape[0]
    xz, xdbl, delta, y = (_f64(saved[k]) for k in ("xz", "xdbl", "delta", "y"))
    xn = rmsnorm_fwd(x, p["norm_w"], eps)
    x_b, z = xz[..., :di], xz[..., di:]
    c = conv1d_fwd(x_b, p["conv_w"], p["conv_b"])
    u = silu(c)
    dt_in = xdbl[..., :dt_rank]
    Bm = xdbl[..., dt_rank:dt_rank + d_state]
    Cm = xdbl[..., dt_rank + d_state:dt_rank + 2 * d_state]
    raw = softplus_inv(delta)
    gated = y * silu(z)
    d_out = _f64(d_out)
    # B1 out_proj
    d_gated, dW_out, _ = linear_bwd(gated, p["W_out"], d_out)
    # B2 + B3 gating and scan (the scan oracle does the gating backward itself)
    s = ssm_scan_bwd(u, delta, p["A_log"], Bm, Cm, p["D"], z, d_gated)
    # softplus backward
    d_raw = softplus_bwd(raw, s["d_delta"])
    # B4 dt_proj (with bias)
    d_dt_in, dW_dt, db_dt = linear_bwd(dt_in, p["W_dt"], d_raw)
    d_xdbl = np.concatenate([d_dt_in, s["d_B"], s["d_C"]], axis=-1)
    # B5 x_proj; d_u collects the scan's and x_proj's contributions
    d_u_x, dW_x, _ = linear_bwd(u, p["W_x"], d_xdbl)
    d_u = s["d_u"] + d_u_x
    # B6 SiLU then conv
    d_c = d_u * silu_grad(c)
    d_x_b, d_conv_w, d_conv_b = conv1d_bwd(x_b, p["conv_w"], d_c)
    # B7 in_proj on the concat [d_x_b | d_z]
    d_xz = np.concatenate([d_x_b, s["d_z"]], axis=-1)
    d_xn, dW_in, _ = linear_bwd(xn, p["W_in"], d_xz)
    # B8 RMSNorm + residual
    d_x_norm, d_norm_w = rmsnorm_bwd(x, p["norm_w"], d_xn, eps)
    return {
        "d_x": d_out + d_x_norm, "d_norm_w": d_norm_w, "d_W_in": dW_in,
        "d_conv_w": d_conv_w, "d_conv_b": d_conv_b, "d_W_x": dW_x, "d_W_dt": dW_dt,
        "d_b_dt": db_dt, "d_A_log": s["d_A_log"], "d_D": s["d_D"], "d_W_out": dW_out,
    }


def layer_bwd(p: dict, d_out, d_state: int, dt_rank: int, eps: float = 1e-5) -> dict:
    """The layer's gradient at p: the fp64 forward, then Phases B1-B8 from its activations."""
    act = layer_forward(p, d_state, dt_rank, eps)
    return layer_bwd_saved(p, act, d_out, d_state, dt_rank, eps)
