"""Selective-scan forward and its exact adjoint, plain fp64 NumPy.

TEST INFRASTRUCTURE (see the package header): nothing outside the tests, the
smoke check and the bench's CPU-baseline leg may use this module.

Notation (mamba-rs 0.5.1 ``cpu/backward.rs``, Phase B2 "gating backward" and
Phase B3 "sequential SSM BPTT"), per batch b, step t, channel d and state n:

    A        = -exp(A_log)                       (module note O3)
    a_t      = exp(delta_t * A)                  (the saved ``da_exp``)
    h_t      = a_t * h_{t-1} + delta_t u_t B_t    h_{-1} = 0
    y_t      = sum_n C_t[n] h_t[n] + D u_t
    out_t    = y_t * SiLU(z_t)                   (Phase B2)

Shapes: u, delta, z, d_out [Bt, T, Di]; B, C [Bt, T, N] shared by all channels;
A_log [Di, N] (index d * N + n); D [Di].  Readings of the pages where they are
silent: zero initial state and no final-state gradient (Phase B3 starts from a
zeroed d_h), Euler input term delta*B (Phase B3's d_B and d_u terms), one B and
one C vector per step shared by every channel (Phase B3 reads them from the
x_proj output row), gradients are written, not accumulated.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def ssm_forward(u, delta, A_log, B, C, D, z=None):
    """Forward recurrence; returns (y, out) with out = y * SiLU(z) (None if z is None).

    Vectorised over (batch, channel, state), sequential over t.
    """
    u, delta, B, C = _f64(u), _f64(delta), _f64(B), _f64(C)
    A = -np.exp(_f64(A_log))                      # [Di, N]
    Dv = _f64(D)
    nb, T, di = u.shape
    h = np.zeros((nb, di, A.shape[1]))
    y = np.empty((nb, T, di))
    for t in range(T):
        a = np.exp(delta[:, t, :, None] * A[None])               # [Bt, Di, N]
        h = a * h + (delta[:, t] * u[:, t])[:, :, None] * B[:, t, None, :]
        y[:, t] = np.einsum("bdn,bn->bd", h, C[:, t]) + Dv[None] * u[:, t]
    out = None
    if z is not None:
        z = _f64(z)
        out = y * z * _sigmoid(z)
    return y, out


def gating_bwd(d_out, y, z):
    """Phase B2: gated = y * SiLU(z).

    d_y = d_out * SiLU(z) and d_z = d_out * y * s * (1 + z * (1 - s)), s = sigmoid(z).
    """
    d_out, y, z = _f64(d_out), _f64(y), _f64(z)
    s = _sigmoid(z)
    d_y = d_out * z * s
    d_z = d_out * y * s * (1.0 + z * (1.0 - s))
    return d_y, d_z


def ssm_scan_bwd(u, delta, A_log, B, C, D, z, d_out, chan_block: int = 1024):
    """Exact vector-Jacobian product of out = F(u, delta, A_log, B, C, D, z) with d_out.

    Returns a dict with d_u, d_delta, d_z [Bt, T, Di]; d_B, d_C [Bt, T, N];
    d_A_log [Di, N]; d_D [Di], all float64.

    Follows Phase B2 then Phase B3: the forward states of one batch element and
    one block of channels are kept (as the page keeps h_prev / h_curr per
    step), then one reverse sweep over t with the adjoint g = d_h, started at
    zero, does per step:
        g       += dy_t C_t
        d_delta  = sum_n g * (A a_t h_{t-1} + u_t B_t)
        d_u      = D dy_t + delta_t sum_n g B_t
        d_B[n]  += sum_d g delta_t u_t          (sum over channels)
        d_C[n]  += sum_d dy_t h_t
        d_A_log += A g a_t delta_t h_{t-1}
        d_D     += dy_t u_t
        g        = a_t g
    Channel blocks only bound the memory that the kept states take; channels
    are independent except through the two sums over d, which add the blocks'
    partial sums in block order.
    """
    u, delta, B, C = _f64(u), _f64(delta), _f64(B), _f64(C)
    z, d_out = _f64(z), _f64(d_out)
    A = -np.exp(_f64(A_log))
    Dv = _f64(D)
    nb, T, di = u.shape
    N = A.shape[1]
    res = {
        "d_u": np.empty((nb, T, di)), "d_delta": np.empty((nb, T, di)),
        "d_z": np.empty((nb, T, di)), "d_B": np.zeros((nb, T, N)),
        "d_C": np.zeros((nb, T, N)), "d_A_log": np.zeros((di, N)),
        "d_D": np.zeros(di),
    }
    for b in range(nb):
        for d0 in range(0, di, chan_block):
            d1 = min(di, d0 + chan_block)
            Ab, Db = A[d0:d1], Dv[d0:d1]
            ub, db = u[b, :, d0:d1], delta[b, :, d0:d1]
            Bb, Cb = B[b], C[b]
            # forward: keep every h_t of this block
            hs = np.empty((T, d1 - d0, N))
            h = np.zeros((d1 - d0, N))
            y = np.empty((T, d1 - d0))
            for t in range(T):
                a = np.exp(db[t][:, None] * Ab)
                h = a * h + (db[t] * ub[t])[:, None] * Bb[t][None, :]
                hs[t] = h
                y[t] = h @ Cb[t] + Db * ub[t]
            dy, dz = gating_bwd(d_out[b, :, d0:d1], y, z[b, :, d0:d1])
            res["d_z"][b, :, d0:d1] = dz
            # reverse sweep (BPTT)
            g = np.zeros((d1 - d0, N))
            dA = np.zeros((d1 - d0, N))
            for t in range(T - 1, -1, -1):
                a = np.exp(db[t][:, None] * Ab)
                hp = hs[t - 1] if t > 0 else np.zeros_like(g)
                g = g + dy[t][:, None] * Cb[t][None, :]
                res["d_delta"][b, t, d0:d1] = np.sum(
                    g * (Ab * a * hp + ub[t][:, None] * Bb[t][None, :]), axis=1)
                res["d_u"][b, t, d0:d1] = Db * dy[t] + db[t] * np.sum(g * Bb[t][None, :], axis=1)
                res["d_B"][b, t] += np.sum(g * (db[t] * ub[t])[:, None], axis=0)
                res["d_C"][b, t] += np.sum(dy[t][:, None] * hs[t], axis=0)
                dA += Ab * g * a * db[t][:, None] * hp
                g = a * g
            res["d_A_log"][d0:d1] += dA
            res["d_D"][d0:d1] += np.sum(dy * ub, axis=0)
    return res


def ssm_scan_fwd_outputs(u, delta, A_log, B, C, D, z=None):
    """Forward outputs in the library's terms: y and (if z is given) out = y * SiLU(z)."""
    y, out = ssm_forward(u, delta, A_log, B, C, D, z)
    return {"y": y, "out": out}


def ssm_states_at(u, delta, A_log, B, steps):
    """States h_{t} for the listed steps t (the state after step t), [Bt, len(steps), N, Di].

    Used to check chunk-boundary checkpoints; plain forward recurrence.
    """
    u, delta, B = _f64(u), _f64(delta), _f64(B)
    A = -np.exp(_f64(A_log))
    nb, T, di = u.shape
    want = {int(s): i for i, s in enumerate(steps)}
    out = np.zeros((nb, len(want), A.shape[1], di))
    h = np.zeros((nb, di, A.shape[1]))
    for t in range(T):
        a = np.exp(delta[:, t, :, None] * A[None])
        h = a * h + (delta[:, t] * u[:, t])[:, :, None] * B[:, t, None, :]
        if t in want:
            out[:, want[t]] = np.transpose(h, (0, 2, 1))
    return out
