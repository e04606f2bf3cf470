"""Pins of the fp64 layer oracle (CPU only): finite differences over every input
and parameter element of a tiny layer, the independent tape, and closed forms
for RMSNorm, the conv carry and softplus."""
import numpy as np
import pytest

from oracle import layer, tape
from synth import layer_inputs
from tests._util import norm_err

DIMS = dict(batch=2, seqlen=8, d_model=8, d_inner=16, d_state=4, dt_rank=2, d_conv=4)
EPS = 1e-5


def _params(variant="perturbed", seed=3):
    p = layer_inputs(**DIMS, dtype="f32", seed=seed, variant=variant)
    p = {k: v.astype(np.float64) for k, v in p.items()}
    # larger weights than the workload's 0.02 so that every path carries signal
    for k in ("W_in", "W_x", "W_dt", "W_out", "conv_w"):
        p[k] = p[k] * 20.0
    rng = np.random.default_rng(seed + 7)
    p["A_log"] = p["A_log"] + 0.3 * rng.standard_normal(p["A_log"].shape)
    p["D"] = p["D"] + 0.3 * rng.standard_normal(p["D"].shape)
    return p


def _loss(p, d_out):
    act = layer.layer_forward(p, DIMS["d_state"], DIMS["dt_rank"], EPS)
    return float(np.sum(act["out"] * d_out))


GRAD_OF = {"x": "d_x", "norm_w": "d_norm_w", "W_in": "d_W_in", "conv_w": "d_conv_w",
           "conv_b": "d_conv_b", "W_x": "d_W_x", "W_dt": "d_W_dt", "b_dt": "d_b_dt",
           "A_log": "d_A_log", "D": "d_D", "W_out": "d_W_out"}


def test_layer_finite_differences_every_element():
    p = _params()
    d_out = p.pop("d_out")
    g = layer.layer_bwd(p, d_out, DIMS["d_state"], DIMS["dt_rank"], EPS)
    h = 1e-6
    for name, gk in GRAD_OF.items():
        X = p[name]
        fd = np.zeros_like(X)
        for i in range(X.size):
            q = dict(p)
            xp, xm = X.copy().reshape(-1), X.copy().reshape(-1)
            xp[i] += h
            xm[i] -= h
            q[name] = xp.reshape(X.shape)
            lp = _loss(q, d_out)
            q[name] = xm.reshape(X.shape)
            lm = _loss(q, d_out)
            fd.reshape(-1)[i] = (lp - lm) / (2 * h)
        assert norm_err(g[gk], fd) < 1e-6, (name, norm_err(g[gk], fd))


def _tape_layer(p):
    ds, r, K = DIMS["d_state"], DIMS["dt_rank"], DIMS["d_conv"]
    L = {k: tape.leaf(v) for k, v in p.items() if k != "d_out"}
    x = L["x"]
    nb, T, dm = p["x"].shape
    di = p["D"].shape[0]
    # RMSNorm from Sqr, Mean, scalar add, Sqrt, Recip, Mul (the page leaves RmsNorm unsupported)
    ms = tape.mean(tape.sqr(x), 2)
    inv_r = tape.recip(tape.sqrt(tape.add_scalar(ms, EPS)))
    inv_b = tape.broadcast_as(tape.reshape(inv_r, (nb, T, 1)), (nb, T, dm))
    xn = tape.mul(tape.mul(x, inv_b), tape.broadcast_as(L["norm_w"], (nb, T, dm)))
    xz = tape.matmul(xn, tape.transpose_last(L["W_in"]))
    x_b = tape.narrow(xz, 2, 0, di)
    z = tape.narrow(xz, 2, di, di)
    # causal depthwise conv via zero padding and shifted narrows
    pad = tape.cat([tape.leaf(np.zeros((nb, K - 1, di))), x_b], 1)
    c = tape.broadcast_as(L["conv_b"], (nb, T, di))
    for k in range(K):
        wk = tape.reshape(tape.narrow(L["conv_w"], 1, k, 1), (di,))
        c = tape.add(c, tape.mul(tape.narrow(pad, 1, k, T), tape.broadcast_as(wk, (nb, T, di))))
    u = tape.silu(c)
    xdbl = tape.matmul(u, tape.transpose_last(L["W_x"]))
    dt_in = tape.narrow(xdbl, 2, 0, r)
    Bm = tape.narrow(xdbl, 2, r, ds)
    Cm = tape.narrow(xdbl, 2, r + ds, ds)
    raw = tape.add(tape.matmul(dt_in, tape.transpose_last(L["W_dt"])),
                   tape.broadcast_as(L["b_dt"], (nb, T, di)))
    assert np.all(raw.value < 20.0)
    delta = tape.ln(tape.add_scalar(tape.exp(raw), 1.0))        # softplus below the threshold
    A3 = tape.broadcast_as(tape.neg(tape.exp(L["A_log"])), (nb, di, ds))
    h = tape.leaf(np.zeros((nb, di, ds)))
    ys = []
    for t in range(T):
        u_t = tape.reshape(tape.narrow(u, 1, t, 1), (nb, di))
        d_t = tape.reshape(tape.narrow(delta, 1, t, 1), (nb, di))
        B_t = tape.broadcast_as(tape.reshape(tape.narrow(Bm, 1, t, 1), (nb, 1, ds)), (nb, di, ds))
        C_t = tape.broadcast_as(tape.reshape(tape.narrow(Cm, 1, t, 1), (nb, 1, ds)), (nb, di, ds))
        a = tape.exp(tape.mul(tape.broadcast_as(tape.reshape(d_t, (nb, di, 1)), (nb, di, ds)), A3))
        du3 = tape.broadcast_as(tape.reshape(tape.mul(d_t, u_t), (nb, di, 1)), (nb, di, ds))
        h = tape.add(tape.mul(a, h), tape.mul(du3, B_t))
        y_t = tape.add(tape.sum_(tape.mul(h, C_t), 2), tape.mul(tape.broadcast_as(L["D"], (nb, di)), u_t))
        ys.append(tape.reshape(y_t, (nb, 1, di)))
    y = tape.cat(ys, 1)
    gated = tape.mul(y, tape.silu(z))
    out = tape.add(tape.matmul(gated, tape.transpose_last(L["W_out"])), x)
    return L, out


def test_layer_tape_agrees():
    p = _params()
    d_out = p["d_out"]
    L, out = _tape_layer(p)
    act = layer.layer_forward(p, DIMS["d_state"], DIMS["dt_rank"], EPS)
    np.testing.assert_allclose(out.value, act["out"], rtol=1e-12, atol=1e-12)
    grads = tape.backward(out, seed=d_out)
    q = {k: v for k, v in p.items() if k != "d_out"}
    g = layer.layer_bwd(q, d_out, DIMS["d_state"], DIMS["dt_rank"], EPS)
    for name, gk in GRAD_OF.items():
        assert norm_err(g[gk], grads[id(L[name])]) < 1e-11, name


# ---------------------------------------------------------------------------
def _rms_fd(x, w, dy, eps, h=1e-6):
    dx = np.zeros_like(x)
    for i in range(x.size):
        xp, xm = x.copy().reshape(-1), x.copy().reshape(-1)
        xp[i] += h
        xm[i] -= h
        dx.reshape(-1)[i] = (np.sum(layer.rmsnorm_fwd(xp.reshape(x.shape), w, eps) * dy)
                             - np.sum(layer.rmsnorm_fwd(xm.reshape(x.shape), w, eps) * dy)) / (2 * h)
    return dx


def test_rmsnorm_bwd_matches_fd_and_rejects_the_extra_factor():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((5, 12)) * 3.0
    w = 1.0 + 0.2 * rng.standard_normal(12)
    dy = rng.standard_normal((5, 12))
    dx, dw = layer.rmsnorm_bwd(x, w, dy, 1e-5)
    assert norm_err(dx, _rms_fd(x, w, dy, 1e-5)) < 1e-8
    inv_r = 1.0 / np.sqrt(np.mean(x * x, -1, keepdims=True) + 1e-5)
    np.testing.assert_allclose(dw, np.sum(dy * x * inv_r, 0), rtol=1e-13)
    # the cross term is inv_r^3; an inv_r^4 version (the slip the rlx-cpu page
    # records) must be told apart by the same finite-difference check
    dot = np.mean(dy * w * x, -1, keepdims=True)
    wrong = inv_r * w * dy - inv_r ** 4 * x * dot
    assert norm_err(wrong, _rms_fd(x, w, dy, 1e-5)) > 1e-3


def test_conv1d_bwd_equals_page_shift_register_loop():
    """Phase B6 walks t backwards with a (d_conv-1)-long carry per channel; the
    stencil in ``conv1d_bwd`` must give the same d_x exactly."""
    rng = np.random.default_rng(8)
    T, di, K = 11, 3, 4
    w = rng.standard_normal((di, K))
    g = rng.standard_normal((T, di))
    x = rng.standard_normal((T, di))
    dx_stencil, dw, db = layer.conv1d_bwd(x, w, g)
    # reverse loop with the carry: the current tap contributes g[t] * w[:, K-1];
    # position k of the carry holds what older inputs still owe
    dx = np.zeros((T, di))
    carry = np.zeros((di, K - 1))
    for t in range(T - 1, -1, -1):
        dx[t] = g[t] * w[:, K - 1] + carry[:, 0]
        for k in range(K - 2):
            carry[:, k] = carry[:, k + 1] + g[t] * w[:, K - 2 - k]
        carry[:, K - 2] = g[t] * w[:, 0]
    np.testing.assert_allclose(dx_stencil, dx, rtol=1e-14, atol=1e-14)
    # weight and bias gradients against the forward by finite differences
    h = 1e-6
    for k in range(K):
        for d in range(di):
            wp, wm = w.copy(), w.copy()
            wp[d, k] += h
            wm[d, k] -= h
            fd = (np.sum(layer.conv1d_fwd(x, wp, np.zeros(di)) * g)
                  - np.sum(layer.conv1d_fwd(x, wm, np.zeros(di)) * g)) / (2 * h)
            assert abs(fd - dw[d, k]) < 1e-7 * max(1.0, abs(fd))
    np.testing.assert_allclose(db, g.sum(0), rtol=1e-14)


def test_softplus_bwd_identities():
    raw = np.array([-30.0, -3.0, -0.5, 0.0, 0.7, 5.0, 19.9, 20.0, 20.1, 45.0])
    d = np.linspace(-1.0, 2.0, raw.size)
    got = layer.softplus_bwd(raw, d)
    delta = layer.softplus_fwd(raw)
    # below the threshold sigmoid(raw) = 1 - exp(-softplus(raw)); above it the gradient passes through
    below = raw <= 20.0
    np.testing.assert_allclose(got[below], d[below] * (1.0 - np.exp(-delta[below])), rtol=1e-12)
    np.testing.assert_array_equal(got[~below], d[~below])
    np.testing.assert_array_equal(delta[~below], raw[~below])
    # the backward from saved activations gets raw back from delta: an exact inverse, except
    # on (20, softplus(20)] = (20, 20 + 2.1e-9] where delta > 20 is read as a pass-through
    np.testing.assert_allclose(layer.softplus_inv(delta), raw, rtol=1e-12, atol=2.1e-9)
    np.testing.assert_allclose(layer.softplus_bwd(layer.softplus_inv(delta), d), got, rtol=2.1e-9)


def test_layer_bwd_saved_needs_only_the_saved_activations():
    """The backward from saved activations reads x, xz, xdbl, delta and y and nothing
    else the forward made: poisoning every other activation changes nothing."""
    p = layer_inputs(1, 12, 8, 16, 4, 2, 4, "f32", seed=3, variant="perturbed")
    act = layer.layer_forward(p, 4, 2)
    ref = layer.layer_bwd_saved(p, act, p["d_out"], 4, 2)
    poisoned = {k: (v if k in ("x", "xz", "xdbl", "delta", "y") else np.full_like(v, np.nan)) for k, v in act.items()}
    got = layer.layer_bwd_saved(p, poisoned, p["d_out"], 4, 2)
    for k in ref:
        np.testing.assert_array_equal(got[k], ref[k])


@pytest.mark.parametrize("T", [1, 2, 3])
def test_conv1d_short_sequences(T):
    rng = np.random.default_rng(T)
    x = rng.standard_normal((2, T, 3))
    w = rng.standard_normal((3, 4))
    g = rng.standard_normal((2, T, 3))
    dx, dw, db = layer.conv1d_bwd(x, w, g)
    h = 1e-6
    fd = np.zeros_like(x)
    for i in range(x.size):
        xp, xm = x.copy().reshape(-1), x.copy().reshape(-1)
        xp[i] += h
        xm[i] -= h
        fd.reshape(-1)[i] = (np.sum(layer.conv1d_fwd(xp.reshape(x.shape), w, np.zeros(3)) * g)
                             - np.sum(layer.conv1d_fwd(xm.reshape(x.shape), w, np.zeros(3)) * g)) / (2 * h)
    assert norm_err(dx, fd) < 1e-8
