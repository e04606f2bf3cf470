"""Pins of the fp64 scan oracle against things other than itself (CPU only).

Each check is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign, an off-by-one step, a transposed operand) fails at least one:
  * a hand-worked example (tests/golden/ssm_scalar_T2.json);
  * central finite differences on every input element of the tiny workload;
  * an independent unrolled-graph reverse-mode tape (oracle.tape);
  * closed forms: d_D = sum dy u; delta = 0; a memoryless state (a = 0); T = 1;
  * the scalar recurrence written as an explicit sum over steps;
  * a dot-product (adjoint) test at a larger shape;
  * invariants: linearity in d_out, batch additivity, causality.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import ssm, tape
from synth import CONFIGS, scan_inputs
from tests._util import SCAN_OUTPUTS, norm_err

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _problem(nb, T, di, N, seed, variant="default", random_A=True):
    p = scan_inputs(nb, T, di, N, "f32", seed=seed, variant=variant)
    p = {k: v.astype(np.float64) for k, v in p.items()}
    if random_A:
        rng = np.random.default_rng(seed + 1000)
        p["A_log"] = p["A_log"] + 0.5 * rng.standard_normal(p["A_log"].shape)
        p["D"] = p["D"] + 0.5 * rng.standard_normal(p["D"].shape)
    return p


def _bwd(p, **kw):
    return ssm.ssm_scan_bwd(p["u"], p["delta"], p["A_log"], p["B"], p["C"], p["D"],
                            p["z"], p["d_out"], **kw)


def _loss(p):
    _, out = ssm.ssm_forward(p["u"], p["delta"], p["A_log"], p["B"], p["C"], p["D"], p["z"])
    return np.sum(out * p["d_out"], axis=(1, 2))


# ---------------------------------------------------------------------------
def test_golden_scalar_worked_example():
    with open(os.path.join(GOLDEN, "ssm_scalar_T2.json")) as f:
        fx = json.load(f)
    env = {"math": math}
    inp = {k: np.array(eval(v, env), dtype=np.float64) for k, v in fx["inputs"].items()}
    exp = {k: np.array(eval(v, env), dtype=np.float64) for k, v in fx["expected"].items()}
    y, _ = ssm.ssm_forward(inp["u"], inp["delta"], inp["A_log"], inp["B"], inp["C"], inp["D"])
    np.testing.assert_allclose(y, exp["y"], rtol=1e-14, atol=1e-14)
    g = _bwd(inp)
    for k in SCAN_OUTPUTS:
        np.testing.assert_allclose(g[k], exp[k], rtol=1e-13, atol=1e-13, err_msg=k)


# ---------------------------------------------------------------------------
def _fd_batched(p, name, eps=1e-6):
    """Central differences for every element of a [B, T, *] input, all at once.

    Each perturbed copy is one extra batch element; the loss is per batch element.
    """
    X = p[name]
    n = X[0].size
    nb = X.shape[0]
    assert nb == 1
    reps = {k: np.repeat(v, 2 * n, axis=0) for k, v in p.items()
            if k in ("u", "delta", "B", "C", "z", "d_out")}
    flat = reps[name].reshape(2 * n, -1)
    idx = np.arange(n)
    flat[idx, idx] += eps
    flat[n + idx, idx] -= eps
    q = dict(p)
    q.update(reps)
    L = _loss(q)
    return ((L[:n] - L[n:]) / (2 * eps)).reshape(X.shape)


def _fd_param(p, name, eps=1e-6):
    X = p[name]
    out = np.zeros_like(X)
    for i in range(X.size):
        q = dict(p)
        xp = X.copy().reshape(-1)
        xm = X.copy().reshape(-1)
        xp[i] += eps
        xm[i] -= eps
        q[name] = xp.reshape(X.shape)
        Lp = _loss(q).sum()
        q[name] = xm.reshape(X.shape)
        Lm = _loss(q).sum()
        out.reshape(-1)[i] = (Lp - Lm) / (2 * eps)
    return out


def test_finite_differences_every_element_tiny_workload():
    c = CONFIGS["tiny"]
    p = {k: v.astype(np.float64) for k, v in
         scan_inputs(c.batch, c.seqlen, c.d_inner, c.d_state, c.dtype, c.seed).items()}
    g = _bwd(p)
    fd = {
        "d_u": _fd_batched(p, "u"), "d_delta": _fd_batched(p, "delta"),
        "d_z": _fd_batched(p, "z"), "d_B": _fd_batched(p, "B"), "d_C": _fd_batched(p, "C"),
        "d_A_log": _fd_param(p, "A_log"), "d_D": _fd_param(p, "D"),
    }
    for k in SCAN_OUTPUTS:
        assert norm_err(g[k], fd[k]) < 1e-6, (k, norm_err(g[k], fd[k]))


def test_finite_differences_random_A_long_memory():
    p = _problem(1, 24, 5, 4, seed=7, variant="long_memory")
    g = _bwd(p)
    fd = {
        "d_u": _fd_batched(p, "u"), "d_delta": _fd_batched(p, "delta"),
        "d_z": _fd_batched(p, "z"), "d_B": _fd_batched(p, "B"), "d_C": _fd_batched(p, "C"),
        "d_A_log": _fd_param(p, "A_log"), "d_D": _fd_param(p, "D"),
    }
    for k in SCAN_OUTPUTS:
        assert norm_err(g[k], fd[k]) < 1e-6, (k, norm_err(g[k], fd[k]))


# ---------------------------------------------------------------------------
def _tape_scan(p):
    """The forward rebuilt from primitive tape ops, unrolled over t."""
    L = {k: tape.leaf(p[k]) for k in ("u", "delta", "A_log", "B", "C", "D", "z")}
    nb, T, di = p["u"].shape
    N = p["B"].shape[2]
    A = tape.neg(tape.exp(L["A_log"]))
    A3 = tape.broadcast_as(A, (nb, di, N))
    h = tape.leaf(np.zeros((nb, di, N)))
    ys = []
    for t in range(T):
        u_t = tape.reshape(tape.narrow(L["u"], 1, t, 1), (nb, di))
        d_t = tape.reshape(tape.narrow(L["delta"], 1, t, 1), (nb, di))
        B_t = tape.broadcast_as(tape.reshape(tape.narrow(L["B"], 1, t, 1), (nb, 1, N)), (nb, di, N))
        C_t = tape.broadcast_as(tape.reshape(tape.narrow(L["C"], 1, t, 1), (nb, 1, N)), (nb, di, N))
        d3 = tape.broadcast_as(tape.reshape(d_t, (nb, di, 1)), (nb, di, N))
        a = tape.exp(tape.mul(d3, A3))
        du3 = tape.broadcast_as(tape.reshape(tape.mul(d_t, u_t), (nb, di, 1)), (nb, di, N))
        h = tape.add(tape.mul(a, h), tape.mul(du3, B_t))
        y_t = tape.add(tape.sum_(tape.mul(h, C_t), 2),
                       tape.mul(tape.broadcast_as(L["D"], (nb, di)), u_t))
        ys.append(tape.reshape(y_t, (nb, 1, di)))
    y = tape.cat(ys, 1)
    out = tape.mul(y, tape.silu(L["z"]))
    return L, y, out


@pytest.mark.parametrize("variant", ["default", "long_memory"])
def test_tape_autodiff_agrees(variant):
    p = _problem(2, 9, 3, 4, seed=3, variant=variant)
    L, y, out = _tape_scan(p)
    y_or, out_or = ssm.ssm_forward(p["u"], p["delta"], p["A_log"], p["B"], p["C"], p["D"], p["z"])
    np.testing.assert_allclose(y.value, y_or, rtol=1e-13, atol=1e-13)
    grads = tape.backward(out, seed=p["d_out"])
    g = _bwd(p)
    names = {"d_u": "u", "d_delta": "delta", "d_A_log": "A_log", "d_B": "B", "d_C": "C",
             "d_D": "D", "d_z": "z"}
    for k, leaf in names.items():
        assert norm_err(g[k], grads[id(L[leaf])]) < 1e-12, k


# ---------------------------------------------------------------------------
def test_closed_form_dD():
    p = _problem(3, 17, 6, 4, seed=11)
    g = _bwd(p)
    y, _ = ssm.ssm_forward(p["u"], p["delta"], p["A_log"], p["B"], p["C"], p["D"])
    s = 0.5 * (1 + np.tanh(0.5 * p["z"]))
    dy = p["d_out"] * p["z"] * s
    np.testing.assert_allclose(g["d_D"], np.sum(dy * p["u"], axis=(0, 1)), rtol=1e-13)


def _reverse_inclusive_cumsum(x, axis):
    """rlx-cpu 0.2.17 ``cumsum_backward_row`` (inclusive): suffix sums from the end."""
    return np.flip(np.cumsum(np.flip(x, axis=axis), axis=axis), axis=axis)


def test_closed_form_zero_delta():
    """delta = 0: h stays 0, y = D u, and d_delta_t = u_t sum_n B_t[n] G_t[n], G = suffix-sum of dy C."""
    p = _problem(2, 13, 5, 3, seed=5, variant="zero_delta")
    g = _bwd(p)
    s = 0.5 * (1 + np.tanh(0.5 * p["z"]))
    dy = p["d_out"] * p["z"] * s
    y = p["D"] * p["u"]
    assert np.all(g["d_B"] == 0) and np.all(g["d_C"] == 0) and np.all(g["d_A_log"] == 0)
    np.testing.assert_allclose(g["d_u"], p["D"] * dy, rtol=1e-14)
    np.testing.assert_allclose(g["d_z"], p["d_out"] * y * s * (1 + p["z"] * (1 - s)), rtol=1e-13)
    G = _reverse_inclusive_cumsum(dy[..., None] * p["C"][:, :, None, :], axis=1)  # [B,T,Di,N]
    want = p["u"] * np.sum(p["B"][:, :, None, :] * G, axis=-1)
    np.testing.assert_allclose(g["d_delta"], want, rtol=1e-12, atol=1e-12)
    assert np.max(np.abs(g["d_delta"])) > 0.1  # not the zero the loose wording suggests


def test_closed_form_memoryless():
    """A_log = 50: a = exp(delta A) is exactly 0, so each step stands alone."""
    p = _problem(2, 7, 4, 3, seed=9, random_A=False)
    p["A_log"] = np.full_like(p["A_log"], 50.0)
    g = _bwd(p)
    s = 0.5 * (1 + np.tanh(0.5 * p["z"]))
    dy = p["d_out"] * p["z"] * s
    BC = np.sum(p["B"] * p["C"], axis=-1)[..., None]       # [B, T, 1]
    np.testing.assert_allclose(g["d_delta"], p["u"] * dy * BC, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g["d_u"], p["D"] * dy + p["delta"] * dy * BC, rtol=1e-12, atol=1e-14)
    du = p["delta"] * p["u"]
    np.testing.assert_allclose(g["d_B"], np.sum(dy * du, axis=2)[..., None] * p["C"], rtol=1e-12,
                               atol=1e-14)
    np.testing.assert_allclose(g["d_C"], np.sum(dy * du, axis=2)[..., None] * p["B"], rtol=1e-12,
                               atol=1e-14)
    assert np.all(g["d_A_log"] == 0)


def test_closed_form_single_step():
    p = _problem(2, 1, 3, 4, seed=13)
    g = _bwd(p)
    s = 0.5 * (1 + np.tanh(0.5 * p["z"]))
    dy = p["d_out"] * p["z"] * s
    BC = np.sum(p["B"] * p["C"], axis=-1)[..., None]
    np.testing.assert_allclose(g["d_delta"], dy * p["u"] * BC, rtol=1e-13)
    np.testing.assert_allclose(g["d_u"], p["D"] * dy + p["delta"] * dy * BC, rtol=1e-13)
    assert np.all(g["d_A_log"] == 0)


def test_scalar_recurrence_explicit_sum():
    """d_inner = d_state = batch = 1: h_t = sum_s (prod_{r=s+1..t} a_r) delta_s u_s B_s."""
    T = 7
    p = _problem(1, T, 1, 1, seed=21)
    u, dl, B, C = (p[k].reshape(T) for k in ("u", "delta", "B", "C"))
    A = -math.exp(p["A_log"].item())
    Dv = p["D"].item()
    a = np.exp(dl * A)
    prod = lambda s, t: float(np.prod(a[s + 1:t + 1]))  # noqa: E731
    h = np.array([sum(prod(s, t) * dl[s] * u[s] * B[s] for s in range(t + 1)) for t in range(T)])
    y = C * h + Dv * u
    y_or, _ = ssm.ssm_forward(p["u"], p["delta"], p["A_log"], p["B"], p["C"], p["D"])
    np.testing.assert_allclose(y_or.reshape(T), y, rtol=1e-13)
    z = p["z"].reshape(T)
    s_ = 0.5 * (1 + np.tanh(0.5 * z))
    dy = p["d_out"].reshape(T) * z * s_
    # explicit derivatives of L = sum_t dy_t y_t
    du = np.array([Dv * dy[s] + sum(dy[t] * C[t] * prod(s, t) for t in range(s, T)) * dl[s] * B[s]
                   for s in range(T)])
    dB = np.array([sum(dy[t] * C[t] * prod(s, t) for t in range(s, T)) * dl[s] * u[s]
                   for s in range(T)])
    dC = dy * h
    # d/d delta_s: the input term at s, plus every later state through a_s
    hprev = np.concatenate([[0.0], h[:-1]])
    dd = np.array([sum(dy[t] * C[t] * prod(s, t) for t in range(s, T)) * (u[s] * B[s] + A * a[s] * hprev[s])
                   for s in range(T)])
    dAlog = A * sum(sum(dy[t] * C[t] * prod(s, t) for t in range(s, T)) * a[s] * dl[s] * hprev[s]
                    for s in range(T))
    g = _bwd(p)
    np.testing.assert_allclose(g["d_u"].reshape(T), du, rtol=1e-12)
    np.testing.assert_allclose(g["d_B"].reshape(T), dB, rtol=1e-12)
    np.testing.assert_allclose(g["d_C"].reshape(T), dC, rtol=1e-12)
    np.testing.assert_allclose(g["d_delta"].reshape(T), dd, rtol=1e-12)
    np.testing.assert_allclose(g["d_A_log"].item(), dAlog, rtol=1e-12)


# ---------------------------------------------------------------------------
def test_dot_product_adjoint():
    p = _problem(2, 96, 40, 16, seed=17)
    g = _bwd(p, chan_block=16)
    rng = np.random.default_rng(99)
    keys = {"u": "d_u", "delta": "d_delta", "A_log": "d_A_log", "B": "d_B", "C": "d_C",
            "D": "d_D", "z": "d_z"}
    v = {k: rng.standard_normal(p[k].shape) for k in keys}
    ana = sum(float(np.sum(g[gk] * v[k])) for k, gk in keys.items())
    eps = 1e-6
    qp, qm = dict(p), dict(p)
    for k in keys:
        qp[k] = p[k] + eps * v[k]
        qm[k] = p[k] - eps * v[k]
    num = float((_loss(qp).sum() - _loss(qm).sum()) / (2 * eps))
    assert abs(ana - num) / abs(ana) < 1e-7


def test_linear_in_d_out():
    p = _problem(2, 20, 5, 4, seed=23)
    q = dict(p)
    rng = np.random.default_rng(1)
    q["d_out"] = rng.standard_normal(p["d_out"].shape)
    r = dict(p)
    r["d_out"] = 2.0 * p["d_out"] - 3.0 * q["d_out"]
    gp, gq, gr = _bwd(p), _bwd(q), _bwd(r)
    for k in SCAN_OUTPUTS:
        np.testing.assert_allclose(gr[k], 2.0 * gp[k] - 3.0 * gq[k], rtol=1e-11, atol=1e-11)


def test_batch_additivity_and_independence():
    p = _problem(3, 15, 4, 4, seed=29)
    g = _bwd(p)
    acc_A = np.zeros_like(g["d_A_log"])
    acc_D = np.zeros_like(g["d_D"])
    for b in range(3):
        q = {k: (v[b:b + 1] if v.ndim == 3 else v) for k, v in p.items()}
        gb = _bwd(q)
        for k in ("d_u", "d_delta", "d_z", "d_B", "d_C"):
            np.testing.assert_allclose(gb[k][0], g[k][b], rtol=1e-13, atol=1e-14)
        acc_A += gb["d_A_log"]
        acc_D += gb["d_D"]
    np.testing.assert_allclose(acc_A, g["d_A_log"], rtol=1e-12)
    np.testing.assert_allclose(acc_D, g["d_D"], rtol=1e-12)


def test_causality():
    """Steps appended with d_out = 0 change no gradient of the earlier steps."""
    p = _problem(1, 30, 4, 4, seed=31)
    q = {k: (v[:, :20] if v.ndim == 3 else v) for k, v in p.items()}
    p["d_out"][:, 20:] = 0.0
    gp, gq = _bwd(p), _bwd(q)
    for k in ("d_u", "d_delta", "d_z", "d_B", "d_C"):
        np.testing.assert_allclose(gp[k][:, :20], gq[k], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(gp["d_A_log"], gq["d_A_log"], rtol=1e-12)
    for k in ("d_u", "d_delta", "d_z", "d_B", "d_C"):   # no cotangent reaches the later steps
        assert np.all(gp[k][:, 20:] == 0.0), k


def test_channel_blocks_do_not_change_results():
    p = _problem(1, 12, 10, 4, seed=37)
    g1 = _bwd(p, chan_block=3)
    g2 = _bwd(p, chan_block=1024)
    for k in SCAN_OUTPUTS:
        np.testing.assert_allclose(g1[k], g2[k], rtol=1e-13, atol=1e-15)


def test_states_at_matches_outputs():
    p = _problem(2, 11, 3, 4, seed=41)
    steps = [0, 4, 10]
    hs = ssm.ssm_states_at(p["u"], p["delta"], p["A_log"], p["B"], steps)   # [B, S, N, Di]
    y, _ = ssm.ssm_forward(p["u"], p["delta"], p["A_log"], p["B"], p["C"], p["D"])
    for i, t in enumerate(steps):
        yt = np.einsum("bnd,bn->bd", hs[:, i], p["C"][:, t]) + p["D"] * p["u"][:, t]
        np.testing.assert_allclose(yt, y[:, t], rtol=1e-13)
