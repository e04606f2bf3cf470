"""Pins of the fp64 backbone oracle (CPU only): finite differences over every
input and parameter element of a tiny two-layer backbone, and the composition
checks that a wrong layer input, a lost residual or a misplaced norm_f would fail."""
import numpy as np

from oracle import backbone, layer
from synth import backbone_inputs
from tests._util import norm_err

DIMS = dict(batch=2, seqlen=6, d_model=8, d_inner=16, d_state=4, dt_rank=2, d_conv=3)
EPS = 1e-5


def _params(seed=11):
    bp, layers = backbone_inputs(n_layers=2, input_dim=5, dtype="f32", seed=seed, **DIMS)
    bp = {k: v.astype(np.float64) for k, v in bp.items()}
    rng = np.random.default_rng(seed)
    out = []
    for p in layers:
        p = {k: v.astype(np.float64) for k, v in p.items()}
        for k in ("W_in", "W_x", "W_dt", "W_out", "conv_w"):   # every path carries signal
            p[k] = p[k] * 20.0
        p["A_log"] = p["A_log"] + 0.3 * rng.standard_normal(p["A_log"].shape)
        out.append(p)
    bp["W_ip"] = bp["W_ip"] * 5.0
    bp["norm_f_w"] = 1.0 + 0.2 * rng.standard_normal(bp["norm_f_w"].shape)
    return bp, out


def _loss(bp, layers, d_out):
    return float(np.sum(backbone.backbone_forward(bp, layers, DIMS["d_state"], DIMS["dt_rank"], EPS)["out"] * d_out))


def _fd(f, X, h=1e-6):
    g = np.zeros_like(X)
    for i in range(X.size):
        xp, xm = X.copy().reshape(-1), X.copy().reshape(-1)
        xp[i] += h
        xm[i] -= h
        g.reshape(-1)[i] = (f(xp.reshape(X.shape)) - f(xm.reshape(X.shape))) / (2 * h)
    return g


def test_backbone_finite_differences_every_element():
    bp, layers = _params()
    d_out = bp.pop("d_out")
    g = backbone.backbone_bwd(bp, layers, d_out, DIMS["d_state"], DIMS["dt_rank"], EPS)
    for name, gk in (("inp", "d_inp"), ("W_ip", "d_W_ip"), ("b_ip", "d_b_ip"), ("norm_f_w", "d_norm_f_w")):
        fd = _fd(lambda v: _loss(dict(bp, **{name: v}), layers, d_out), bp[name])
        assert norm_err(g[gk], fd) < 1e-6, (name, norm_err(g[gk], fd))
    for l in range(2):
        for name in ("norm_w", "W_in", "conv_w", "conv_b", "W_x", "W_dt", "b_dt", "A_log", "D", "W_out"):
            def f(v, l=l, name=name):
                ls = [dict(p) for p in layers]
                ls[l][name] = v
                return _loss(bp, ls, d_out)
            fd = _fd(f, layers[l][name])
            assert norm_err(g["layers"][l]["d_" + name], fd) < 1e-6, (l, name)


def test_one_layer_backbone_is_input_proj_layer_norm_f():
    """With one layer the chain is explicit: norm_f backward, the layer oracle, then the input projection."""
    bp, layers = _params(seed=4)
    d_out = bp.pop("d_out")
    layers = layers[:1]
    f = backbone.backbone_forward(bp, layers, DIMS["d_state"], DIMS["dt_rank"], EPS)
    x0 = bp["inp"] @ bp["W_ip"].T + bp["b_ip"]
    assert np.allclose(f["xs"][0], x0, atol=1e-12)
    g = backbone.backbone_bwd(bp, layers, d_out, DIMS["d_state"], DIMS["dt_rank"], EPS)
    d1, dnf = layer.rmsnorm_bwd(f["xs"][1], bp["norm_f_w"], d_out, EPS)
    gl = layer.layer_bwd(dict(layers[0], x=x0), d1, DIMS["d_state"], DIMS["dt_rank"], EPS)
    assert np.allclose(g["d_norm_f_w"], dnf, atol=1e-12)
    assert np.allclose(g["layers"][0]["d_W_in"], gl["d_W_in"], atol=1e-12)
    assert np.allclose(g["d_W_ip"], gl["d_x"].reshape(-1, 8).T @ bp["inp"].reshape(-1, 5), atol=1e-10)
    assert np.allclose(g["d_b_ip"], gl["d_x"].reshape(-1, 8).sum(0), atol=1e-10)
