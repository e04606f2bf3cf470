"""GPU parity of mamba_backbone_fwd / mamba_backbone_bwd (input projection, layers,
norm_f; mamba-rs backward_mamba_backbone_batched) against the fp64 oracle.

Routes as for the layer: backward only (the oracle's activations, rounded to
bf16, go to both sides; bar 2e-2) and end to end (the GPU forward feeds the GPU
backward; the oracle differentiates at the exact activations; bar 2e-2 on the
forward outputs, 3e-2 on the gradients, the reduced-size end-to-end bar the
layer tests derive).  Weights are drawn with std 0.02 sqrt(1536 / d_model), as
in the layer tests, so that reduced layers have the full layer's activation scale.
"""
import numpy as np
import pytest
import torch

from oracle import backbone as orc
from synth import backbone_inputs, round_bf16
from tests._util import norm_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-2
TOL_END_TO_END = 3e-2
BF16 = ("inp", "W_ip", "d_out", "W_in", "W_x", "W_dt", "W_out")
LAYER_KEYS = ("norm_w", "W_in", "conv_w", "conv_b", "W_x", "W_dt", "b_dt", "A_log", "D", "W_out")


def _ssm():
    import selective_state_space_bwd_amd as ssm
    return ssm


def _t(k, v):
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return (t.to(torch.bfloat16) if k in BF16 else t).to(DEV)


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _inputs(shape, seed):
    L, Bt, T, mid, dm, di, N, R, K = shape
    return backbone_inputs(L, mid, Bt, T, dm, di, N, R, K, "bf16", seed=seed, weight_std=0.02 * np.sqrt(1536.0 / dm))


def _dev(bp, layers):
    return {k: _t(k, v) for k, v in bp.items()}, [{k: _t(k, v) for k, v in p.items()} for p in layers]


def _check(got, ref, label, tol):
    errs = {k: norm_err(got[k], ref[k]) for k in ref}
    print(f"  {label}: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{label}: {bad} exceed {tol}"


def _grads(g):
    out = {k: _np(g[k]) for k in ("d_W_ip", "d_b_ip", "d_norm_f_w") if k in g}
    for l, gl in enumerate(g["layers"]):
        out.update({f"{l}.{k}": _np(v) for k, v in gl.items()})
    return out


def _ref_grads(r):
    out = {k: r[k] for k in ("d_W_ip", "d_b_ip", "d_norm_f_w")}
    for l, gl in enumerate(r["layers"]):
        out.update({f"{l}.d_{k}": gl["d_" + k] for k in LAYER_KEYS})
    return out


# (n_layers, batch, seqlen, input_dim, d_model, d_inner, d_state, dt_rank, d_conv)
SHAPES = [(2, 2, 150, 32, 64, 128, 16, 8, 4), (3, 1, 210, 24, 136, 200, 8, 16, 3)]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"L{s[0]}B{s[1]}T{s[2]}in{s[3]}dm{s[4]}" for s in SHAPES])
def test_backbone_bwd_from_oracle_activations(shape):
    L, Bt, T, mid, dm, di, N, R, K = shape
    bp, layers = _inputs(shape, seed=sum(shape))
    f = orc.backbone_forward(bp, layers, N, R)
    xs = [round_bf16(x) for x in f["xs"]]
    saved = [{k: round_bf16(a[k]) for k in ("xz", "xdbl", "delta", "y")} for a in f["acts"]]
    tb, tl = _dev(bp, layers)
    kept = {"xs": [_t("inp", x) for x in xs], "saved": [{k: _t("inp", v) for k, v in s.items()} for s in saved]}
    print(f"case: backbone bwd from oracle activations {shape}", flush=True)
    g = _ssm().mamba_backbone_bwd(tb["inp"], tb["W_ip"], tb["norm_f_w"], tl, kept, tb["d_out"], need_d_inp=True)
    torch.cuda.synchronize()
    r = orc.backbone_bwd_saved(bp, layers, xs, saved, bp["d_out"], N, R)
    ref = _ref_grads(r)
    ref["d_inp"] = r["d_inp"]
    got = _grads(g)
    got["d_inp"] = _np(g["d_inp"])
    _check(got, ref, "backward", TOL)


@pytest.mark.parametrize("keep", [(False, False), (True, False), (False, True)],
                         ids=["rebuilt-states", "kept-states", "kept-gemm-inputs"])
@pytest.mark.parametrize("shape", SHAPES[:1])
def test_backbone_end_to_end(shape, keep):
    L, Bt, T, mid, dm, di, N, R, K = shape
    bp, layers = _inputs(shape, seed=3 + sum(shape))
    tb, tl = _dev(bp, layers)
    print(f"case: backbone fwd + bwd {shape} keep_scan_states, keep_gemm_inputs {keep}", flush=True)
    out, kept = _ssm().mamba_backbone_fwd(tb["inp"], tb["W_ip"], tb["b_ip"], tb["norm_f_w"], tl,
                                          keep_scan_states=keep[0], keep_gemm_inputs=keep[1])
    g = _ssm().mamba_backbone_bwd(tb["inp"], tb["W_ip"], tb["norm_f_w"], tl, kept, tb["d_out"])
    torch.cuda.synchronize()
    f = orc.backbone_forward(bp, layers, N, R)
    fwd = {"out": _np(out), **{f"xs{l}": _np(x) for l, x in enumerate(kept["xs"])}}
    _check(fwd, {"out": f["out"], **{f"xs{l}": x for l, x in enumerate(f["xs"])}}, "forward", TOL)
    r = orc.backbone_bwd(bp, layers, bp["d_out"], N, R)
    _check(_grads(g), _ref_grads(r), "backward", TOL_END_TO_END)


def test_backbone_bwd_accumulate_two_micro_batches_and_determinism():
    shape = SHAPES[0]
    L, Bt, T, mid, dm, di, N, R, K = shape
    bp, layers = _inputs(shape, seed=77)
    tb, tl = _dev(bp, layers)
    ssm = _ssm()
    print(f"case: backbone bwd accumulate over micro-batches {shape}", flush=True)
    _, kept = ssm.mamba_backbone_fwd(tb["inp"], tb["W_ip"], tb["b_ip"], tb["norm_f_w"], tl)
    full = ssm.mamba_backbone_bwd(tb["inp"], tb["W_ip"], tb["norm_f_w"], tl, kept, tb["d_out"])
    again = ssm.mamba_backbone_bwd(tb["inp"], tb["W_ip"], tb["norm_f_w"], tl, kept, tb["d_out"])
    acc = None
    for b in range(Bt):
        kb = {"xs": [x[b:b + 1].contiguous() for x in kept["xs"]],
              "saved": [{k: v[b:b + 1].contiguous() for k, v in s.items()} for s in kept["saved"]]}
        args = (tb["inp"][b:b + 1].contiguous(), tb["W_ip"], tb["norm_f_w"], tl, kb, tb["d_out"][b:b + 1].contiguous())
        acc = ssm.mamba_backbone_bwd(*args) if acc is None else ssm.mamba_backbone_bwd(*args, out=acc, accumulate=True)
    torch.cuda.synchronize()
    gf, ga, g2 = _grads(full), _grads(acc), _grads(again)
    for k in gf:
        assert np.array_equal(gf[k], g2[k]), k          # bitwise repeatable
        assert norm_err(ga[k], gf[k]) < 1e-4, k         # only the float summation order differs


def test_backbone_keep_inputs_recomputes_the_same_gradients():
    """SSM_KEEP_INPUTS keeps only the layer inputs and reruns each layer's forward in
    the backward: the same kernels rebuild the same activations, so the forward's
    outputs and every gradient equal those of SSM_KEEP_ALL bitwise."""
    shape = SHAPES[1]
    L, Bt, T, mid, dm, di, N, R, K = shape
    bp, layers = _inputs(shape, seed=91)
    tb, tl = _dev(bp, layers)
    ssm = _ssm()
    print(f"case: backbone keep inputs vs keep all {shape}", flush=True)
    out_a, kept_a = ssm.mamba_backbone_fwd(tb["inp"], tb["W_ip"], tb["b_ip"], tb["norm_f_w"], tl, keep="all")
    out_i, kept_i = ssm.mamba_backbone_fwd(tb["inp"], tb["W_ip"], tb["b_ip"], tb["norm_f_w"], tl, keep="inputs")
    assert kept_i["saved"] is None
    ga = ssm.mamba_backbone_bwd(tb["inp"], tb["W_ip"], tb["norm_f_w"], tl, kept_a, tb["d_out"], need_d_inp=True)
    gi = ssm.mamba_backbone_bwd(tb["inp"], tb["W_ip"], tb["norm_f_w"], tl, kept_i, tb["d_out"], need_d_inp=True)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_i)
    for xa, xi in zip(kept_a["xs"], kept_i["xs"]):
        assert torch.equal(xa, xi)
    a, i = _grads(ga), _grads(gi)
    for k in a:
        assert np.array_equal(a[k], i[k]), k
    assert torch.equal(ga["d_inp"], gi["d_inp"])


def test_backbone_keep_inputs_accumulates_like_keep_all():
    """Two micro-batches summed into one set of gradient buffers under SSM_KEEP_INPUTS
    (each backward reruns the layer forwards into its workspace) equal the same sum
    under SSM_KEEP_ALL bitwise; asking the inputs plan to keep scan states is refused."""
    shape = SHAPES[1]
    ssm = _ssm()
    print(f"case: backbone keep inputs, two accumulated micro-batches {shape}", flush=True)
    sums = {}
    for keep in ("all", "inputs"):
        acc = None
        for seed in (93, 94):
            bp, layers = _inputs(shape, seed=seed)
            tb, tl = _dev(bp, layers)
            _, kept = ssm.mamba_backbone_fwd(tb["inp"], tb["W_ip"], tb["b_ip"], tb["norm_f_w"], tl, keep=keep)
            args = (tb["inp"], tb["W_ip"], tb["norm_f_w"], tl, kept, tb["d_out"])
            acc = ssm.mamba_backbone_bwd(*args) if acc is None else ssm.mamba_backbone_bwd(*args, out=acc,
                                                                                          accumulate=True)
        torch.cuda.synchronize()
        sums[keep] = _grads(acc)
    for k in sums["all"]:
        assert np.array_equal(sums["all"][k], sums["inputs"][k]), k
    with pytest.raises(Exception):
        ssm.mamba_backbone_fwd(tb["inp"], tb["W_ip"], tb["b_ip"], tb["norm_f_w"], tl, keep="inputs",
                               keep_scan_states=True)
    with pytest.raises(Exception):
        ssm.mamba_backbone_fwd(tb["inp"], tb["W_ip"], tb["b_ip"], tb["norm_f_w"], tl, keep="inputs",
                               keep_gemm_inputs=True)
