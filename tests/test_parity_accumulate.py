"""GPU parity of the accumulate mode (SSM_BWD_ACCUMULATE): parameter gradients are
added into the caller's buffers, as mamba-rs's `+=` gradient accumulators take
them (Phase B3's d_layer.a_log and d_param), so that micro-batches sum into one
set of buffers.

Each entry point gets its parameter-gradient buffers pre-filled with random
values R of the gradients' own scale and must return R + oracle, to the same
bars as its overwrite mode (max |gpu - expected| / max |expected|); per-element
gradients are still written.  The layer check adds two micro-batches into one
set of buffers and compares them with one call over both.
"""
import numpy as np
import pytest
import torch

from oracle import layer as orc
from oracle import ssm as orc_ssm
from synth import round_bf16, round_storage, scan_inputs, layer_inputs
from tests._util import SCAN_OUTPUTS, norm_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {"f32": 1e-4, "bf16": 2e-2}


def _ssm():
    import selective_state_space_bwd_amd as ssm
    return ssm


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _prefill(ref, seed):
    """float32 values of the reference's scale, as a device tensor and as fp64."""
    rng = np.random.default_rng(seed)
    r = (rng.standard_normal(np.shape(ref)) * (np.max(np.abs(ref)) + 1e-30)).astype(np.float32)
    return torch.from_numpy(r).to(DEV), r.astype(np.float64)


def _dev(x, dt):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float32 if dt == "f32" else torch.bfloat16).to(DEV)


@pytest.mark.parametrize("dt,ckpt", [("f32", False), ("bf16", False), ("f32", True)])
def test_scan_bwd_accumulate(dt, ckpt):
    nb, T, di, N = 2, 150, 96, 16
    p = scan_inputs(nb, T, di, N, dt, seed=61, variant="long_memory")
    ref = orc_ssm.ssm_scan_bwd(p["u"], p["delta"], p["A_log"], p["B"], p["C"], p["D"], p["z"], p["d_out"])
    t = {k: (torch.from_numpy(np.ascontiguousarray(v)).to(DEV) if k in ("A_log", "D") else _dev(v, dt))
         for k, v in p.items()}
    ra, ra64 = _prefill(ref["d_A_log"], 1)
    rd, rd64 = _prefill(ref["d_D"], 2)
    out = {"d_A_log": ra.clone(), "d_D": rd.clone()}
    args = (t["u"], t["delta"], t["A_log"], t["B"], t["C"], t["D"], t["z"], t["d_out"])
    print(f"case: ssm_scan_bwd{'_ckpt' if ckpt else ''} accumulate B{nb} T{T} Di{di} N{N} {dt} seg_len 32", flush=True)
    if ckpt:
        h = _ssm().ssm_scan_fwd(*args[:6], want_y=False, want_out=False, ckpt_every=8)["h_ckpt"]
        g = _ssm().ssm_scan_bwd_ckpt(*args, h, accumulate=True, out=out, seg_len=32)
    else:
        g = _ssm().ssm_scan_bwd(*args, accumulate=True, out=out, seg_len=32)
    torch.cuda.synchronize()
    assert norm_err(_np(g["d_A_log"]), ra64 + ref["d_A_log"]) < TOL[dt]
    assert norm_err(_np(g["d_D"]), rd64 + ref["d_D"]) < TOL[dt]
    for k in ("d_u", "d_delta", "d_z", "d_B", "d_C"):
        assert norm_err(_np(g[k]), ref[k]) < TOL[dt], k


@pytest.mark.parametrize("M,K,N", [(300, 72, 200), (2048, 96, 3072), (777, 1536, 640)])
def test_linear_bwd_accumulate(M, K, N):
    """Both the single-pass epilogue and the split-k reduction (dt_proj shape) add into dW; db adds too."""
    rng = np.random.default_rng(M + K + N)
    X = round_bf16(rng.standard_normal((M, K)))
    W = round_bf16(rng.standard_normal((N, K)) * 0.02)
    dY = round_bf16(rng.standard_normal((M, N)))
    rx, rw, rb = orc.linear_bwd(X, W, dY)
    pw, pw64 = _prefill(rw, 3)
    pb, pb64 = _prefill(rb, 4)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).to(DEV)
    print(f"case: linear_bwd accumulate M {M} K {K} N {N}", flush=True)
    dX, dW, db = _ssm().linear_bwd(bf(X), bf(W), bf(dY), need_db=True, dW=pw.clone(), db=pb.clone(), accumulate=True)
    torch.cuda.synchronize()
    assert norm_err(_np(dX), rx) < 1e-2
    assert norm_err(_np(dW), pw64 + rw) < 1e-4
    assert norm_err(_np(db), pb64 + rb) < 1e-4


@pytest.mark.parametrize("di,dt", [(64, "bf16"), (70, "f32")])   # vector and one-channel-per-thread kernels
def test_conv1d_bwd_accumulate(di, dt):
    nb, T, K = 2, 150, 4
    rng = np.random.default_rng(di)
    x = round_storage(rng.standard_normal((nb, T, di)), dt)
    w = rng.standard_normal((di, K)).astype(np.float32) * 0.5
    bias = rng.standard_normal(di).astype(np.float32) * 0.3
    du = round_storage(rng.standard_normal((nb, T, di)), dt)
    g = du * orc.silu_grad(orc.conv1d_fwd(x, w, bias))
    rdx, rdw, rdb = orc.conv1d_bwd(x, w, g)
    pw, pw64 = _prefill(rdw, 5)
    pb, pb64 = _prefill(rdb, 6)
    print(f"case: conv1d_bwd accumulate B{nb} T{T} Di{di} K{K} {dt}", flush=True)
    dx, dw, db = _ssm().conv1d_bwd(_dev(x, dt), torch.from_numpy(w).to(DEV), torch.from_numpy(bias).to(DEV),
                                   _dev(du, dt), d_w=pw.clone(), d_b=pb.clone(), accumulate=True)
    torch.cuda.synchronize()
    assert norm_err(_np(dx), rdx) < TOL[dt]
    assert norm_err(_np(dw), pw64 + rdw) < TOL[dt]
    assert norm_err(_np(db), pb64 + rdb) < TOL[dt]


@pytest.mark.parametrize("rows,dim,dt", [(300, 1536, "bf16"), (33, 4096, "f32")])   # wave and block kernels
def test_rmsnorm_bwd_accumulate(rows, dim, dt):
    rng = np.random.default_rng(rows)
    x = round_storage(rng.standard_normal((rows, dim)) * 2.0, dt)
    dy = round_storage(rng.standard_normal((rows, dim)), dt)
    w = (1.0 + 0.2 * rng.standard_normal(dim)).astype(np.float32)
    rdx, rdw = orc.rmsnorm_bwd(x, w, dy, 1e-5)
    pw, pw64 = _prefill(rdw, 7)
    print(f"case: rmsnorm_bwd accumulate rows {rows} dim {dim} {dt}", flush=True)
    dx, dw = _ssm().rmsnorm_bwd(_dev(x, dt), torch.from_numpy(w).to(DEV), _dev(dy, dt), None, 1e-5,
                                dw=pw.clone(), accumulate=True)
    torch.cuda.synchronize()
    assert norm_err(_np(dx), rdx) < TOL[dt]
    assert norm_err(_np(dw), pw64 + rdw) < TOL[dt]


def test_layer_bwd_two_micro_batches():
    """Two one-sequence calls, the second accumulating, equal one two-sequence call
    (only the float summation order of the parameter sums differs), and the
    accumulated gradients match the oracle's for both sequences."""
    Bt, T, dm, di, N, R, K = 2, 160, 64, 128, 16, 8, 4
    p = layer_inputs(Bt, T, dm, di, N, R, K, "bf16", seed=71, weight_std=0.02 * np.sqrt(1536.0 / dm))
    bfk = ("x", "d_out", "W_in", "W_x", "W_dt", "W_out")
    t = {k: (torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16) if k in bfk
             else torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))).to(DEV) for k, v in p.items()}
    ssm = _ssm()
    W = {k: t[k] for k in ssm.LAYER_WEIGHTS}
    print(f"case: mamba_layer_bwd accumulate over 2 micro-batches B{Bt} T{T} dm{dm} di{di}", flush=True)
    _, saved = ssm.mamba_layer_fwd(t["x"], W)
    full = ssm.mamba_layer_bwd(t["x"], W, saved, t["d_out"])
    acc = None
    for b in range(Bt):
        xb, db = t["x"][b:b + 1].contiguous(), t["d_out"][b:b + 1].contiguous()
        sb = {k: v[b:b + 1].contiguous() for k, v in saved.items()}
        if acc is None:
            acc = ssm.mamba_layer_bwd(xb, W, sb, db)
        else:
            o = {k: v for k, v in acc.items() if k != "d_x"}
            acc = ssm.mamba_layer_bwd(xb, W, sb, db, out=o, accumulate=True)
    torch.cuda.synchronize()
    params = [k for k in ssm.LAYER_GRADS]
    for k in params:
        assert norm_err(_np(acc[k]), _np(full[k])) < 1e-4, k
    ref = orc.layer_bwd(p, p["d_out"], N, R)
    for k in params:
        assert norm_err(_np(acc[k]), ref[k]) < 3e-2, k
