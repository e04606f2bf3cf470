"""GPU parity of gating_bwd, conv1d_bwd and rmsnorm_bwd against the fp64 oracle."""
import numpy as np
import pytest
import torch

from oracle import layer as orc
from oracle import ssm as orc_ssm
from synth import round_storage
from tests._util import norm_err

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}
DEV = "cuda:0"


def _ssm():
    import selective_state_space_bwd_amd as ssm
    return ssm


def _dev(x, dt):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float32 if dt == "f32" else torch.bfloat16).to(DEV)


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [1, 1000, 65537])
def test_gating_bwd(dt, n):
    rng = np.random.default_rng(n)
    d_out, y, z = (round_storage(rng.standard_normal(n) * s, dt) for s in (1.0, 2.0, 3.0))
    print(f"case: gating_bwd n {n} {dt}", flush=True)
    d_y, d_z = _ssm().gating_bwd(_dev(d_out, dt), _dev(y, dt), _dev(z, dt))
    torch.cuda.synchronize()
    ry, rz = orc_ssm.gating_bwd(d_out, y, z)
    assert norm_err(_np(d_y), ry) < TOL[dt]
    assert norm_err(_np(d_z), rz) < TOL[dt]


# batch, seqlen, d_inner, d_conv, dtype, row stride of x (>= d_inner).  Rows of whole
# 16-byte vectors (f32 d_inner and stride multiples of 4, bf16 of 8) take the vector
# kernel (128-step blocks, ragged here), the others the one-channel-per-thread kernel.
CONV = [
    (2, 150, 70, 4, "f32", 70),
    (1, 3, 9, 4, "f32", 9),
    (3, 64, 33, 2, "f32", 40),
    (2, 129, 256, 4, "bf16", 512),
    (1, 200, 16, 1, "f32", 16),
    (2, 65, 20, 8, "f32", 20),
    (2, 300, 136, 3, "bf16", 136),
    (1, 77, 36, 4, "bf16", 36),
    (1, 140, 64, 8, "bf16", 64),
    (2, 260, 64, 4, "f32", 96),
]


@pytest.mark.parametrize("case", CONV, ids=[f"B{c[0]}T{c[1]}D{c[2]}K{c[3]}-{c[4]}-ld{c[5]}" for c in CONV])
def test_conv1d_bwd(case):
    nb, T, di, K, dt, ldx = case
    rng = np.random.default_rng(T * 7 + K)
    xw = round_storage(rng.standard_normal((nb, T, ldx)), dt)
    x = xw[:, :, :di]
    w = rng.standard_normal((di, K)).astype(np.float32) * 0.5
    bias = rng.standard_normal(di).astype(np.float32) * 0.3
    du = round_storage(rng.standard_normal((nb, T, di)), dt)
    c = orc.conv1d_fwd(x, w, bias)
    g = du * orc.silu_grad(c)
    rdx, rdw, rdb = orc.conv1d_bwd(x, w, g)
    xt = _dev(xw, dt)[:, :, :di]
    print(f"case: conv1d_bwd B{nb} T{T} Di{di} K{K} {dt} ld_x {ldx}", flush=True)
    dx, dw, db = _ssm().conv1d_bwd(xt, torch.from_numpy(w).to(DEV), torch.from_numpy(bias).to(DEV), _dev(du, dt))
    torch.cuda.synchronize()
    assert norm_err(_np(dx), rdx) < TOL[dt]
    assert norm_err(_np(dw), rdw) < TOL[dt]
    assert norm_err(_np(db), rdb) < TOL[dt]


# rows of 16-byte vectors up to 6 per lane take the wave-per-row kernels (f32 dim 12, 100, 1536;
# bf16 dim 1000, 1536, 2048, 3072); the rest the block-per-rows kernels (f32 4096, bf16 36, 4096)
RMS = [(5, 12, "f32", False), (300, 1536, "f32", True), (64, 1536, "bf16", True), (33, 4096, "f32", False),
       (1, 100, "f32", True), (70, 1000, "bf16", False), (17, 36, "bf16", True), (130, 4096, "bf16", True),
       (1000, 2048, "bf16", True), (200, 3072, "bf16", False)]


@pytest.mark.parametrize("case", RMS, ids=[f"R{c[0]}D{c[1]}-{c[2]}-res{int(c[3])}" for c in RMS])
def test_rmsnorm_bwd(case):
    rows, dim, dt, res = case
    rng = np.random.default_rng(rows + dim)
    x = round_storage(rng.standard_normal((rows, dim)) * 2.0, dt)
    dy = round_storage(rng.standard_normal((rows, dim)), dt)
    w = (1.0 + 0.2 * rng.standard_normal(dim)).astype(np.float32)
    dr = round_storage(rng.standard_normal((rows, dim)), dt) if res else None
    rdx, rdw = orc.rmsnorm_bwd(x, w, dy, 1e-5)
    if res:
        rdx = rdx + dr
    print(f"case: rmsnorm_bwd rows {rows} dim {dim} {dt} residual {res}", flush=True)
    dx, dw = _ssm().rmsnorm_bwd(_dev(x, dt), torch.from_numpy(w).to(DEV), _dev(dy, dt),
                                _dev(dr, dt) if res else None, 1e-5)
    torch.cuda.synchronize()
    assert norm_err(_np(dx), rdx) < TOL[dt]
    assert norm_err(_np(dw), rdw) < TOL[dt]
