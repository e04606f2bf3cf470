"""GPU parity of ssm_scan_bwd_ckpt (the backward that starts every 8-step chunk
from the forward's saved state) against the fp64 oracle.

Two sources for the chunk states:
  * the oracle's own forward states h_{8k-1}, rounded to float32, so that both
    sides take the same inputs;
  * the GPU forward (ssm_scan_fwd with ckpt_every = 8), end to end, as a
    training step would run it; the oracle still sees only u, delta, A_log, B, C,
    D, z and d_out.
Bars as for ssm_scan_bwd: 1e-4 (float32 storage) and 2e-2 (bfloat16 storage) on
max |gpu - oracle| / max |oracle| per output tensor.
"""
import numpy as np
import pytest
import torch

from oracle import layer as orc_layer
from oracle import ssm as orc
from synth import CONFIGS, scan_inputs
from tests._util import SCAN_OUTPUTS, norm_err

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}
DEV = "cuda:0"


def _ssm():
    import selective_state_space_bwd_amd as ssm
    return ssm


def _to_dev(p, dtype):
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    return {k: (torch.from_numpy(np.ascontiguousarray(v)) if k in ("A_log", "D")
                else torch.from_numpy(np.ascontiguousarray(v)).to(tdt)).to(DEV) for k, v in p.items()}


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _check(g, r, tol, keys=SCAN_OUTPUTS, label=""):
    errs = {k: norm_err(g[k], r[k]) for k in keys}
    print(f"  {label} errors: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{label}: {bad} exceed {tol}"


def oracle_ckpt(p):
    """h_ckpt[b, k] = h_{8k-1} (zero for k = 0) from the oracle's forward, float32."""
    nb, T, di = p["u"].shape
    N = p["A_log"].shape[1]
    nk = (T + 7) // 8
    ck = np.zeros((nb, nk, N, di))
    if nk > 1:
        ck[:, 1:] = orc.ssm_states_at(p["u"], p["delta"], p["A_log"], p["B"], [8 * k - 1 for k in range(1, nk)])
    return torch.from_numpy(ck.astype(np.float32)).to(DEV)


def gpu_bwd_ckpt(p, dt, h_ckpt, **kw):
    t = _to_dev(p, dt)
    g = _ssm().ssm_scan_bwd_ckpt(t["u"], t["delta"], t["A_log"], t["B"], t["C"], t["D"], t["z"], t["d_out"],
                                 h_ckpt, **kw)
    torch.cuda.synchronize()
    return {k: _np(v) for k, v in g.items()}


def oracle_bwd(p):
    return orc.ssm_scan_bwd(p["u"], p["delta"], p["A_log"], p["B"], p["C"], p["D"], p["z"], p["d_out"])


def _random_params(p, seed):
    rng = np.random.default_rng(seed)
    p["A_log"] = (p["A_log"] + rng.standard_normal(p["A_log"].shape)).astype(np.float32)
    p["D"] = (p["D"] + 0.5 * rng.standard_normal(p["D"].shape)).astype(np.float32)
    return p


SHAPES = [
    # batch, seqlen, d_inner, d_state, dtype, variant, seg_len
    (2, 63, 33, 16, "f32", "default", 0),
    (1, 1000, 100, 8, "f32", "random_A", 64),
    (3, 1, 7, 4, "f32", "default", 0),
    (2, 257, 300, 16, "f32", "long_memory", 16),
    (1, 200, 64, 16, "f32", "last_chunk", 8),
    (2, 96, 40, 16, "f32", "zero_delta", 8),
    (2, 512, 256, 4, "f32", "random_A", 128),
    (1, 9, 1, 16, "f32", "long_memory", 8),
    (2, 130, 520, 8, "bf16", "default", 32),
    (1, 300, 70, 16, "bf16", "long_memory", 24),
    (2, 77, 129, 16, "bf16", "random_A", 0),
    (2, 45, 67, 4, "bf16", "default", 16),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{s[0]}T{s[1]}D{s[2]}N{s[3]}-{s[4]}-{s[5]}-seg{s[6]}"
                                              for s in SHAPES])
def test_from_oracle_states(shape):
    nb, T, di, N, dt, variant, seg = shape
    p = scan_inputs(nb, T, di, N, dt, seed=200 + T, variant=variant, last_steps=24)
    if variant == "random_A":
        p = _random_params(p, 9)
    ck = oracle_ckpt(p)
    print(f"case: ssm_scan_bwd_ckpt B{nb} T{T} Di{di} N{N} {dt} {variant} seg_len {seg}", flush=True)
    _check(gpu_bwd_ckpt(p, dt, ck, seg_len=seg), oracle_bwd(p), TOL[dt], label=variant)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_from_gpu_forward(dt):
    """Forward with checkpoints, then the backward from them; also agrees with the
    backward that rebuilds the states itself."""
    nb, T, di, N = 2, 333, 96, 16
    p = _random_params(scan_inputs(nb, T, di, N, dt, seed=51, variant="long_memory"), 6)
    t = _to_dev(p, dt)
    print(f"case: ssm_scan_fwd ckpt_every 8 -> ssm_scan_bwd_ckpt B{nb} T{T} Di{di} N{N} {dt}", flush=True)
    f = _ssm().ssm_scan_fwd(t["u"], t["delta"], t["A_log"], t["B"], t["C"], t["D"], t["z"], want_y=False,
                            want_out=False, ckpt_every=8)
    g = _ssm().ssm_scan_bwd_ckpt(t["u"], t["delta"], t["A_log"], t["B"], t["C"], t["D"], t["z"], t["d_out"],
                                 f["h_ckpt"], seg_len=40)
    h = _ssm().ssm_scan_bwd(t["u"], t["delta"], t["A_log"], t["B"], t["C"], t["D"], t["z"], t["d_out"], seg_len=40)
    torch.cuda.synchronize()
    g = {k: _np(v) for k, v in g.items()}
    _check(g, oracle_bwd(p), TOL[dt], label="end to end")
    _check(g, {k: _np(v) for k, v in h.items()}, 2e-5 if dt == "f32" else 1e-2, label="vs ssm_scan_bwd")


def test_carry_only_gradient_reaches_early_steps():
    """d_out is zero except in the last 8 steps, so every earlier gradient comes
    through the adjoint-only carry across 64 segments."""
    p = scan_inputs(1, 512, 64, 16, "f32", seed=5, variant="last_chunk", last_steps=8)
    p["delta"] = (p["delta"] * 0.02).astype(np.float32)
    r = oracle_bwd(p)
    assert np.max(np.abs(r["d_u"][:, :100])) > 1e-3 * np.max(np.abs(r["d_u"]))
    print("case: ssm_scan_bwd_ckpt carry-only B1 T512 Di64 N16 seg_len 8", flush=True)
    _check(gpu_bwd_ckpt(p, "f32", oracle_ckpt(p), seg_len=8), r, TOL["f32"], label="carry-only")


def test_softplus_epilogue():
    nb, T, di, N = 2, 100, 48, 16
    p = scan_inputs(nb, T, di, N, "f32", seed=23)
    rng = np.random.default_rng(8)
    raw = rng.standard_normal((nb, T, di)) * 3.0
    raw[1, -5:, :4] = 30.0
    p["delta"] = orc_layer.softplus_fwd(raw).astype(np.float32)
    r = oracle_bwd(p)
    want = orc_layer.softplus_bwd(raw, r["d_delta"])
    print("case: ssm_scan_bwd_ckpt softplus epilogue B2 T100 Di48 N16 seg_len 16", flush=True)
    g = gpu_bwd_ckpt(p, "f32", oracle_ckpt(p), softplus_epilogue=True, seg_len=16)
    assert norm_err(g["d_delta"], want) < TOL["f32"]
    _check(g, r, TOL["f32"], keys=("d_u", "d_A_log", "d_B", "d_C", "d_D", "d_z"), label="softplus")


def test_bitwise_deterministic_and_workspace_reuse():
    p = scan_inputs(2, 300, 200, 16, "f32", seed=19)
    t = _to_dev(p, "f32")
    ck = oracle_ckpt(p)
    ssm = _ssm()
    dims = ssm.ssm_dims(2, 300, 200, 16, 16, 16, 32, 0)
    import ctypes
    nbytes = int(ssm.lib().ssm_scan_bwd_ckpt_workspace_size(ctypes.byref(dims), ssm.SSM_F32))
    ws = torch.full((nbytes,), 255, dtype=torch.uint8, device=DEV)   # NaN patterns
    print("case: ssm_scan_bwd_ckpt determinism B2 T300 Di200 N16 seg_len 32", flush=True)
    args = (t["u"], t["delta"], t["A_log"], t["B"], t["C"], t["D"], t["z"], t["d_out"], ck)
    a = ssm.ssm_scan_bwd_ckpt(*args, seg_len=32, workspace=ws)
    a = {k: v.clone() for k, v in a.items()}
    b = ssm.ssm_scan_bwd_ckpt(*args, seg_len=32, workspace=ws)
    torch.cuda.synchronize()
    for k in SCAN_OUTPUTS:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.timeout(900)
def test_full_size_sampled_mamba370m():
    """The mamba-370m-shaped workload (B8 T2048 Di2048 N16 f32) forward with
    checkpoints and the backward from them on the GPU, in the bench's launch
    configuration; the oracle recomputes 48 sampled channels and batch element 0."""
    c = CONFIGS["mamba370m"]
    print(f"case: {c.name} seed {c.seed}: generating inputs", flush=True)
    p = scan_inputs(c.batch, c.seqlen, c.d_inner, c.d_state, c.dtype, c.seed)
    t = _to_dev(p, c.dtype)
    print(f"case: {c.name}: ssm_scan_fwd ckpt_every 8 + ssm_scan_bwd_ckpt on the GPU", flush=True)
    f = _ssm().ssm_scan_fwd(t["u"], t["delta"], t["A_log"], t["B"], t["C"], t["D"], t["z"], want_y=False,
                            want_out=False, ckpt_every=8)
    g = _ssm().ssm_scan_bwd_ckpt(t["u"], t["delta"], t["A_log"], t["B"], t["C"], t["D"], t["z"], t["d_out"],
                                 f["h_ckpt"])
    torch.cuda.synchronize()
    del f, t
    g = {k: _np(v) for k, v in g.items()}
    for k in SCAN_OUTPUTS:
        assert np.all(np.isfinite(g[k])), k
    rng = np.random.default_rng(1)
    ch = np.sort(rng.choice(c.d_inner, 48, replace=False))
    q = {k: (np.ascontiguousarray(v[:, :, ch]) if k in ("u", "delta", "z", "d_out") else v) for k, v in p.items()}
    q["A_log"], q["D"] = p["A_log"][ch], p["D"][ch]
    print(f"case: {c.name}: oracle on 48 channels", flush=True)
    r = oracle_bwd(q)
    sub = {k: g[k][:, :, ch] for k in ("d_u", "d_delta", "d_z")}
    sub["d_A_log"], sub["d_D"] = g["d_A_log"][ch], g["d_D"][ch]
    _check(sub, r, TOL[c.dtype], keys=("d_u", "d_delta", "d_z", "d_A_log", "d_D"), label="channels")
    print(f"case: {c.name}: oracle on batch element 0", flush=True)
    q = {k: (v[:1] if v.ndim == 3 else v) for k, v in p.items()}
    r = oracle_bwd(q)
    _check({"d_B": g["d_B"][:1], "d_C": g["d_C"][:1]}, r, TOL[c.dtype], keys=("d_B", "d_C"), label="batch 0")


@pytest.mark.parametrize("nb,T", [(0, 16), (2, 0)])
def test_empty_inputs(nb, T):
    """Sums over nothing: d_A_log and d_D are zeroed, or left as they are when accumulating."""
    p = scan_inputs(1, 8, 12, 8, "f32", seed=1)
    t = _to_dev(p, "f32")
    e = torch.empty((nb, T, 12), device=DEV)
    eb = torch.empty((nb, T, 8), device=DEV)
    h = torch.empty((nb, (T + 7) // 8, 8, 12), device=DEV)
    print(f"case: ssm_scan_bwd_ckpt empty batch {nb} seqlen {T}", flush=True)
    g = _ssm().ssm_scan_bwd_ckpt(e, e, t["A_log"], eb, eb, t["D"], e, e, h,
                                 out={"d_A_log": torch.full_like(t["A_log"], 3.0), "d_D": torch.full_like(t["D"], 3.0)})
    a = _ssm().ssm_scan_bwd_ckpt(e, e, t["A_log"], eb, eb, t["D"], e, e, h, accumulate=True,
                                 out={"d_A_log": torch.full_like(t["A_log"], 3.0), "d_D": torch.full_like(t["D"], 3.0)})
    torch.cuda.synchronize()
    assert torch.all(g["d_A_log"] == 0) and torch.all(g["d_D"] == 0)
    assert torch.all(a["d_A_log"] == 3.0) and torch.all(a["d_D"] == 3.0)
