"""GPU parity of the selective-scan kernels against the fp64 oracle.

Error metric per output tensor: max |gpu - oracle| / max |oracle| (absolute if
the oracle tensor is all zero).  Bars: 1e-4 for float32 storage, 2e-2 for
bfloat16 storage (both sides take the same bf16-rounded inputs; the GPU
computes in float32, the oracle in float64).
"""
import numpy as np
import pytest
import torch

from oracle import layer as orc_layer
from oracle import ssm as orc
from synth import CONFIGS, round_bf16, scan_inputs
from tests._util import SCAN_OUTPUTS, norm_err

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}
DEV = "cuda:0"


def _ssm():
    import selective_state_space_bwd_amd as ssm
    return ssm


def _to_dev(p, dtype):
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    out = {}
    for k, v in p.items():
        t = torch.from_numpy(np.ascontiguousarray(v))
        if k not in ("A_log", "D"):
            t = t.to(tdt)
        out[k] = t.to(DEV)
    return out


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def gpu_bwd(p, dtype, **kw):
    t = _to_dev(p, dtype)
    g = _ssm().ssm_scan_bwd(t["u"], t["delta"], t["A_log"], t["B"], t["C"], t["D"], t["z"], t["d_out"], **kw)
    torch.cuda.synchronize()
    return {k: _np(v) for k, v in g.items()}


def oracle_bwd(p):
    return orc.ssm_scan_bwd(p["u"], p["delta"], p["A_log"], p["B"], p["C"], p["D"], p["z"], p["d_out"])


def _check(g, r, tol, keys=SCAN_OUTPUTS, label=""):
    errs = {k: norm_err(g[k], r[k]) for k in keys}
    print(f"  {label} errors: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{label}: {bad} exceed {tol}"


def _random_params(p, seed):
    rng = np.random.default_rng(seed)
    p["A_log"] = (p["A_log"] + rng.standard_normal(p["A_log"].shape)).astype(np.float32)
    p["D"] = (p["D"] + 0.5 * rng.standard_normal(p["D"].shape)).astype(np.float32)
    return p


def test_tiny_workload():
    c = CONFIGS["tiny"]
    print(f"case: {c.name} seed {c.seed} ssm_scan_bwd", flush=True)
    p = scan_inputs(c.batch, c.seqlen, c.d_inner, c.d_state, c.dtype, c.seed)
    _check(gpu_bwd(p, c.dtype), oracle_bwd(p), TOL[c.dtype], label=c.name)


SHAPES = [
    # batch, seqlen, d_inner, d_state, dtype, variant, seg_len
    (2, 63, 33, 16, "f32", "default", 0),
    (1, 1000, 100, 8, "f32", "random_A", 64),
    (3, 1, 7, 4, "f32", "default", 0),
    (2, 257, 300, 16, "f32", "long_memory", 16),
    (1, 200, 64, 16, "f32", "last_chunk", 16),
    (2, 96, 40, 16, "f32", "zero_delta", 8),
    (2, 512, 256, 4, "f32", "random_A", 128),
    (1, 64, 256, 16, "f32", "default", 8),
    (1, 9, 1, 16, "f32", "long_memory", 8),
    (2, 130, 520, 8, "bf16", "default", 32),
    (1, 300, 70, 16, "bf16", "long_memory", 24),
    (2, 77, 129, 16, "bf16", "random_A", 0),
    (2, 45, 67, 4, "bf16", "default", 16),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{s[0]}T{s[1]}D{s[2]}N{s[3]}-{s[4]}-{s[5]}-seg{s[6]}"
                                              for s in SHAPES])
def test_shapes_and_variants(shape):
    nb, T, di, N, dt, variant, seg = shape
    print(f"case: ssm_scan_bwd B{nb} T{T} Di{di} N{N} {dt} {variant} seg_len {seg}", flush=True)
    p = scan_inputs(nb, T, di, N, dt, seed=100 + T, variant=variant, last_steps=24)
    if variant == "random_A":
        p = _random_params(p, 7)
    _check(gpu_bwd(p, dt, seg_len=seg), oracle_bwd(p), TOL[dt], label=variant)


def test_segment_length_invariance():
    p = _random_params(scan_inputs(2, 384, 96, 16, "f32", seed=11, variant="long_memory"), 3)
    r = oracle_bwd(p)
    outs = []
    for seg in (8, 16, 64, 128, 384, 0):
        print(f"case: long-memory B2 T384 Di96 N16 seg_len {seg}", flush=True)
        g = gpu_bwd(p, "f32", seg_len=seg)
        _check(g, r, TOL["f32"], label=f"seg {seg}")
        outs.append(g)
    for g in outs[1:]:
        for k in SCAN_OUTPUTS:
            assert norm_err(g[k], outs[0][k]) < 2e-5, k


def test_carry_only_gradient_reaches_early_steps():
    """d_out is zero except in the last 8 steps: every earlier d_u / d_delta comes
    through the adjoint carry across many segments."""
    p = scan_inputs(1, 512, 64, 16, "f32", seed=5, variant="last_chunk", last_steps=8)
    p["delta"] = (p["delta"] * 0.02).astype(np.float32)     # long memory
    r = oracle_bwd(p)
    assert np.max(np.abs(r["d_u"][:, :100])) > 1e-3 * np.max(np.abs(r["d_u"]))
    print("case: carry-only B1 T512 Di64 N16 seg_len 8", flush=True)
    _check(gpu_bwd(p, "f32", seg_len=8), r, TOL["f32"], label="carry-only")


def test_bitwise_deterministic():
    p = scan_inputs(2, 300, 200, 16, "f32", seed=9)
    t = _to_dev(p, "f32")
    ssm = _ssm()
    print("case: determinism B2 T300 Di200 N16", flush=True)
    a = ssm.ssm_scan_bwd(t["u"], t["delta"], t["A_log"], t["B"], t["C"], t["D"], t["z"], t["d_out"], seg_len=32)
    b = ssm.ssm_scan_bwd(t["u"], t["delta"], t["A_log"], t["B"], t["C"], t["D"], t["z"], t["d_out"], seg_len=32)
    torch.cuda.synchronize()
    for k in SCAN_OUTPUTS:
        assert torch.equal(a[k], b[k]), k


def test_softplus_epilogue():
    nb, T, di, N = 2, 100, 48, 16
    p = scan_inputs(nb, T, di, N, "f32", seed=21)
    rng = np.random.default_rng(4)
    raw = rng.standard_normal((nb, T, di)) * 3.0
    raw[0, :5, :3] = 25.0                         # above the threshold: pass-through
    p["delta"] = orc_layer.softplus_fwd(raw).astype(np.float32)
    r = oracle_bwd(p)
    want = orc_layer.softplus_bwd(raw, r["d_delta"])
    print("case: softplus epilogue B2 T100 Di48 N16", flush=True)
    g = gpu_bwd(p, "f32", softplus_epilogue=True)
    assert norm_err(g["d_delta"], want) < TOL["f32"]
    _check(g, r, TOL["f32"], keys=("d_u", "d_A_log", "d_B", "d_C", "d_D", "d_z"), label="softplus")


def test_softplus_epilogue_bf16():
    """The bf16 sweep (lane pairs) with the softplus epilogue.  delta is stored as the bf16-rounded
    softplus of raw, so the oracle's softplus derivative is taken at the raw value that maps to the
    rounded delta.  d_inner 67 is odd: the last lane pair has an idle partner."""
    nb, T, di, N = 2, 100, 67, 16
    p = scan_inputs(nb, T, di, N, "bf16", seed=22)
    rng = np.random.default_rng(5)
    raw = rng.standard_normal((nb, T, di)) * 3.0
    raw[0, :5, :3] = 25.0                         # above the threshold: pass-through
    p["delta"] = round_bf16(orc_layer.softplus_fwd(raw)).astype(np.float32)
    r = oracle_bwd(p)
    want = orc_layer.softplus_bwd(orc_layer.softplus_inv(p["delta"]), r["d_delta"])
    print("case: softplus epilogue bf16 B2 T100 Di67 N16", flush=True)
    g = gpu_bwd(p, "bf16", softplus_epilogue=True)
    assert norm_err(g["d_delta"], want) < TOL["bf16"]
    _check(g, r, TOL["bf16"], keys=("d_u", "d_A_log", "d_B", "d_C", "d_D", "d_z"), label="softplus bf16")


def test_strided_B_C_inside_xdbl_rows():
    """B and C read from, and d_B / d_C written into, a wider [dt | B | C] row."""
    nb, T, di, N, r_ = 2, 70, 64, 16, 6
    p = scan_inputs(nb, T, di, N, "bf16", seed=31)
    t = _to_dev(p, "bf16")
    xdbl = torch.zeros(nb, T, r_ + 2 * N, dtype=torch.bfloat16, device=DEV)
    xdbl[:, :, r_:r_ + N] = t["B"]
    xdbl[:, :, r_ + N:] = t["C"]
    dx = torch.full((nb, T, r_ + 2 * N), 7.0, dtype=torch.bfloat16, device=DEV)
    out = {"d_B": dx[:, :, r_:r_ + N], "d_C": dx[:, :, r_ + N:]}
    print("case: strided B/C bf16 B2 T70 Di64 N16", flush=True)
    g = _ssm().ssm_scan_bwd(t["u"], t["delta"], t["A_log"], xdbl[:, :, r_:r_ + N], xdbl[:, :, r_ + N:], t["D"],
                            t["z"], t["d_out"], out=out, seg_len=16)
    torch.cuda.synchronize()
    assert torch.all(dx[:, :, :r_] == 7.0)
    r = oracle_bwd(p)
    gg = {k: _np(v) for k, v in g.items()}
    _check(gg, r, TOL["bf16"], label="strided")


def test_gate_inside_in_proj_rows():
    """z read from, and d_z written into, the second half of a wider [x | z] row;
    the forward's gated output reads the same strided z."""
    nb, T, di, N = 2, 90, 40, 16
    p = scan_inputs(nb, T, di, N, "bf16", seed=33)
    t = _to_dev(p, "bf16")
    xz = torch.zeros(nb, T, 2 * di + 8, dtype=torch.bfloat16, device=DEV)
    xz[:, :, di:2 * di] = t["z"]
    dxz = torch.full((nb, T, 2 * di + 8), 7.0, dtype=torch.bfloat16, device=DEV)
    print("case: strided z / d_z bf16 B2 T90 Di40 N16", flush=True)
    g = _ssm().ssm_scan_bwd(t["u"], t["delta"], t["A_log"], t["B"], t["C"], t["D"], xz[:, :, di:2 * di],
                            t["d_out"], out={"d_z": dxz[:, :, di:2 * di]}, seg_len=24)
    f = _ssm().ssm_scan_fwd(t["u"], t["delta"], t["A_log"], t["B"], t["C"], t["D"], xz[:, :, di:2 * di])
    torch.cuda.synchronize()
    assert torch.all(dxz[:, :, :di] == 7.0) and torch.all(dxz[:, :, 2 * di:] == 7.0)
    r = oracle_bwd(p)
    gg = {k: _np(v) for k, v in g.items()}
    _check(gg, r, TOL["bf16"], label="strided z")
    _, out = orc.ssm_forward(p["u"], p["delta"], p["A_log"], p["B"], p["C"], p["D"], p["z"])
    assert norm_err(_np(f["out"]), out) < TOL["bf16"]


@pytest.mark.parametrize("nb,T", [(0, 16), (2, 0)])
def test_empty_inputs(nb, T):
    p = scan_inputs(max(nb, 1), max(T, 1), 12, 8, "f32", seed=1)
    t = _to_dev(p, "f32")
    e = torch.empty((nb, T, 12), device=DEV)
    eb = torch.empty((nb, T, 8), device=DEV)
    print(f"case: empty batch {nb} seqlen {T}", flush=True)
    g = _ssm().ssm_scan_bwd(e, e, t["A_log"], eb, eb, t["D"], e, e,
                            out={"d_A_log": torch.full_like(t["A_log"], 3.0), "d_D": torch.full_like(t["D"], 3.0)})
    torch.cuda.synchronize()
    assert torch.all(g["d_A_log"] == 0) and torch.all(g["d_D"] == 0)
    assert g["d_u"].numel() == 0


# (seqlen, ckpt_every, seg_len): whole chunks; a ragged last chunk in the last
# segment with the layer's ckpt_every; a single short segment
FWD_CASES = [(200, 16, 24), (203, 8, 24), (37, 8, 0)]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("T,ce,seg", FWD_CASES, ids=[f"T{c[0]}-ck{c[1]}-seg{c[2]}" for c in FWD_CASES])
def test_forward_outputs_and_checkpoints(dt, T, ce, seg):
    nb, di, N = 2, 72, 16
    p = _random_params(scan_inputs(nb, T, di, N, dt, seed=41, variant="long_memory"), 5)
    t = _to_dev(p, dt)
    print(f"case: ssm_scan_fwd B{nb} T{T} Di{di} N{N} {dt} ckpt_every {ce} seg_len {seg}", flush=True)
    f = _ssm().ssm_scan_fwd(t["u"], t["delta"], t["A_log"], t["B"], t["C"], t["D"], t["z"], ckpt_every=ce,
                            seg_len=seg)
    torch.cuda.synchronize()
    y, out = orc.ssm_forward(p["u"], p["delta"], p["A_log"], p["B"], p["C"], p["D"], p["z"])
    assert norm_err(_np(f["y"]), y) < TOL[dt]
    assert norm_err(_np(f["out"]), out) < TOL[dt]
    steps = [k * ce - 1 for k in range(1, (T + ce - 1) // ce)]
    hs = orc.ssm_states_at(p["u"], p["delta"], p["A_log"], p["B"], steps)      # [B, K-1, N, Di]
    ck = _np(f["h_ckpt"])
    assert np.all(ck[:, 0] == 0)
    assert norm_err(ck[:, 1:], hs) < TOL[dt]


FULL = ["mamba130m", "mamba370m", "mamba2p8b"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    """Full workload on the GPU in the bench's launch configuration; the oracle
    recomputes 48 sampled channels (every per-channel output and the parameter
    gradients of those channels) and the first and last batch elements in full
    (d_B, d_C, sums over every channel)."""
    c = CONFIGS[name]
    print(f"case: {c.name} seed {c.seed}: generating inputs", flush=True)
    p = scan_inputs(c.batch, c.seqlen, c.d_inner, c.d_state, c.dtype, c.seed)
    print(f"case: {c.name}: ssm_scan_bwd on the GPU", flush=True)
    g = gpu_bwd(p, c.dtype)
    for k in SCAN_OUTPUTS:
        assert np.all(np.isfinite(g[k])), k
    rng = np.random.default_rng(0)
    ch = np.sort(rng.choice(c.d_inner, 48, replace=False))
    q = {k: (np.ascontiguousarray(v[:, :, ch]) if k in ("u", "delta", "z", "d_out") else v) for k, v in p.items()}
    q["A_log"], q["D"] = p["A_log"][ch], p["D"][ch]
    print(f"case: {c.name}: oracle on 48 channels", flush=True)
    r = oracle_bwd(q)
    sub = {k: g[k][:, :, ch] for k in ("d_u", "d_delta", "d_z")}
    sub["d_A_log"], sub["d_D"] = g["d_A_log"][ch], g["d_D"][ch]
    _check(sub, r, TOL[c.dtype], keys=("d_u", "d_delta", "d_z", "d_A_log", "d_D"), label="channels")
    for b in sorted({0, c.batch - 1}):
        print(f"case: {c.name}: oracle on batch element {b}", flush=True)
        q = {k: (v[b:b + 1] if v.ndim == 3 else v) for k, v in p.items()}
        r = oracle_bwd(q)
        sub = {"d_B": g["d_B"][b:b + 1], "d_C": g["d_C"][b:b + 1]}
        _check(sub, r, TOL[c.dtype], keys=("d_B", "d_C"), label=f"batch {b}")
