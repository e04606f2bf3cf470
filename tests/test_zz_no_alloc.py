"""ssm_scan_bwd_ckpt_noalloc (scratch in a static device array, no workspace
argument) against ssm_scan_bwd_ckpt (caller workspace) and the fp64 oracle.

The entry point is called through the C ABI with every output preallocated.
Two calls run back to back, the second on a smaller input, so the second one
starts from the first one's leftovers in the shared scratch.  Bars as for the
scan backward: 1e-4 (float32 storage) and 2e-2 (bfloat16 storage) on
max |gpu - ref| / max |ref| per output tensor; the two entry points run the
same kernels on the same plan, so their outputs are also compared bit for bit.
"""
import ctypes

import numpy as np
import pytest
import torch

from oracle import ssm as orc
from synth import scan_inputs
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


def _oracle_ckpt(p):
    """h_ckpt[b, k] = h_{8k-1} (zero for k = 0) from the oracle's forward, rounded to float32."""
    nb, T, di = p["u"].shape
    N = p["A_log"].shape[1]
    nk = (T + 7) // 8
    ck = np.zeros((nb, nk, N, di))
    if nk > 1:
        ck[:, 1:] = orc.ssm_states_at(p["u"], p["delta"], p["A_log"], p["B"], [8 * k - 1 for k in range(1, nk)])
    return torch.from_numpy(ck.astype(np.float32)).to(DEV)


def _outputs(t):
    """Every output of one call, allocated before it."""
    nb, T, di = t["u"].shape
    N = t["A_log"].shape[1]
    o = {k: torch.full_like(t["u"], float("nan")) for k in ("d_u", "d_delta", "d_z")}
    o["d_B"] = torch.full((nb, T, N), float("nan"), dtype=t["u"].dtype, device=DEV)
    o["d_C"] = torch.full((nb, T, N), float("nan"), dtype=t["u"].dtype, device=DEV)
    o["d_A_log"] = torch.full_like(t["A_log"], float("nan"))
    o["d_D"] = torch.full_like(t["D"], float("nan"))
    return o


def _call_noalloc(t, ck, o, dtype, seg_len):
    ssm = _ssm()
    nb, T, di = t["u"].shape
    N = t["A_log"].shape[1]
    dims = ssm.ssm_dims(nb, T, di, N, N, N, seg_len, 0)
    p = lambda x: ctypes.c_void_p(x.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = ssm.lib().ssm_scan_bwd_ckpt_noalloc(
        p(t["u"]), p(t["delta"]), p(t["A_log"]), p(t["B"]), p(t["C"]), p(t["D"]), p(t["z"]), p(t["d_out"]), p(ck),
        p(o["d_u"]), p(o["d_delta"]), p(o["d_A_log"]), p(o["d_B"]), p(o["d_C"]), p(o["d_D"]), p(o["d_z"]), 0,
        ctypes.byref(dims), ssm.SSM_F32 if dtype == "f32" else ssm.SSM_BF16, stream)
    assert rc == 0, ssm.lib().ssm_last_error()


def _np(x):
    return x.float().cpu().numpy().astype(np.float64)


CASES = {
    # two calls in a row, the second on a smaller input: (batch, seqlen, d_inner, d_state, variant, seg_len)
    "f32": [(2, 300, 160, 16, "random_A", 40), (1, 77, 33, 16, "long_memory", 0)],
    "bf16": [(2, 257, 300, 16, "default", 24), (1, 40, 64, 8, "long_memory", 8)],
}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noalloc_matches_workspace_entry(dtype):
    ssm = _ssm()
    for i, (nb, T, di, N, variant, seg) in enumerate(CASES[dtype]):
        print(f"case: call {i + 1} ssm_scan_bwd_ckpt_noalloc B{nb} T{T} Di{di} N{N} {dtype} {variant} "
              f"seg_len {seg}", flush=True)
        p = scan_inputs(nb, T, di, N, dtype, seed=70 + i, variant=variant)
        if variant == "random_A":
            rng = np.random.default_rng(3)
            p["A_log"] = (p["A_log"] + rng.standard_normal(p["A_log"].shape)).astype(np.float32)
        t = _to_dev(p, dtype)
        ck = _oracle_ckpt(p)
        o = _outputs(t)
        _call_noalloc(t, ck, o, dtype, seg)
        ref = ssm.ssm_scan_bwd_ckpt(t["u"], t["delta"], t["A_log"], t["B"], t["C"], t["D"], t["z"], t["d_out"], ck,
                                    seg_len=seg)
        torch.cuda.synchronize()
        got = {k: _np(v) for k, v in o.items()}
        want = {k: _np(v) for k, v in ref.items()}
        orc_r = orc.ssm_scan_bwd(p["u"], p["delta"], p["A_log"], p["B"], p["C"], p["D"], p["z"], p["d_out"])
        errs = {k: norm_err(got[k], want[k]) for k in SCAN_OUTPUTS}
        oerr = {k: norm_err(got[k], orc_r[k]) for k in SCAN_OUTPUTS}
        print("  vs ssm_scan_bwd_ckpt: " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
        print("  vs oracle:            " + " ".join(f"{k}={v:.1e}" for k, v in oerr.items()), flush=True)
        assert all(v <= TOL[dtype] for v in errs.values()), errs
        assert all(v <= TOL[dtype] for v in oerr.values()), oerr
        for k in SCAN_OUTPUTS:
            assert torch.equal(o[k], ref[k]), f"{k} differs bitwise from ssm_scan_bwd_ckpt"


def test_noalloc_rejects_oversize():
    """A shape whose plan needs more than the static scratch fails before any launch."""
    ssm = _ssm()
    cap = ssm.ssm_scan_bwd_ckpt_noalloc_capacity()
    dims = ssm.ssm_dims(64, 16384, 4096, 16, 16, 16, 256, 0)
    need = ssm.lib().ssm_scan_bwd_ckpt_workspace_size(ctypes.byref(dims), ssm.SSM_F32)
    assert need > cap
    fake = ctypes.c_void_p(0x1000)
    rc = ssm.lib().ssm_scan_bwd_ckpt_noalloc(*([fake] * 16), 0, ctypes.byref(dims), ssm.SSM_F32, None)
    assert rc == ssm.SSM_ERR_WORKSPACE
    assert b"static scratch" in ssm.lib().ssm_last_error()
