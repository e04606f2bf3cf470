"""GPU parity of reverse_linear_scan against the fp64 oracle (oracle.recurrence):
x_t = b_t + a_{t+1} x_{t+1} along t, and with a = 1 the cumsum backward of rlx-cpu
training_bwd.rs cumsum_backward_row.  Bars as for the scan: 1e-4 (float32
storage), 2e-2 (bfloat16 storage) on max |gpu - oracle| / max |oracle|."""
import numpy as np
import pytest
import torch

from oracle import recurrence as orc
from synth import CONFIGS, recurrence_inputs
from tests._util import norm_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {"f32": 1e-4, "bf16": 2e-2}


def _ssm():
    import selective_state_space_bwd_amd as ssm
    return ssm


def _dev(x, dt):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float32 if dt == "f32" else torch.bfloat16).to(DEV)


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


# batch, seqlen, channels, dtype: one step; one segment; ragged channel tiles and
# several segments; many segments of a long sequence; bf16 storage
SHAPES = [(1, 1, 1, "f32"), (2, 37, 70, "f32"), (3, 1000, 300, "f32"), (2, 4096, 64, "f32"),
          (2, 777, 520, "bf16")]


@pytest.mark.parametrize("exclusive", [False, True])
@pytest.mark.parametrize("decay", [None, "uniform", "ssm"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{s[0]}T{s[1]}C{s[2]}-{s[3]}" for s in SHAPES])
def test_reverse_linear_scan(shape, decay, exclusive):
    nb, T, C, dt = shape
    p = recurrence_inputs(nb, T, C, dt, seed=T + C, decay=decay)
    print(f"case: reverse_linear_scan B{nb} T{T} C{C} {dt} decay {decay} exclusive {exclusive}", flush=True)
    x = _ssm().reverse_linear_scan(None if p["a"] is None else _dev(p["a"], dt), _dev(p["b"], dt),
                                   exclusive=exclusive)
    torch.cuda.synchronize()
    ref = orc.reverse_linear_scan(p["a"], p["b"], exclusive)
    assert norm_err(_np(x), ref) < TOL[dt]


def test_deterministic():
    p = recurrence_inputs(2, 3000, 300, "f32", seed=3, decay="ssm")
    a, b = _dev(p["a"], "f32"), _dev(p["b"], "f32")
    print("case: reverse_linear_scan determinism B2 T3000 C300", flush=True)
    x1 = _ssm().reverse_linear_scan(a, b)
    x2 = _ssm().reverse_linear_scan(a, b)
    torch.cuda.synchronize()
    assert torch.equal(x1, x2)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("decay", [None, "ssm"])
def test_full_size_sampled(decay):
    """The bench's workload (B8 T2048 C2048 f32) in one call; the oracle recomputes 64 sampled channels."""
    c = CONFIGS["revscan"]
    p = recurrence_inputs(c.batch, c.seqlen, c.channels, c.dtype, seed=c.seed, decay=decay)
    print(f"case: {c.name} decay {decay}", flush=True)
    x = _ssm().reverse_linear_scan(None if p["a"] is None else _dev(p["a"], c.dtype), _dev(p["b"], c.dtype))
    torch.cuda.synchronize()
    ch = np.sort(np.random.default_rng(0).choice(c.channels, 64, replace=False))
    sub = {k: (None if v is None else np.ascontiguousarray(v[:, :, ch])) for k, v in p.items()}
    ref = orc.reverse_linear_scan(sub["a"], sub["b"])
    assert norm_err(_np(x)[:, :, ch], ref) < TOL[c.dtype]
