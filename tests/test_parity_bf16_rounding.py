"""bf16 stores round to nearest, ties to even, bit for bit.

Every kernel writes bf16 through one conversion (gfx950's v_cvt_pk_bf16_f32).
A matrix-core product with two nonzero terms per output, Y = a + b, is exact in
float32 when a and b are bf16 values whose exponents differ by at most 15, so
the only rounding is the store: Y must equal the nearest-even bf16 of the exact
sum.  The cases include exact ties (b = +-half a unit in a's last place), values
just above and below a tie, sign changes and random pairs; both the 16-byte
epilogue (N a multiple of 16) and the element-wise edge path (N = 8) are taken.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _rne_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 bit patterns of finite float32 values, written out: keep
    the upper 16 bits, add one unit when the dropped half is above 0x8000, or
    equal to it with an odd kept part."""
    bits = x32.view(np.uint32).astype(np.uint64)
    keep = bits >> 16
    drop = bits & 0xFFFF
    up = (drop > 0x8000) | ((drop == 0x8000) & ((keep & 1) == 1))
    return (keep + up.astype(np.uint64)).astype(np.uint16)


def _bf16_values(rng, n, lo_exp, hi_exp):
    """Random bf16 values (8 significant bits) with exponents in [lo_exp, hi_exp]."""
    mant = 128 + rng.integers(0, 128, n)  # 8-bit significand 1.xxxxxxx
    e = rng.integers(lo_exp, hi_exp + 1, n)
    sign = np.where(rng.random(n) < 0.5, -1.0, 1.0)
    return sign * mant.astype(np.float64) * np.exp2(e - 7.0)


def _pairs(seed, m):
    rng = np.random.default_rng(seed)
    a = _bf16_values(rng, m, -20, 20)
    ulp = np.exp2(np.floor(np.log2(np.abs(a))) - 7.0)  # a's last place in bf16
    kind = np.arange(m) % 6
    b = np.empty(m)
    b[kind == 0] = 0.5 * ulp[kind == 0]                       # exact tie, upward half
    b[kind == 1] = -0.5 * ulp[kind == 1]                      # exact tie, downward half
    b[kind == 2] = 0.5 * ulp[kind == 2] * (1 + 2.0 ** -7)     # just above a tie
    b[kind == 3] = -0.5 * ulp[kind == 3] * (1 - 2.0 ** -7)    # just short of a tie
    r = _bf16_values(rng, m, -20, 20)
    sh = rng.integers(0, 16, m)                               # exponent gap 0..15: sum exact in float32
    mag = np.exp2(np.floor(np.log2(np.abs(a))) - sh)
    b[kind >= 4] = (np.sign(r) * (np.abs(r) / np.exp2(np.floor(np.log2(np.abs(r))))) * mag)[kind >= 4]
    # every b is a bf16 value and a + b is exact in float32
    for v in (b,):
        v32 = v.astype(np.float32)
        assert np.array_equal(v32.astype(np.float64), v)
        assert np.array_equal((v32.view(np.uint32) & 0xFFFF), np.zeros(m, np.uint32))
    s = a + b
    assert np.array_equal(s.astype(np.float32).astype(np.float64), s)
    return a, b, s


@pytest.mark.parametrize("N", [8, 32])
def test_bf16_store_rounds_to_nearest_even(N):
    import selective_state_space_bwd_amd as ssm
    M, K = 3000, 8
    a, b, s = _pairs(7 + N, M)
    X = np.zeros((M, K), np.float32)
    X[:, 0], X[:, 1] = a, b
    # column n scales both terms by 2^(n % 5 - 2): exact, and moves the sum's exponent
    scale = np.exp2((np.arange(N) % 5) - 2.0).astype(np.float32)
    W = np.zeros((N, K), np.float32)
    W[:, 0] = scale
    W[:, 1] = scale
    Xt = torch.from_numpy(X).to(torch.bfloat16).to(DEV)
    Wt = torch.from_numpy(W).to(torch.bfloat16).to(DEV)
    assert np.array_equal(Xt.float().cpu().numpy(), X)  # inputs are exact bf16 values
    Y = ssm.linear_fwd(Xt, Wt)
    torch.cuda.synchronize()
    got = Y.view(torch.int16).cpu().numpy().view(np.uint16)
    exact = (s[:, None] * scale[None, :].astype(np.float64)).astype(np.float32)
    want = _rne_bf16_bits(np.ascontiguousarray(exact))
    bad = np.argwhere(got != want)
    assert bad.size == 0, (f"{len(bad)} of {got.size} outputs differ; first at {tuple(bad[0])}: "
                           f"got {got[tuple(bad[0])]:#06x} want {want[tuple(bad[0])]:#06x}")
