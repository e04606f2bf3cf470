"""GPU parity of linear_bwd / linear_fwd (bf16 matrix-core GEMMs) against the fp64 oracle.

Tolerances follow from the arithmetic: inputs are bf16 values (exact in both
paths), products accumulate in float32, so dW and db (float outputs) agree to
~1e-6 of their scale; dX and Y are rounded to bf16 once, a relative error of at
most 2^-9 of the element, so their max error over the tensor's max stays under
4e-3 (1e-2 is asserted, with float accumulation on top).
"""
import numpy as np
import pytest
import torch

from oracle import layer as orc
from synth import round_bf16
from tests._util import norm_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_F32 = 1e-4
TOL_BF16 = 1e-2


def _ssm():
    import selective_state_space_bwd_amd as ssm
    return ssm


def _bf(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).to(DEV)


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def _mats(M, K, N, seed, x_cols=None, dy_cols=None):
    """bf16-valued X [M, x_cols >= K], W [N, K] (scale 0.02), dY [M, dy_cols >= N]."""
    rng = np.random.default_rng(seed)
    X = round_bf16(rng.standard_normal((M, x_cols or K)))
    W = round_bf16(rng.standard_normal((N, K)) * 0.02)
    dY = round_bf16(rng.standard_normal((M, dy_cols or N)))
    return X, W, dY


# (M, K, N): ragged in every dim, k not a multiple of the 32-wide k tile, split-k
# on skinny outputs (dt_proj / x_proj shapes), a single row and a single column tile
SHAPES = [
    (300, 72, 200),
    (1, 8, 8),
    (129, 40, 264),
    (2048, 96, 3072),   # dt_proj: dX [M, 96] and dW [3072, 96] split over M
    (2048, 3072, 128),  # x_proj:  dX [M, 3072], dW [128, 3072] split over M
    (777, 1536, 640),
]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_linear_bwd(M, K, N):
    X, W, dY = _mats(M, K, N, seed=M + 7 * K + 13 * N)
    print(f"case: linear_bwd M {M} K {K} N {N}", flush=True)
    dX, dW, db = _ssm().linear_bwd(_bf(X), _bf(W), _bf(dY), need_db=True)
    torch.cuda.synchronize()
    rx, rw, rb = orc.linear_bwd(X, W, dY)
    assert norm_err(_np(dX), rx) < TOL_BF16
    assert norm_err(_np(dW), rw) < TOL_F32
    assert norm_err(_np(db), rb) < TOL_F32


def test_linear_bwd_strided_views_and_accumulate():
    """X and dY as column slices of wider rows (dt_in inside the x_proj output), dX added
    into an existing buffer that is itself a slice (d_dt_in inside d_xdbl)."""
    M, K, N = 1000, 96, 1024
    X, W, dY = _mats(M, K, N, seed=5, x_cols=128, dy_cols=1536)
    base = round_bf16(np.random.default_rng(6).standard_normal((M, 128)))
    print("case: linear_bwd strided views + accumulate", flush=True)
    Xg, dYg = _bf(X)[:, :K], _bf(dY)[:, 256:256 + N]
    dXbuf = _bf(base)
    dX, dW, db = _ssm().linear_bwd(Xg, _bf(W), dYg, need_db=True, dX=dXbuf[:, 16:16 + K], accumulate_dx=True)
    torch.cuda.synchronize()
    rx, rw, rb = orc.linear_bwd(X[:, :K], W, dY[:, 256:256 + N])
    got = _np(dXbuf)
    assert norm_err(got[:, 16:16 + K], base[:, 16:16 + K] + rx) < TOL_BF16
    assert np.array_equal(got[:, :16], base[:, :16]) and np.array_equal(got[:, 16 + K:], base[:, 16 + K:])
    assert norm_err(_np(dW), rw) < TOL_F32
    assert norm_err(_np(db), rb) < TOL_F32


def test_linear_bwd_3d_and_skips():
    """[B, T, *] activations; dX only, then dW only."""
    Bt, T, K, N = 2, 300, 64, 136
    X, W, dY = _mats(Bt * T, K, N, seed=11)
    Xg, dYg = _bf(X).view(Bt, T, K), _bf(dY).view(Bt, T, N)
    print("case: linear_bwd 3-d, dX only / dW only", flush=True)
    dX, dW, db = _ssm().linear_bwd(None, _bf(W), dYg, need_dw=False)
    assert dW is None and db is None and dX.shape == (Bt, T, K)
    dX2, dW2, _ = _ssm().linear_bwd(Xg, _bf(W), dYg, need_dx=False)
    torch.cuda.synchronize()
    assert dX2 is None
    rx, rw, _ = orc.linear_bwd(X, W, dY)
    assert norm_err(_np(dX).reshape(-1, K), rx) < TOL_BF16
    assert norm_err(_np(dW2), rw) < TOL_F32


@pytest.mark.parametrize("M,K,N", [(777, 1536, 640), (2048, 3072, 128), (4096, 1536, 6144)])
def test_paired_launch_matches_single_products(M, K, N):
    """dX and dW requested together run as one launch (and dW's k split is chosen
    for the pair).  dX alone may take a k split that the paired dX does not, so
    the two differ only in the float summation order before the one bf16
    rounding: at most one bf16 step apart, 2^-8 of the tensor's largest value.  dW matches the
    dW-only call to float rounding (its split may differ)."""
    X, W, dY = _mats(M, K, N, seed=11 + M)
    print(f"case: paired linear_bwd M {M} K {K} N {N}", flush=True)
    Xg, Wg, dYg = _bf(X), _bf(W), _bf(dY)
    dX, dW, _ = _ssm().linear_bwd(Xg, Wg, dYg)
    dX1, _, _ = _ssm().linear_bwd(None, Wg, dYg, need_dw=False)
    _, dW1, _ = _ssm().linear_bwd(Xg, Wg, dYg, need_dx=False)
    torch.cuda.synchronize()
    rx, rw, _ = orc.linear_bwd(X, W, dY)
    a, b = _np(dX), _np(dX1)
    print(f"  dX vs oracle {norm_err(a, rx):.1e} / {norm_err(b, rx):.1e}, paired vs alone {norm_err(a, b):.1e}")
    assert norm_err(a, rx) < TOL_BF16 and norm_err(b, rx) < TOL_BF16
    assert norm_err(a, b) <= 2.0 ** -8 + 1e-6
    assert norm_err(_np(dW), _np(dW1)) < 1e-6
    assert norm_err(_np(dW), rw) < TOL_F32


@pytest.mark.parametrize("M,K,N,offset", [(1024, 512, 768, 128), (512, 256, 4096, 128), (1024, 512, 768, 4)])
def test_whole_tile_products_accumulate_into_views(M, K, N, offset):
    """Shapes made of whole 256 x 256 tiles and 64-wide k steps (the big-tile kernels: dX
    and dW paired, dW split over M), with dX added into a column slice of a wider buffer
    and dW / db accumulated into given buffers.  A slice starting 4 elements in takes no
    16-byte vectors, so dX then goes to the smaller tiles."""
    X, W, dY = _mats(M, K, N, seed=M + K + N + offset)
    rng = np.random.default_rng(offset)
    base = round_bf16(rng.standard_normal((M, K + 256)))
    w0 = rng.standard_normal((N, K)).astype(np.float32)
    b0 = rng.standard_normal(N).astype(np.float32)
    print(f"case: whole-tile linear_bwd M {M} K {K} N {N} dX offset {offset}", flush=True)
    dXbuf = _bf(base)
    dWg = torch.from_numpy(w0).to(DEV)
    dbg = torch.from_numpy(b0).to(DEV)
    _ssm().linear_bwd(_bf(X), _bf(W), _bf(dY), need_db=True, dX=dXbuf[:, offset:offset + K], accumulate_dx=True,
                      dW=dWg, db=dbg, accumulate=True)
    torch.cuda.synchronize()
    rx, rw, rb = orc.linear_bwd(X, W, dY)
    got = _np(dXbuf)
    assert norm_err(got[:, offset:offset + K], base[:, offset:offset + K] + rx) < TOL_BF16
    assert np.array_equal(got[:, :offset], base[:, :offset])
    assert np.array_equal(got[:, offset + K:], base[:, offset + K:])
    assert norm_err(_np(dWg), w0 + rw) < TOL_F32
    assert norm_err(_np(dbg), b0 + rb) < TOL_F32
    Y = _ssm().linear_fwd(_bf(X), _bf(W))
    torch.cuda.synchronize()
    assert norm_err(_np(Y), orc.linear_fwd(X, W)) < TOL_BF16


# (M, K, N): a narrow input K (at most 128) against whole 256-row tiles in M and N
# takes the paired 256 x 128 tiles (dX and dW split over k, db as dW's extra
# column when K < 128); a narrow output N (at most 128) against whole tiles in M
# and K takes dW's transpose on 256 x 128 tiles beside dX on 256 x 256 tiles.
NARROW = [
    (256, 96, 256, True),      # narrow input, one row tile, db in the product
    (1024, 64, 768, True),
    (4096, 128, 512, True),    # K = 128: no room for the bias column, db summed apart
    (2048, 96, 3072, False),   # dt_proj's shape, no db
    (2048, 512, 128, False),   # narrow output (x_proj's shape at fewer rows)
    (1024, 768, 64, False),
    (2048, 512, 96, True),     # narrow output ending inside the 128-wide tile
]


@pytest.mark.parametrize("M,K,N,need_db", NARROW)
def test_narrow_products_accumulate(M, K, N, need_db):
    """dX added into a column slice of a wider buffer, dW and db accumulated into given buffers."""
    X, W, dY = _mats(M, K, N, seed=7 * M + K + 3 * N)
    rng = np.random.default_rng(K + N)
    base = round_bf16(rng.standard_normal((M, K + 128)))
    w0 = rng.standard_normal((N, K)).astype(np.float32)
    b0 = rng.standard_normal(N).astype(np.float32)
    print(f"case: narrow linear_bwd M {M} K {K} N {N} db {need_db}", flush=True)
    dXbuf = _bf(base)
    dWg = torch.from_numpy(w0).to(DEV)
    dbg = torch.from_numpy(b0).to(DEV) if need_db else None
    _ssm().linear_bwd(_bf(X), _bf(W), _bf(dY), need_db=need_db, dX=dXbuf[:, 64:64 + K], accumulate_dx=True,
                      dW=dWg, db=dbg, accumulate=True)
    torch.cuda.synchronize()
    rx, rw, rb = orc.linear_bwd(X, W, dY)
    got = _np(dXbuf)
    assert norm_err(got[:, 64:64 + K], base[:, 64:64 + K] + rx) < TOL_BF16
    assert np.array_equal(got[:, :64], base[:, :64]) and np.array_equal(got[:, 64 + K:], base[:, 64 + K:])
    assert norm_err(_np(dWg), w0 + rw) < TOL_F32
    if need_db:
        assert norm_err(_np(dbg), b0 + rb) < TOL_F32
    # and written fresh, without accumulation
    dX2, dW2, db2 = _ssm().linear_bwd(_bf(X), _bf(W), _bf(dY), need_db=need_db)
    torch.cuda.synchronize()
    assert norm_err(_np(dX2), rx) < TOL_BF16
    assert norm_err(_np(dW2), rw) < TOL_F32
    if need_db:
        assert norm_err(_np(db2), rb) < TOL_F32


def test_linear_bwd_empty_rows():
    """M = 0: dW and db are zero (sums over no rows)."""
    W = _bf(np.ones((24, 16)))
    X = torch.empty((0, 16), dtype=torch.bfloat16, device=DEV)
    dY = torch.empty((0, 24), dtype=torch.bfloat16, device=DEV)
    print("case: linear_bwd M 0", flush=True)
    dX, dW, db = _ssm().linear_bwd(X, W, dY, need_db=True)
    torch.cuda.synchronize()
    assert dX.shape == (0, 16)
    assert torch.count_nonzero(dW).item() == 0 and torch.count_nonzero(db).item() == 0


@pytest.mark.parametrize("M,K,N", [(300, 72, 200), (2048, 1536, 6144), (1000, 3072, 128)])
def test_linear_fwd(M, K, N):
    X, W, _ = _mats(M, K, N, seed=3 * M + K)
    print(f"case: linear_fwd M {M} K {K} N {N}", flush=True)
    Y = _ssm().linear_fwd(_bf(X), _bf(W))
    torch.cuda.synchronize()
    assert norm_err(_np(Y), orc.linear_fwd(X, W)) < TOL_BF16


# rows of dX checked at the layer's size: the last nine 256-row tiles in full
# (the blocks the paired launch hands out last) plus a random sample of the
# others
def _full_size_rows(M, n_random, seed=0):
    rng = np.random.default_rng(seed)
    return np.union1d(rng.choice(M - 2304, n_random, replace=False), np.arange(M - 2304, M))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("which", ["in_proj", "out_proj"])
def test_linear_bwd_full_layer_sampled(which):
    """The layer's two large GEMMs at full size (16384 rows), checked on sampled
    rows of dX and sampled columns of dW, each computed by the oracle on its own."""
    M = 8 * 2048
    K, N = (1536, 6144) if which == "in_proj" else (3072, 1536)
    X, W, dY = _mats(M, K, N, seed=K + N)
    print(f"case: linear_bwd full-size {which} M {M} K {K} N {N}", flush=True)
    dX, dW, db = _ssm().linear_bwd(_bf(X), _bf(W), _bf(dY), need_db=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = _full_size_rows(M, 64)
    cols = np.sort(rng.choice(K, 16, replace=False))
    rx, _, _ = orc.linear_bwd(X[rows], W, dY[rows])
    _, rw, rb = orc.linear_bwd(X[:, cols], W[:, cols], dY)
    assert norm_err(_np(dX[rows]), rx) < TOL_BF16
    assert norm_err(_np(dW[:, cols]), rw) < TOL_F32
    assert norm_err(_np(db), rb) < TOL_F32


@pytest.mark.timeout(600)
def test_linear_bwd_full_layer_accumulate_dx():
    """in_proj at full size with dX added into a column slice of a wider buffer
    and dW accumulated: every checked row adds to its old values, and the
    columns outside the slice keep theirs."""
    M, K, N = 8 * 2048, 1536, 6144
    X, W, dY = _mats(M, K, N, seed=77)
    rng = np.random.default_rng(7)
    base = round_bf16(rng.standard_normal((M, K + 256)))
    w0 = rng.standard_normal((N, K)).astype(np.float32)
    print(f"case: linear_bwd full-size in_proj M {M} K {K} N {N}, dX accumulated into a view", flush=True)
    dXbuf = _bf(base)
    dWg = torch.from_numpy(w0).to(DEV)
    _ssm().linear_bwd(_bf(X), _bf(W), _bf(dY), dX=dXbuf[:, 128:128 + K], accumulate_dx=True, dW=dWg,
                      accumulate=True)
    torch.cuda.synchronize()
    rows = _full_size_rows(M, 32, seed=1)
    cols = np.sort(rng.choice(K, 8, replace=False))
    rx, _, _ = orc.linear_bwd(X[rows], W, dY[rows])
    _, rw, _ = orc.linear_bwd(X[:, cols], W[:, cols], dY)
    got = _np(dXbuf)[rows]
    assert norm_err(got[:, 128:128 + K], base[rows, 128:128 + K] + rx) < TOL_BF16
    assert np.array_equal(got[:, :128], base[rows, :128])
    assert np.array_equal(got[:, 128 + K:], base[rows, 128 + K:])
    assert norm_err(_np(dWg)[:, cols], w0[:, cols] + rw) < TOL_F32
