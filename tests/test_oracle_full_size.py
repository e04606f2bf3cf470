"""Pin of the oracle at the full sizes of the three scan workloads (CPU only).

Dot-product (adjoint) test: for a random direction v over every input of the
scan backward (u, delta, A_log, B, C, D, z), the oracle's gradient must give
<grad, v> equal to the central difference (L(x + eps v) - L(x - eps v)) / (2 eps)
of L = sum d_out * out computed by the oracle's forward, at the real shapes
(mamba-130m-, mamba-370m- and mamba-2.8b-shaped workloads, their seeded inputs).
A wrong transposed operand, sign or index anywhere in the backward shows up at
any size; this one checks it where element-wise finite differences cannot go.

Channels are independent apart from the sums over them (d_B, d_C, and L itself),
and batch elements are independent apart from the sums over them (d_A_log, d_D,
L), so every quantity splits into (batch element, 1024-channel block) shards
whose partial dot products and losses are added in shard order.  The shards run
in a fork pool of the host's cores.
"""
import multiprocessing as mp
import os

import numpy as np
import pytest

from oracle import ssm
from synth import CONFIGS, scan_inputs

BLOCK = 1024
EPS = 1e-5   # the difference error is the O(eps^2) truncation here (7e-9 relative on the mamba-130m shape)
KEYS = {"u": "d_u", "delta": "d_delta", "A_log": "d_A_log", "B": "d_B", "C": "d_C", "D": "d_D", "z": "d_z"}

_P = {}
_V = {}


def _init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def _slice(src, b, d0, d1, step=0.0):
    """Inputs of shard (b, channels d0:d1), moved by step * v."""
    q = {}
    for k, x in src.items():
        if k in ("u", "delta", "z", "d_out"):
            s = np.s_[b:b + 1, :, d0:d1]
        elif k in ("B", "C"):
            s = np.s_[b:b + 1]
        else:                      # A_log [Di, N], D [Di]
            s = np.s_[d0:d1]
        q[k] = x[s] + step * _V[k][s] if (step and k in _V) else x[s]
    return q


def _grad_dot(task):
    b, d0, d1 = task
    q = _slice(_P, b, d0, d1)
    g = ssm.ssm_scan_bwd(q["u"], q["delta"], q["A_log"], q["B"], q["C"], q["D"], q["z"], q["d_out"])
    v = _slice(_V, b, d0, d1)
    return float(sum(np.sum(g[gk] * v[k]) for k, gk in KEYS.items()))


def _loss(task):
    b, d0, d1, step = task
    q = _slice(_P, b, d0, d1, step)
    _, out = ssm.ssm_forward(q["u"], q["delta"], q["A_log"], q["B"], q["C"], q["D"], q["z"])
    return float(np.sum(out * q["d_out"]))


@pytest.mark.slow
@pytest.mark.timeout(1800)
@pytest.mark.parametrize("name", ["mamba130m", "mamba370m", "mamba2p8b"])
def test_dot_product_full_size(name):
    c = CONFIGS[name]
    p = scan_inputs(c.batch, c.seqlen, c.d_inner, c.d_state, c.dtype, c.seed)
    _P.clear()
    _P.update({k: v.astype(np.float64) for k, v in p.items()})
    del p
    rng = np.random.default_rng(1000 + c.seed)
    _V.clear()
    _V.update({k: rng.standard_normal(_P[k].shape) for k in KEYS})
    shards = [(b, d0, min(d0 + BLOCK, c.d_inner)) for b in range(c.batch) for d0 in range(0, c.d_inner, BLOCK)]
    workers = max(1, min(len(os.sched_getaffinity(0)), 16, len(shards)))
    with mp.get_context("fork").Pool(workers, initializer=_init) as pool:
        ana = sum(pool.map(_grad_dot, shards, chunksize=1))
        lp = pool.map(_loss, [s + (EPS,) for s in shards], chunksize=1)
        lm = pool.map(_loss, [s + (-EPS,) for s in shards], chunksize=1)
    num = sum(a - b for a, b in zip(lp, lm)) / (2 * EPS)
    _P.clear()
    _V.clear()
    rel = abs(ana - num) / abs(ana)
    print(f"{c.name}: <grad, v> = {ana:.10e}, central difference {num:.10e}, relative {rel:.2e}", flush=True)
    assert rel < 1e-7
