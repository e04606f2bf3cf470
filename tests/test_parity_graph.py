"""The backward entry points captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

An entry point only launches kernels on the caller's stream: it allocates
nothing, never synchronises with the host and clears memory with its own fill
kernels rather than memset nodes, so one stream capture records the whole call.
A replay must give the eager call's bits (the kernels use no atomics, so equal
inputs give equal bits).  Each graph is replayed three times with eager work
between the replays: new values copied into the captured inputs, the captured
outputs overwritten with NaN, and a host synchronisation; replay 1 and 3 take
input set 1, replay 2 input set 2, and every replay is compared bitwise with an
eager call on the same inputs.
"""
import numpy as np
import pytest
import torch

from synth import layer_inputs, scan_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _ssm():
    import selective_state_space_bwd_amd as ssm
    return ssm


def _dev(p, dtype, keep_f32=()):
    out = {}
    for k, v in p.items():
        t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
        out[k] = (t if k in keep_f32 else t.to(dtype)).to(DEV)
    return out


def _flat(res):
    """Tensors of a result (dict, tuple or tensor) in a fixed order."""
    if isinstance(res, dict):
        return [v for k in sorted(res) for v in _flat(res[k])]
    if isinstance(res, (tuple, list)):
        return [v for r in res for v in _flat(r)]
    return [res] if isinstance(res, torch.Tensor) else []


def _replay_matches_eager(run, static, inputs, label):
    """run(): the call on the tensors in `static` (dict of captured inputs);
    inputs: two dicts of input values with the keys of `static`."""
    def load(k):
        for name, t in static.items():
            t.copy_(inputs[k][name])

    want = []
    for k in (0, 1):
        load(k)
        want.append([t.clone() for t in _flat(run())])
    torch.cuda.synchronize()
    load(0)
    run()  # once more on the side of the capture, as torch advises
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = _flat(run())
    torch.cuda.synchronize()
    for rep, k in enumerate((0, 1, 0)):
        load(k)
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        print(f"case: {label} graph replay {rep} (input set {k})", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        assert len(outs) == len(want[k])
        for i, (got, ref) in enumerate(zip(outs, want[k])):
            assert torch.equal(got, ref), f"{label}: replay {rep}, output {i} differs from the eager call"
    del graph


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_scan_bwd_graph_replay(dt):
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    nb, T, di, N = 2, 300, 200, 16
    keys = ("u", "delta", "B", "C", "z", "d_out")
    sets = [_dev(scan_inputs(nb, T, di, N, dt, seed=s), tdt, keep_f32=("A_log", "D")) for s in (21, 22)]
    static = {k: sets[0][k].clone() for k in keys}
    par = {k: sets[0][k] for k in ("A_log", "D")}
    ws = torch.empty(_ssm().ssm_scan_bwd_workspace_size(_ssm().scan_dims(static["u"], static["B"], seg_len=32), tdt),
                     dtype=torch.uint8, device=DEV)

    def run():
        s = static
        return _ssm().ssm_scan_bwd(s["u"], s["delta"], par["A_log"], s["B"], s["C"], par["D"], s["z"], s["d_out"],
                                   seg_len=32, workspace=ws)

    _replay_matches_eager(run, static, [{k: p[k] for k in keys} for p in sets], f"ssm_scan_bwd {dt}")


def test_linear_bwd_graph_replay():
    """A split-k product (dX and dW in one launch, then the fixed-order reduce)."""
    M, K, N = 2048, 3072, 128
    rng = np.random.default_rng(4)
    mk = lambda *s, sc=1.0: torch.from_numpy((rng.standard_normal(s) * sc).astype(np.float32)).to(torch.bfloat16).to(DEV)
    W = mk(N, K, sc=0.02)
    sets = [{"X": mk(M, K), "dY": mk(M, N)} for _ in range(2)]
    static = {k: v.clone() for k, v in sets[0].items()}

    def run():
        return _ssm().linear_bwd(static["X"], W, static["dY"], need_db=True)

    _replay_matches_eager(run, static, sets, "linear_bwd")


def test_layer_bwd_graph_replay():
    Bt, T, dm, di, N, R, Kc = 2, 150, 64, 128, 16, 8, 4
    bf = ("x", "d_out", "W_in", "W_x", "W_dt", "W_out")
    sets = []
    for seed in (31, 32):
        p = layer_inputs(Bt, T, dm, di, N, R, Kc, "bf16", seed=seed, variant="perturbed",
                         weight_std=0.02 * np.sqrt(1536.0 / dm))
        sets.append({k: (torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
                         if k in bf else torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))).to(DEV)
                     for k, v in p.items()})
    wkeys = ("norm_w", "W_in", "conv_w", "conv_b", "W_x", "W_dt", "b_dt", "A_log", "D", "W_out")
    w = {k: sets[0][k] for k in wkeys}
    ssm = _ssm()
    # saved activations of each input set from the eager forward (same weights)
    saved = []
    for s in sets:
        _, sv = ssm.mamba_layer_fwd(s["x"], w)
        saved.append({k: v.clone() for k, v in sv.items()})
    torch.cuda.synchronize()
    skeys = tuple(saved[0])
    static = {"x": sets[0]["x"].clone(), "d_out": sets[0]["d_out"].clone()}
    static.update({"s_" + k: saved[0][k].clone() for k in skeys})
    inputs = [dict({"x": s["x"], "d_out": s["d_out"]}, **{"s_" + k: sv[k] for k in skeys})
              for s, sv in zip(sets, saved)]
    ws = torch.empty(ssm.mamba_layer_bwd_workspace_size(static["x"], w), dtype=torch.uint8, device=DEV)

    def run():
        sv = {k: static["s_" + k] for k in skeys}
        return ssm.mamba_layer_bwd(static["x"], w, sv, static["d_out"], workspace=ws)

    _replay_matches_eager(run, static, inputs, "mamba_layer_bwd")
