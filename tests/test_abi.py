"""The C ABI as seen from the host, without a GPU: the library loads, exports
every symbol the header declares, and rejects bad arguments before launching."""
import ctypes

import pytest

ssm = pytest.importorskip("selective_state_space_bwd_amd")
L = ssm.lib()
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def test_exports_every_header_symbol():
    syms = ssm.header_symbols()
    assert {"ssm_scan_bwd", "ssm_scan_fwd", "gating_bwd", "conv1d_bwd", "rmsnorm_bwd"} <= set(syms)
    for s in syms:
        assert hasattr(L, s), s


def test_status_strings():
    assert L.ssm_status_string(0) == b"ok"
    for code in range(1, 5):
        assert L.ssm_status_string(code) not in (b"ok", b"unknown status")
    assert L.ssm_status_string(99) == b"unknown status"


def _dims(**kw):
    d = dict(batch=2, seqlen=64, d_inner=32, d_state=16, ld_bc=16, ld_dbc=16, seg_len=0, ld_z=0)
    d.update(kw)
    return ssm.ssm_dims(**d)


def _bwd(dims, ws_bytes=1 << 40, dtype=0, ws=FAKE, **ptrs):
    p = [ptrs.get(k, FAKE) for k in ("u", "delta", "A_log", "B", "C", "D", "z", "d_out", "d_u", "d_delta",
                                    "d_A_log", "d_B", "d_C", "d_D", "d_z")]
    return L.ssm_scan_bwd(*p, 0, ws, ws_bytes, ctypes.byref(dims) if dims is not None else None, dtype, None)


def test_workspace_size():
    assert L.ssm_scan_bwd_workspace_size(ctypes.byref(_dims()), 0) > 0
    assert L.ssm_scan_bwd_workspace_size(ctypes.byref(_dims(d_state=5)), 0) == 0
    assert L.ssm_scan_bwd_workspace_size(None, 0) == 0
    small = L.ssm_scan_bwd_workspace_size(ctypes.byref(_dims(seqlen=64)), 0)
    big = L.ssm_scan_bwd_workspace_size(ctypes.byref(_dims(seqlen=4096)), 0)
    assert big > small


@pytest.mark.parametrize("kw,code", [
    (dict(d_state=5), ssm.SSM_ERR_UNSUPPORTED),
    (dict(d_state=32), ssm.SSM_ERR_UNSUPPORTED),
    (dict(batch=-1), ssm.SSM_ERR_INVALID_ARG),
    (dict(d_inner=0), ssm.SSM_ERR_INVALID_ARG),
    (dict(seg_len=12), ssm.SSM_ERR_INVALID_ARG),
    (dict(ld_bc=8), ssm.SSM_ERR_INVALID_ARG),
    (dict(ld_z=16), ssm.SSM_ERR_INVALID_ARG),
    (dict(seqlen=1 << 20, ld_z=1 << 12), ssm.SSM_ERR_UNSUPPORTED),
])
def test_bwd_rejects_bad_dims(kw, code):
    assert _bwd(_dims(**kw)) == code
    assert L.ssm_last_error()


def test_bwd_rejects_null_and_workspace():
    assert _bwd(None) == ssm.SSM_ERR_INVALID_ARG
    assert _bwd(_dims(), u=None) == ssm.SSM_ERR_INVALID_ARG
    assert _bwd(_dims(), ws_bytes=16) == ssm.SSM_ERR_WORKSPACE
    assert _bwd(_dims(), ws=None) == ssm.SSM_ERR_WORKSPACE
    assert _bwd(_dims(), dtype=7) == ssm.SSM_ERR_INVALID_ARG
    # bf16 rows must have even strides
    assert _bwd(_dims(ld_bc=17), dtype=1) == ssm.SSM_ERR_UNSUPPORTED


def _bwd_ckpt(dims, h_ckpt=FAKE, ws_bytes=1 << 40, dtype=0, ws=FAKE):
    p = [FAKE] * 8 + [h_ckpt] + [FAKE] * 7
    return L.ssm_scan_bwd_ckpt(*p, 0, ws, ws_bytes, ctypes.byref(dims) if dims is not None else None, dtype, None,
                               None)


def test_bwd_ckpt_validates():
    d = _dims(seqlen=4096, seg_len=256)
    full = L.ssm_scan_bwd_workspace_size(ctypes.byref(d), 0)
    given = L.ssm_scan_bwd_ckpt_workspace_size(ctypes.byref(d), 0)
    assert 0 < given < full   # no local checkpoints or forward carries
    assert L.ssm_scan_bwd_ckpt_workspace_size(ctypes.byref(_dims(d_state=5)), 0) == 0
    assert _bwd_ckpt(_dims(), h_ckpt=None) == ssm.SSM_ERR_INVALID_ARG
    assert _bwd_ckpt(None) == ssm.SSM_ERR_INVALID_ARG
    assert _bwd_ckpt(_dims(seg_len=12)) == ssm.SSM_ERR_INVALID_ARG
    assert _bwd_ckpt(_dims(), ws_bytes=16) == ssm.SSM_ERR_WORKSPACE


MISALIGNED = ctypes.c_void_p(0x1000 + 64)  # 64-byte aligned, not 256


def test_workspace_must_be_256_byte_aligned():
    assert _bwd(_dims(), ws=MISALIGNED) == ssm.SSM_ERR_WORKSPACE
    assert _bwd_ckpt(_dims(), ws=MISALIGNED) == ssm.SSM_ERR_WORKSPACE
    assert L.ssm_scan_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, 0, MISALIGNED, 1 << 40,
                          ctypes.byref(_dims()), 0, None) == ssm.SSM_ERR_WORKSPACE
    assert L.reverse_linear_scan(FAKE, FAKE, FAKE, 2, 4096, 64, 0, MISALIGNED, 1 << 30, 0,
                                 None) == ssm.SSM_ERR_WORKSPACE
    assert L.conv1d_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 4, 4, 4, 4, 4, 0, MISALIGNED, 1 << 30, 0,
                        None) == ssm.SSM_ERR_WORKSPACE
    assert L.rmsnorm_bwd(FAKE, FAKE, FAKE, None, FAKE, FAKE, 4, 64, ctypes.c_float(1e-5), 0, MISALIGNED, 1 << 30,
                         0, None) == ssm.SSM_ERR_WORKSPACE
    # split-k product (dt_proj shape): its partial sums need the aligned workspace
    assert L.linear_bwd(FAKE, 96, FAKE, FAKE, 3072, None, 0, 0, FAKE, None, 16384, 96, 3072, MISALIGNED, 1 << 40,
                        1, None) == ssm.SSM_ERR_WORKSPACE
    assert L.ssm_status_string(ssm.SSM_ERR_WORKSPACE).decode().endswith("misaligned")


def test_other_entry_points_validate():
    assert L.gating_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 0, None) == ssm.SSM_ERR_INVALID_ARG
    assert L.gating_bwd(None, FAKE, FAKE, FAKE, FAKE, 10, 0, None) == ssm.SSM_ERR_INVALID_ARG
    assert L.gating_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, None) == ssm.SSM_OK   # nothing to do
    assert L.conv1d_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 4, 9, 4, 4, 4, 0, FAKE, 1 << 30, 0,
                        None) == ssm.SSM_ERR_UNSUPPORTED
    assert L.conv1d_bwd_workspace_size(1, 8, 4, 9) == 0
    assert L.rmsnorm_bwd(FAKE, FAKE, FAKE, None, FAKE, FAKE, 4, 8192, ctypes.c_float(1e-5), 0, FAKE, 1 << 30, 0,
                         None) == ssm.SSM_ERR_UNSUPPORTED
    assert L.rmsnorm_bwd(FAKE, FAKE, FAKE, None, FAKE, FAKE, 4, 64, ctypes.c_float(-1.0), 0, FAKE, 1 << 30, 0,
                         None) == ssm.SSM_ERR_INVALID_ARG
    dims = _dims()
    assert L.ssm_scan_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, 0, FAKE, 1 << 40,
                          ctypes.byref(dims), 0, None) == ssm.SSM_ERR_INVALID_ARG   # out needs z
    assert L.ssm_scan_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 12, FAKE, 1 << 40,
                          ctypes.byref(dims), 0, None) == ssm.SSM_ERR_INVALID_ARG   # ckpt_every % 8


def test_unknown_flags_are_rejected():
    p = [FAKE] * 15
    d = _dims()
    assert L.ssm_scan_bwd(*p, 8, FAKE, 1 << 40, ctypes.byref(d), 0, None) == ssm.SSM_ERR_INVALID_ARG
    assert L.ssm_scan_bwd(*p, 0x100, FAKE, 1 << 40, ctypes.byref(d), 0, None) == ssm.SSM_ERR_INVALID_ARG
    assert L.conv1d_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 4, 4, 4, 4, 4, 1, FAKE, 1 << 30, 0,
                        None) == ssm.SSM_ERR_INVALID_ARG
    assert L.rmsnorm_bwd(FAKE, FAKE, FAKE, None, FAKE, FAKE, 4, 64, ctypes.c_float(1e-5), 4, FAKE, 1 << 30, 0,
                         None) == ssm.SSM_ERR_INVALID_ARG
    assert L.linear_bwd(FAKE, 64, FAKE, FAKE, 64, FAKE, 64, 1, FAKE, FAKE, 16, 64, 64, FAKE, 1 << 40, 1,
                        None) == ssm.SSM_ERR_INVALID_ARG
    # accumulating over an empty batch leaves the parameter gradients alone: nothing is launched
    e = _dims(batch=0)
    assert L.ssm_scan_bwd(*p, ssm.SSM_BWD_ACCUMULATE, None, 0, ctypes.byref(e), 0, None) == ssm.SSM_OK
    assert L.conv1d_bwd(None, FAKE, None, None, None, FAKE, FAKE, 0, 8, 4, 4, 4, 4, 4, ssm.SSM_BWD_ACCUMULATE, None, 0,
                        0, None) == ssm.SSM_OK
    assert L.rmsnorm_bwd(None, FAKE, None, None, None, FAKE, 0, 64, ctypes.c_float(1e-5), ssm.SSM_BWD_ACCUMULATE,
                         None, 0, 0, None) == ssm.SSM_OK
    assert L.linear_bwd(None, 64, FAKE, None, 64, None, 64, ssm.SSM_BWD_ACCUMULATE, FAKE, FAKE, 0, 64, 64, None, 0,
                        1, None) == ssm.SSM_OK


def test_reverse_linear_scan_validates():
    assert L.reverse_linear_scan(FAKE, FAKE, FAKE, 2, 64, 32, 0, FAKE, 1 << 30, 5, None) == ssm.SSM_ERR_INVALID_ARG
    assert L.reverse_linear_scan(FAKE, None, FAKE, 2, 64, 32, 0, FAKE, 1 << 30, 0, None) == ssm.SSM_ERR_INVALID_ARG
    assert L.reverse_linear_scan(FAKE, FAKE, FAKE, -1, 64, 32, 0, FAKE, 1 << 30, 0, None) == ssm.SSM_ERR_INVALID_ARG
    assert L.reverse_linear_scan(None, None, None, 0, 64, 32, 0, None, 0, 0, None) == ssm.SSM_OK   # nothing to do
    need = L.reverse_linear_scan_workspace_size(2, 4096, 64, 1)
    assert need > L.reverse_linear_scan_workspace_size(2, 4096, 64, 0) > 0   # decay products need their own half
    assert L.reverse_linear_scan(FAKE, FAKE, FAKE, 2, 4096, 64, 0, FAKE, need - 1, 0, None) == ssm.SSM_ERR_WORKSPACE
    assert L.reverse_linear_scan_workspace_size(1, 16, 8, 1) == 0   # one segment
    # batch is a grid dimension; one carry thread per (batch, channel)
    assert L.reverse_linear_scan(FAKE, FAKE, FAKE, 70000, 2, 8, 0, FAKE, 1 << 30, 0, None) == ssm.SSM_ERR_INVALID_ARG
    assert L.reverse_linear_scan(FAKE, FAKE, FAKE, 4, 2, 1 << 29, 0, FAKE, 1 << 62, 0, None) == ssm.SSM_ERR_INVALID_ARG


def test_backbone_entry_points_validate():
    lay = ssm.ssm_layer_dims(2, 64, 64, 128, 16, 8, 4, 0, 1e-5)
    ok = ssm.ssm_backbone_dims(lay, 2, 32)
    assert L.mamba_backbone_bwd_workspace_size(ctypes.byref(ok)) > L.mamba_layer_bwd_workspace_size(ctypes.byref(lay))
    assert L.mamba_backbone_fwd_workspace_size(ctypes.byref(ssm.ssm_backbone_dims(lay, 0, 32))) == 0    # no layers
    assert L.mamba_backbone_fwd_workspace_size(ctypes.byref(ssm.ssm_backbone_dims(lay, 2, 30))) == 0    # input_dim % 8
    assert L.mamba_backbone_fwd_workspace_size(ctypes.byref(ssm.ssm_backbone_dims(lay, 2, 32, 5))) == 0  # keep plan
    # keeping only the layer inputs: one layer's activations move into the workspaces
    inputs = ssm.ssm_backbone_dims(lay, 2, 32, ssm.SSM_KEEP_INPUTS)
    assert L.mamba_backbone_bwd_workspace_size(ctypes.byref(inputs)) > L.mamba_backbone_bwd_workspace_size(ctypes.byref(ok))
    assert L.mamba_backbone_fwd_workspace_size(ctypes.byref(inputs)) > L.mamba_backbone_fwd_workspace_size(ctypes.byref(ok))
    # null layer arrays are rejected before anything is launched
    assert L.mamba_backbone_bwd(FAKE, FAKE, FAKE, None, None, None, FAKE, None, None, FAKE, FAKE, FAKE, 0, FAKE,
                                1 << 40, ctypes.byref(ok), None) == ssm.SSM_ERR_INVALID_ARG
    assert L.mamba_backbone_fwd(FAKE, FAKE, None, FAKE, None, None, None, FAKE, FAKE, 1 << 40, ctypes.byref(ok),
                                None) == ssm.SSM_ERR_INVALID_ARG


def test_linear_entry_points_validate():
    ok_ws = 1 << 40
    # bf16 only
    assert L.linear_bwd(FAKE, 64, FAKE, FAKE, 64, FAKE, 64, 0, FAKE, FAKE, 16, 64, 64, FAKE, ok_ws, 0,
                        None) == ssm.SSM_ERR_UNSUPPORTED
    # negative rows, strides below the row length, null W
    assert L.linear_bwd(FAKE, 64, FAKE, FAKE, 64, FAKE, 64, 0, FAKE, FAKE, -1, 64, 64, FAKE, ok_ws, 1,
                        None) == ssm.SSM_ERR_INVALID_ARG
    assert L.linear_bwd(FAKE, 32, FAKE, FAKE, 64, FAKE, 64, 0, FAKE, FAKE, 16, 64, 64, FAKE, ok_ws, 1,
                        None) == ssm.SSM_ERR_INVALID_ARG
    assert L.linear_bwd(FAKE, 64, None, FAKE, 64, FAKE, 64, 0, FAKE, FAKE, 16, 64, 64, FAKE, ok_ws, 1,
                        None) == ssm.SSM_ERR_INVALID_ARG
    # row strides that break 16-byte rows
    assert L.linear_bwd(FAKE, 68, FAKE, FAKE, 64, FAKE, 64, 0, FAKE, None, 16, 64, 64, FAKE, ok_ws, 1,
                        None) == ssm.SSM_ERR_UNSUPPORTED
    # split-k needs its workspace
    assert L.linear_bwd_workspace_size(16384, 96, 3072) > 0
    assert L.linear_bwd(FAKE, 96, FAKE, FAKE, 3072, None, 0, 0, FAKE, None, 16384, 96, 3072, None, 0, 1,
                        None) == ssm.SSM_ERR_WORKSPACE
    assert L.linear_fwd(FAKE, 64, FAKE, FAKE, FAKE, 64, 16, 64, 64, None, 0, 1, None) == ssm.SSM_ERR_UNSUPPORTED


def _layer_dims(**kw):
    d = dict(batch=8, seqlen=2048, d_model=1536, d_inner=3072, d_state=16, dt_rank=96, d_conv=4, seg_len=0, eps=1e-5)
    d.update(kw)
    return ssm.ssm_layer_dims(**d)


def test_layer_entry_points_validate():
    big = L.mamba_layer_bwd_workspace_size(ctypes.byref(_layer_dims()))
    assert big > L.mamba_layer_bwd_workspace_size(ctypes.byref(_layer_dims(seqlen=64))) > 0
    assert L.mamba_layer_fwd_workspace_size(ctypes.byref(_layer_dims())) > 0
    for bad in (dict(d_state=32), dict(dt_rank=90), dict(d_conv=9), dict(d_model=8192)):
        assert L.mamba_layer_bwd_workspace_size(ctypes.byref(_layer_dims(**bad))) == 0
    w = ssm.ssm_layer_weights(*([FAKE.value] * 10))
    sv = ssm.ssm_layer_saved(*([FAKE.value] * 4))
    g = ssm.ssm_layer_grads(*([FAKE.value] * 10))

    def bwd(dims, w=w, sv=sv, g=g, ws_bytes=big, x=FAKE):
        return L.mamba_layer_bwd(x, ctypes.byref(w), ctypes.byref(sv), FAKE, FAKE, ctypes.byref(g), FAKE, ws_bytes,
                                 ctypes.byref(dims) if dims is not None else None, None)
    assert bwd(None) == ssm.SSM_ERR_INVALID_ARG
    assert bwd(_layer_dims(d_state=5)) == ssm.SSM_ERR_UNSUPPORTED
    assert bwd(_layer_dims(batch=0)) == ssm.SSM_ERR_INVALID_ARG
    assert bwd(_layer_dims(eps=-1.0)) == ssm.SSM_ERR_INVALID_ARG
    assert bwd(_layer_dims(), ws_bytes=1024) == ssm.SSM_ERR_WORKSPACE
    assert bwd(_layer_dims(), x=ctypes.c_void_p(0x1002)) == ssm.SSM_ERR_INVALID_ARG   # misaligned x
    assert bwd(_layer_dims(), w=ssm.ssm_layer_weights(*([FAKE.value] * 9 + [None]))) == ssm.SSM_ERR_INVALID_ARG
    assert bwd(_layer_dims(), g=ssm.ssm_layer_grads(*([None] + [FAKE.value] * 9))) == ssm.SSM_ERR_INVALID_ARG
    # the scan's checks run with the layer's, before any stage launches
    assert bwd(_layer_dims(seg_len=12)) == ssm.SSM_ERR_INVALID_ARG
    assert bwd(_layer_dims(seqlen=1 << 20, d_inner=4096)) == ssm.SSM_ERR_UNSUPPORTED   # rows past 2^32 elements
    misaligned = ssm.ssm_layer_saved(FAKE.value, 0x1008, FAKE.value, FAKE.value)
    assert bwd(_layer_dims(), sv=misaligned) == ssm.SSM_ERR_UNSUPPORTED
    # y may be null only when the gate's output is kept; kept inputs are alignment-checked too
    assert bwd(_layer_dims(), sv=ssm.ssm_layer_saved(FAKE.value, FAKE.value, FAKE.value, None)) == ssm.SSM_ERR_INVALID_ARG
    kept = ssm.ssm_layer_saved(FAKE.value, FAKE.value, FAKE.value, None, None, FAKE.value, FAKE.value, FAKE.value)
    assert bwd(_layer_dims(), sv=kept, ws_bytes=1024) == ssm.SSM_ERR_WORKSPACE   # saved accepted, workspace not
    kept_bad = ssm.ssm_layer_saved(FAKE.value, FAKE.value, FAKE.value, None, None, FAKE.value, 0x1004, FAKE.value)
    assert bwd(_layer_dims(), sv=kept_bad) == ssm.SSM_ERR_UNSUPPORTED
    assert L.mamba_layer_fwd(FAKE, ctypes.byref(w), FAKE, ctypes.byref(sv), FAKE, 16, ctypes.byref(_layer_dims()),
                             None) == ssm.SSM_ERR_WORKSPACE


def test_layer_bad_segment_length_leaves_accumulated_gradients_alone():
    """A segment length the scan rejects fails the whole layer call before its first stage: with
    accumulate set, d_W_out (here host memory, which no launch could reach) keeps its contents."""
    import numpy as np
    buf = np.full(64, 7.0, np.float32)
    w = ssm.ssm_layer_weights(*([FAKE.value] * 10))
    sv = ssm.ssm_layer_saved(*([FAKE.value] * 4))
    g = ssm.ssm_layer_grads(*([FAKE.value] * 9 + [buf.ctypes.data]), 1)
    dims = _layer_dims(seg_len=20)
    big = L.mamba_layer_bwd_workspace_size(ctypes.byref(_layer_dims()))
    rc = L.mamba_layer_bwd(FAKE, ctypes.byref(w), ctypes.byref(sv), FAKE, FAKE, ctypes.byref(g), FAKE, big,
                           ctypes.byref(dims), None)
    assert rc == ssm.SSM_ERR_INVALID_ARG
    assert "seg_len" in L.ssm_last_error().decode()
    assert np.all(buf == 7.0)
    assert L.mamba_layer_fwd(FAKE, ctypes.byref(w), FAKE, ctypes.byref(sv), FAKE, big, ctypes.byref(dims),
                             None) == ssm.SSM_ERR_INVALID_ARG


def test_binding_has_no_cpu_path():
    """The Python functions only marshal: without a GPU they fail instead of computing."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    x = torch.zeros(1, 8, 4)
    with pytest.raises(Exception):
        ssm.ssm_scan_bwd(x, x, torch.zeros(4, 4), torch.zeros(1, 8, 4), torch.zeros(1, 8, 4), torch.ones(4), x, x)
