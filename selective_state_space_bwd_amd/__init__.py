"""Python binding of the gfx950 selective-scan backward library (``libssmbwd.so``).

Argument marshalling only: every function checks shapes, dtypes and strides,
allocates outputs and workspace with torch on the tensors' device, and calls the
C entry point of the same name on torch's current stream.  All arithmetic runs
in the HIP kernels.  There is no fallback: importing this package fails if the
library has not been built (``python -m selective_state_space_bwd_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssmbwd.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "ssmbwd.h")

_lib = None

SSM_OK, SSM_ERR_INVALID_ARG, SSM_ERR_UNSUPPORTED, SSM_ERR_WORKSPACE, SSM_ERR_LAUNCH = range(5)
SSM_F32, SSM_BF16 = 0, 1
SSM_BWD_SOFTPLUS, SSM_BWD_ACCUMULATE, SSM_BWD_ACCUMULATE_DX = 1, 2, 4


class ssm_dims(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in
                ("batch", "seqlen", "d_inner", "d_state", "ld_bc", "ld_dbc", "seg_len", "ld_z")]


class ssm_layer_dims(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in
                ("batch", "seqlen", "d_model", "d_inner", "d_state", "dt_rank", "d_conv", "seg_len")] + \
               [("eps", ctypes.c_float)]


LAYER_WEIGHTS = ("norm_w", "W_in", "conv_w", "conv_b", "W_x", "W_dt", "b_dt", "A_log", "D", "W_out")
LAYER_SAVED = ("xz", "xdbl", "delta", "y")
# optional: the inputs of the out_proj, x_proj and in_proj products (ssm_layer_saved's last fields)
LAYER_KEPT_INPUTS = ("gated", "u", "xn")
LAYER_GRADS = tuple("d_" + k for k in LAYER_WEIGHTS)  # same order as ssm_layer_grads


class ssm_layer_weights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in LAYER_WEIGHTS]


class ssm_layer_saved(ctypes.Structure):
    _fields_ = ([(name, ctypes.c_void_p) for name in LAYER_SAVED] + [("h_ckpt", ctypes.c_void_p)]
                + [(name, ctypes.c_void_p) for name in LAYER_KEPT_INPUTS])


def _saved_struct(saved: dict) -> ssm_layer_saved:
    return ssm_layer_saved(*[_ptr(saved.get(k)) for k in LAYER_SAVED], _ptr(saved.get("h_ckpt")),
                           *[_ptr(saved.get(k)) for k in LAYER_KEPT_INPUTS])


def _new_saved(B_, T_, dims, device, keep_gemm_inputs: bool) -> dict:
    """The saved activations a layer forward writes: {xz, xdbl, delta, y}, or with ``keep_gemm_inputs``
    {xz, xdbl, delta, gated, u, xn} (y is then not needed: only the gate recompute reads it)."""
    di, R2 = dims.d_inner, dims.dt_rank + 2 * dims.d_state
    e = lambda *shp: torch.empty(shp, dtype=torch.bfloat16, device=device)
    saved = {"xz": e(B_, T_, 2 * di), "xdbl": e(B_, T_, R2), "delta": e(B_, T_, di)}
    if keep_gemm_inputs:
        saved.update(gated=e(B_, T_, di), u=e(B_, T_, di), xn=e(B_, T_, dims.d_model))
    else:
        saved["y"] = e(B_, T_, di)
    return saved


def _scan_states(batch, seqlen, d_state, d_inner, device):
    """The scan's state before every 8-step chunk, [B, ceil(T / 8), N, Di] float32."""
    return torch.empty((batch, (seqlen + 7) // 8, d_state, d_inner), dtype=torch.float32, device=device)


class ssm_layer_grads(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in LAYER_GRADS] + [("accumulate", ctypes.c_int32)]


class ssm_backbone_dims(ctypes.Structure):
    _fields_ = [("layer", ssm_layer_dims), ("n_layers", ctypes.c_int32), ("input_dim", ctypes.c_int32),
                ("keep", ctypes.c_int32)]


SSM_KEEP_ALL, SSM_KEEP_INPUTS = 0, 1


_vp, _fp, _i, _i64, _sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
_dims_p = ctypes.POINTER(ssm_dims)

_SIGS = {
    "ssm_status_string": (ctypes.c_char_p, [_i]),
    "ssm_last_error": (ctypes.c_char_p, []),
    "ssm_scan_bwd_workspace_size": (_sz, [_dims_p, _i]),
    "ssm_scan_bwd": (_i, [_vp, _vp, _fp, _vp, _vp, _fp, _vp, _vp, _vp, _vp, _fp, _vp, _vp, _fp, _vp, _i,
                          _vp, _sz, _dims_p, _i, _vp]),
    "ssm_scan_bwd_timed": (_i, [_vp, _vp, _fp, _vp, _vp, _fp, _vp, _vp, _vp, _vp, _fp, _vp, _vp, _fp, _vp, _i,
                                _vp, _sz, _dims_p, _i, _vp, ctypes.POINTER(ctypes.c_void_p)]),
    "ssm_scan_bwd_ckpt_workspace_size": (_sz, [_dims_p, _i]),
    "ssm_scan_bwd_ckpt": (_i, [_vp, _vp, _fp, _vp, _vp, _fp, _vp, _vp, _fp, _vp, _vp, _fp, _vp, _vp, _fp, _vp, _i,
                               _vp, _sz, _dims_p, _i, _vp, ctypes.POINTER(ctypes.c_void_p)]),
    "ssm_scan_bwd_ckpt_noalloc_capacity": (_sz, []),
    "ssm_scan_bwd_ckpt_noalloc": (_i, [_vp, _vp, _fp, _vp, _vp, _fp, _vp, _vp, _fp, _vp, _vp, _fp, _vp, _vp, _fp,
                                       _vp, _i, _dims_p, _i, _vp]),
    "ssm_scan_fwd_workspace_size": (_sz, [_dims_p, _i]),
    "ssm_scan_fwd": (_i, [_vp, _vp, _fp, _vp, _vp, _fp, _vp, _vp, _vp, _fp, _i, _vp, _sz, _dims_p, _i, _vp]),
    "gating_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i64, _i, _vp]),
    "reverse_linear_scan_workspace_size": (_sz, [_i, _i, _i, _i]),
    "reverse_linear_scan": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _vp, _sz, _i, _vp]),
    "conv1d_bwd_workspace_size": (_sz, [_i, _i, _i, _i]),
    "conv1d_bwd": (_i, [_vp, _fp, _fp, _vp, _vp, _fp, _fp, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _i, _vp]),
    "rmsnorm_bwd_workspace_size": (_sz, [_i64, _i]),
    "rmsnorm_bwd": (_i, [_vp, _fp, _vp, _vp, _vp, _fp, _i64, _i, ctypes.c_float, _i, _vp, _sz, _i, _vp]),
    "linear_bwd_workspace_size": (_sz, [_i64, _i, _i]),
    "linear_bwd": (_i, [_vp, _i64, _vp, _vp, _i64, _vp, _i64, _i, _fp, _fp, _i64, _i, _i, _vp, _sz, _i, _vp]),
    "linear_fwd_workspace_size": (_sz, [_i64, _i, _i]),
    "mamba_layer_fwd_workspace_size": (_sz, [ctypes.POINTER(ssm_layer_dims)]),
    "mamba_layer_fwd": (_i, [_vp, ctypes.POINTER(ssm_layer_weights), _vp, ctypes.POINTER(ssm_layer_saved), _vp, _sz,
                             ctypes.POINTER(ssm_layer_dims), _vp]),
    "mamba_layer_bwd_workspace_size": (_sz, [ctypes.POINTER(ssm_layer_dims)]),
    "mamba_layer_bwd": (_i, [_vp, ctypes.POINTER(ssm_layer_weights), ctypes.POINTER(ssm_layer_saved), _vp, _vp,
                             ctypes.POINTER(ssm_layer_grads), _vp, _sz, ctypes.POINTER(ssm_layer_dims), _vp]),
    "mamba_layer_bwd_timed": (_i, [_vp, ctypes.POINTER(ssm_layer_weights), ctypes.POINTER(ssm_layer_saved), _vp, _vp,
                                   ctypes.POINTER(ssm_layer_grads), _vp, _sz, ctypes.POINTER(ssm_layer_dims), _vp,
                                   ctypes.POINTER(ctypes.c_void_p)]),
    "linear_fwd": (_i, [_vp, _i64, _vp, _fp, _vp, _i64, _i64, _i, _i, _vp, _sz, _i, _vp]),
    "mamba_backbone_fwd_workspace_size": (_sz, [ctypes.POINTER(ssm_backbone_dims)]),
    "mamba_backbone_fwd": (_i, [_vp, _vp, _fp, _fp, ctypes.POINTER(ssm_layer_weights), ctypes.POINTER(_vp),
                                ctypes.POINTER(ssm_layer_saved), _vp, _vp, _sz, ctypes.POINTER(ssm_backbone_dims),
                                _vp]),
    "mamba_backbone_bwd_workspace_size": (_sz, [ctypes.POINTER(ssm_backbone_dims)]),
    "mamba_backbone_bwd": (_i, [_vp, _vp, _fp, ctypes.POINTER(ssm_layer_weights), ctypes.POINTER(_vp),
                                ctypes.POINTER(ssm_layer_saved), _vp, _vp, ctypes.POINTER(ssm_layer_grads), _fp, _fp,
                                _fp, _i, _vp, _sz, ctypes.POINTER(ssm_backbone_dims), _vp]),
}


def lib():
    """The loaded library (loaded on first use; raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m selective_state_space_bwd_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(handle, name)
            f.restype = res
            f.argtypes = args
        _lib = handle
    return _lib


def header_symbols() -> list:
    """Function names the C header declares (used to check the library's exports)."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|size_t|int)\s+(\w+)\s*\(", text, re.M)))


class SsmError(RuntimeError):
    def __init__(self, where: str, status: int):
        self.status = status
        msg = lib().ssm_last_error().decode(errors="replace")
        super().__init__(f"{where}: {lib().ssm_status_string(status).decode()} ({status}): {msg}")


def _check(where: str, rc: int):
    if rc != SSM_OK:
        raise SsmError(where, rc)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SSM_F32
    if t.dtype == torch.bfloat16:
        return SSM_BF16
    raise TypeError(f"storage dtype {t.dtype} not supported (float32 or bfloat16)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _row_stride(x: torch.Tensor, batch: int, seqlen: int, n: int, name: str) -> int:
    """B / C may be [B, T, N] views into a wider row (e.g. the x_proj output)."""
    _need(x.dim() == 3 and tuple(x.shape) == (batch, seqlen, n), f"{name} must be [{batch}, {seqlen}, {n}]")
    if x.numel() == 0:
        return n
    _need(x.stride(2) == 1, f"{name} must be contiguous in its last dim")
    ld = x.stride(1) if seqlen > 1 else max(x.stride(1), n)
    _need(batch <= 1 or x.stride(0) == seqlen * ld, f"{name}: rows must be evenly strided")
    return ld


def _workspace(nbytes: int, device, workspace):
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        _need(workspace.device == device and workspace.numel() * workspace.element_size() >= nbytes,
              f"workspace needs {nbytes} bytes on {device}")
        return workspace, workspace.numel() * workspace.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def scan_dims(u, B, d_state=None, seg_len=0, ld_dbc=None) -> ssm_dims:
    batch, seqlen, d_inner = u.shape
    n = d_state if d_state is not None else B.shape[2]
    ld = _row_stride(B, batch, seqlen, n, "B")
    return ssm_dims(batch, seqlen, d_inner, n, ld, ld_dbc if ld_dbc is not None else n, seg_len, 0)


def ssm_scan_bwd_workspace_size(dims: ssm_dims, dtype: torch.dtype) -> int:
    return int(lib().ssm_scan_bwd_workspace_size(ctypes.byref(dims), SSM_F32 if dtype == torch.float32 else SSM_BF16))


def ssm_scan_bwd_ckpt_workspace_size(dims: ssm_dims, dtype: torch.dtype) -> int:
    return int(lib().ssm_scan_bwd_ckpt_workspace_size(ctypes.byref(dims),
                                                      SSM_F32 if dtype == torch.float32 else SSM_BF16))


def ssm_scan_bwd(u, delta, A_log, B, C, D, z, d_out, *, softplus_epilogue: bool = False, accumulate: bool = False,
                 seg_len: int = 0, out: dict | None = None, workspace: torch.Tensor | None = None,
                 stage_events=None) -> dict:
    """Backward of out = y * SiLU(z) through the selective scan; returns the seven gradients.

    ``out`` may supply any of the output tensors (d_B / d_C may be strided views into a
    wider row, as the layer's x_proj gradient).  ``accumulate`` adds d_A_log and d_D into
    ``out["d_A_log"]`` / ``out["d_D"]`` (SSM_BWD_ACCUMULATE).  See ``ssm_scan_bwd`` in include/ssmbwd.h.
    """
    return _scan_bwd(u, delta, A_log, B, C, D, z, d_out, None, _bwd_flags(softplus_epilogue, accumulate), seg_len,
                     out, workspace, stage_events)


def ssm_scan_bwd_ckpt(u, delta, A_log, B, C, D, z, d_out, h_ckpt, *, softplus_epilogue: bool = False,
                      accumulate: bool = False, seg_len: int = 0, out: dict | None = None,
                      workspace: torch.Tensor | None = None, stage_events=None) -> dict:
    """ssm_scan_bwd taking the forward's state before every 8-step chunk, h_ckpt
    [B, ceil(T / 8), N, Di] float32 (``ssm_scan_fwd(..., ckpt_every=8)["h_ckpt"]``)."""
    return _scan_bwd(u, delta, A_log, B, C, D, z, d_out, h_ckpt, _bwd_flags(softplus_epilogue, accumulate),
                     seg_len, out, workspace, stage_events)


def ssm_scan_bwd_ckpt_noalloc(u, delta, A_log, B, C, D, z, d_out, h_ckpt, *, softplus_epilogue: bool = False,
                              accumulate: bool = False, seg_len: int = 0, out: dict | None = None) -> dict:
    """ssm_scan_bwd_ckpt whose scratch is the library's static device array (no workspace
    argument; shapes needing more than ``ssm_scan_bwd_ckpt_noalloc_capacity()`` bytes are
    rejected).  Pass every output in ``out`` for a call that allocates nothing."""
    return _scan_bwd(u, delta, A_log, B, C, D, z, d_out, h_ckpt, _bwd_flags(softplus_epilogue, accumulate),
                     seg_len, out, None, None, noalloc=True)


def ssm_scan_bwd_ckpt_noalloc_capacity() -> int:
    return int(lib().ssm_scan_bwd_ckpt_noalloc_capacity())


def _bwd_flags(softplus_epilogue: bool = False, accumulate: bool = False) -> int:
    return (SSM_BWD_SOFTPLUS if softplus_epilogue else 0) | (SSM_BWD_ACCUMULATE if accumulate else 0)


def _scan_bwd(u, delta, A_log, B, C, D, z, d_out, h_ckpt, flags, seg_len, out, workspace,
              stage_events, noalloc: bool = False) -> dict:
    dt = _dtype_code(u)
    batch, seqlen, d_inner = u.shape
    n = A_log.shape[1]
    for name, t in (("delta", delta), ("d_out", d_out)):
        _need(t.shape == u.shape and t.dtype == u.dtype and t.is_contiguous(), f"{name} must match u")
    _need(z.dtype == u.dtype, "z must have u's dtype")
    ldz = _row_stride(z, batch, seqlen, d_inner, "z")
    _need(u.is_contiguous(), "u must be contiguous")
    _need(B.dtype == u.dtype and C.dtype == u.dtype, "B and C must have u's dtype")
    _need(A_log.dtype == torch.float32 and D.dtype == torch.float32, "A_log and D are float32")
    _need(A_log.shape == (d_inner, n) and A_log.is_contiguous() and D.shape == (d_inner,), "parameter shapes")
    ld = _row_stride(B, batch, seqlen, n, "B")
    _need(_row_stride(C, batch, seqlen, n, "C") == ld, "B and C must share a row stride")
    o = dict(out or {})
    dev = u.device
    for k in ("d_u", "d_delta"):
        o.setdefault(k, torch.empty_like(u))
    if "d_z" not in o:
        o["d_z"] = torch.empty((batch, seqlen, ldz), dtype=u.dtype, device=dev)[..., :d_inner]
    _need(_row_stride(o["d_z"], batch, seqlen, d_inner, "d_z") == ldz, "d_z must share z's row stride")
    o.setdefault("d_A_log", torch.empty_like(A_log))
    o.setdefault("d_D", torch.empty_like(D))
    o.setdefault("d_B", torch.empty((batch, seqlen, n), dtype=u.dtype, device=dev))
    o.setdefault("d_C", torch.empty((batch, seqlen, n), dtype=u.dtype, device=dev))
    ldd = _row_stride(o["d_B"], batch, seqlen, n, "d_B")
    _need(_row_stride(o["d_C"], batch, seqlen, n, "d_C") == ldd, "d_B and d_C must share a row stride")
    dims = ssm_dims(batch, seqlen, d_inner, n, ld, ldd, seg_len, ldz)
    ev = None
    if stage_events is not None:
        ev = (ctypes.c_void_p * 5)(*[ctypes.c_void_p(e) if e else None for e in stage_events])
    if h_ckpt is not None:
        nk = (seqlen + 7) // 8
        _need(h_ckpt.dtype == torch.float32 and tuple(h_ckpt.shape) == (batch, nk, n, d_inner)
              and h_ckpt.is_contiguous(), f"h_ckpt must be float32 [{batch}, {nk}, {n}, {d_inner}], contiguous")
        if noalloc:
            rc = lib().ssm_scan_bwd_ckpt_noalloc(_ptr(u), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D),
                                                 _ptr(z), _ptr(d_out), _ptr(h_ckpt), _ptr(o["d_u"]),
                                                 _ptr(o["d_delta"]), _ptr(o["d_A_log"]), _ptr(o["d_B"]),
                                                 _ptr(o["d_C"]), _ptr(o["d_D"]), _ptr(o["d_z"]), int(flags),
                                                 ctypes.byref(dims), dt, _stream(u))
            _check("ssm_scan_bwd_ckpt_noalloc", rc)
            return o
        nbytes = int(lib().ssm_scan_bwd_ckpt_workspace_size(ctypes.byref(dims), dt))
        ws, wsb = _workspace(nbytes, dev, workspace)
        rc = lib().ssm_scan_bwd_ckpt(_ptr(u), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                     _ptr(d_out), _ptr(h_ckpt), _ptr(o["d_u"]), _ptr(o["d_delta"]),
                                     _ptr(o["d_A_log"]), _ptr(o["d_B"]), _ptr(o["d_C"]), _ptr(o["d_D"]),
                                     _ptr(o["d_z"]), int(flags), _ptr(ws), wsb,
                                     ctypes.byref(dims), dt, _stream(u), ev)
        _check("ssm_scan_bwd_ckpt", rc)
        return o
    nbytes = int(lib().ssm_scan_bwd_workspace_size(ctypes.byref(dims), dt))
    ws, wsb = _workspace(nbytes, dev, workspace)
    args = (_ptr(u), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(d_out),
            _ptr(o["d_u"]), _ptr(o["d_delta"]), _ptr(o["d_A_log"]), _ptr(o["d_B"]),
            _ptr(o["d_C"]), _ptr(o["d_D"]), _ptr(o["d_z"]), int(flags),
            _ptr(ws), wsb, ctypes.byref(dims), dt, _stream(u))
    rc = lib().ssm_scan_bwd(*args) if ev is None else lib().ssm_scan_bwd_timed(*args, ev)
    _check("ssm_scan_bwd", rc)
    return o


def ssm_scan_fwd(u, delta, A_log, B, C, D, z=None, *, want_y: bool = True, want_out: bool = True,
                 ckpt_every: int = 0, seg_len: int = 0, workspace=None) -> dict:
    """Forward scan: y, out = y * SiLU(z) and optional state checkpoints [B, K, N, Di] (float32)."""
    dt = _dtype_code(u)
    batch, seqlen, d_inner = u.shape
    n = A_log.shape[1]
    _need(u.is_contiguous() and delta.shape == u.shape and delta.is_contiguous(), "u / delta")
    ld = _row_stride(B, batch, seqlen, n, "B")
    _need(_row_stride(C, batch, seqlen, n, "C") == ld, "B and C must share a row stride")
    res = {}
    y = torch.empty_like(u) if want_y else None
    o = torch.empty_like(u) if (want_out and z is not None) else None
    ck = None
    if ckpt_every:
        nk = (seqlen + ckpt_every - 1) // ckpt_every
        ck = torch.empty((batch, nk, n, d_inner), dtype=torch.float32, device=u.device)
    ldz = _row_stride(z, batch, seqlen, d_inner, "z") if z is not None else 0
    dims = ssm_dims(batch, seqlen, d_inner, n, ld, n, seg_len, ldz)
    nbytes = int(lib().ssm_scan_fwd_workspace_size(ctypes.byref(dims), dt))
    ws, wsb = _workspace(nbytes, u.device, workspace)
    rc = lib().ssm_scan_fwd(_ptr(u), _ptr(delta), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(y), _ptr(o),
                           _ptr(ck), int(ckpt_every), _ptr(ws), wsb, ctypes.byref(dims), dt, _stream(u))
    _check("ssm_scan_fwd", rc)
    if y is not None:
        res["y"] = y
    if o is not None:
        res["out"] = o
    if ck is not None:
        res["h_ckpt"] = ck
    return res


def reverse_linear_scan(a, b, *, exclusive: bool = False, x=None, workspace=None):
    """x_t = b_t + a_{t+1} x_{t+1} along t of [B, T, C] tensors (a None: a = 1, the cumsum
    backward); ``exclusive`` returns x_t - b_t.  See ``reverse_linear_scan`` in include/ssmbwd.h."""
    dt = _dtype_code(b)
    _need(b.dim() == 3 and b.is_contiguous(), "b must be a contiguous [B, T, C] tensor")
    if a is not None:
        _need(a.shape == b.shape and a.dtype == b.dtype and a.is_contiguous(), "a must match b")
    batch, seqlen, channels = b.shape
    if x is None:
        x = torch.empty_like(b)
    _need(x.shape == b.shape and x.dtype == b.dtype and x.is_contiguous(), "x must match b")
    nbytes = int(lib().reverse_linear_scan_workspace_size(batch, seqlen, channels, int(a is not None)))
    ws, wsb = _workspace(nbytes, b.device, workspace)
    _check("reverse_linear_scan", lib().reverse_linear_scan(_ptr(a), _ptr(b), _ptr(x), batch, seqlen, channels,
                                                           int(bool(exclusive)), _ptr(ws), wsb, dt, _stream(b)))
    return x


def gating_bwd(d_out, y, z):
    """Phase B2 on its own: returns (d_y, d_z)."""
    dt = _dtype_code(d_out)
    for t in (y, z):
        _need(t.shape == d_out.shape and t.dtype == d_out.dtype and t.is_contiguous(), "shapes/dtypes")
    _need(d_out.is_contiguous(), "d_out must be contiguous")
    d_y, d_z = torch.empty_like(d_out), torch.empty_like(d_out)
    _check("gating_bwd", lib().gating_bwd(_ptr(d_out), _ptr(y), _ptr(z), _ptr(d_y), _ptr(d_z), d_out.numel(), dt,
                                         _stream(d_out)))
    return d_y, d_z


def conv1d_bwd(x, w, bias, d_u, *, d_x=None, d_w=None, d_b=None, accumulate: bool = False, workspace=None):
    """Causal depthwise conv + SiLU backward; x and d_u are [B, T, Di] (last-dim contiguous rows).
    ``accumulate`` adds the weight and bias gradients into the given ``d_w`` / ``d_b``."""
    dt = _dtype_code(x)
    batch, seqlen, d_inner = x.shape
    d_conv = w.shape[1]
    _need(w.dtype == torch.float32 and w.shape == (d_inner, d_conv) and w.is_contiguous(), "w is [Di, K] float32")
    _need(bias is None or (bias.dtype == torch.float32 and bias.shape == (d_inner,)), "bias is [Di] float32")
    _need(d_u.shape == x.shape and d_u.dtype == x.dtype, "d_u must match x")
    ldx = _row_stride(x, batch, seqlen, d_inner, "x")
    ldu = _row_stride(d_u, batch, seqlen, d_inner, "d_u")
    if d_x is None:
        d_x = torch.empty((batch, seqlen, d_inner), dtype=x.dtype, device=x.device)
    ldo = _row_stride(d_x, batch, seqlen, d_inner, "d_x")
    _need(not accumulate or (d_w is not None and d_b is not None), "accumulate needs d_w and d_b")
    d_w = torch.empty_like(w) if d_w is None else d_w
    d_b = torch.empty((d_inner,), dtype=torch.float32, device=x.device) if d_b is None else d_b
    _need(d_w.shape == w.shape and d_w.dtype == torch.float32 and d_w.is_contiguous(), "d_w is [Di, K] float32")
    _need(d_b.shape == (d_inner,) and d_b.dtype == torch.float32, "d_b is [Di] float32")
    nbytes = int(lib().conv1d_bwd_workspace_size(batch, seqlen, d_inner, d_conv))
    ws, wsb = _workspace(nbytes, x.device, workspace)
    _check("conv1d_bwd", lib().conv1d_bwd(_ptr(x), _ptr(w), _ptr(bias), _ptr(d_u), _ptr(d_x), _ptr(d_w), _ptr(d_b),
                                         batch, seqlen, d_inner, d_conv, ldx, ldu, ldo,
                                         SSM_BWD_ACCUMULATE if accumulate else 0, _ptr(ws), wsb, dt, _stream(x)))
    return d_x, d_w, d_b


def rmsnorm_bwd(x, w, dy, d_residual=None, eps: float = 1e-5, *, dw=None, accumulate: bool = False,
                workspace=None):
    """RMSNorm (weight only) backward over the last dim, plus an optional residual gradient.
    ``accumulate`` adds the weight gradient into the given ``dw``."""
    dt = _dtype_code(x)
    dim = x.shape[-1]
    rows = x.numel() // dim if dim else 0
    _need(x.is_contiguous() and dy.is_contiguous() and dy.shape == x.shape and dy.dtype == x.dtype, "x / dy")
    _need(w.dtype == torch.float32 and w.shape == (dim,), "w is [dim] float32")
    if d_residual is not None:
        _need(d_residual.shape == x.shape and d_residual.dtype == x.dtype and d_residual.is_contiguous(), "residual")
    dx = torch.empty_like(x)
    _need(not accumulate or dw is not None, "accumulate needs dw")
    dw = torch.empty_like(w) if dw is None else dw
    _need(dw.shape == w.shape and dw.dtype == torch.float32, "dw is [dim] float32")
    nbytes = int(lib().rmsnorm_bwd_workspace_size(rows, dim))
    ws, wsb = _workspace(nbytes, x.device, workspace)
    _check("rmsnorm_bwd", lib().rmsnorm_bwd(_ptr(x), _ptr(w), _ptr(dy), _ptr(d_residual), _ptr(dx), _ptr(dw), rows,
                                           dim, ctypes.c_float(eps), SSM_BWD_ACCUMULATE if accumulate else 0,
                                           _ptr(ws), wsb, dt, _stream(x)))
    return dx, dw


def _matrix(x: torch.Tensor, name: str):
    """View [..., cols] bf16 with contiguous rows as a matrix: returns (rows, cols, row stride)."""
    _need(x.dtype == torch.bfloat16, f"{name} must be bfloat16")
    _need(x.dim() >= 2 and (x.stride(-1) == 1 or x.shape[-1] <= 1), f"{name} must have contiguous rows")
    cols = x.shape[-1]
    rows = 1
    for s_ in x.shape[:-1]:
        rows *= s_
    lead = [d_ for d_ in range(x.dim() - 1) if x.shape[d_] > 1]
    ld = x.stride(lead[-1]) if lead else cols
    step = ld
    for d_ in reversed(lead):  # leading dims must collapse onto rows of stride ld
        _need(x.stride(d_) == step, f"{name}: rows must be evenly strided")
        step *= x.shape[d_]
    return rows, cols, ld


def linear_bwd(X, W, dY, *, need_dx: bool = True, need_dw: bool = True, need_db: bool = False, dX=None,
               accumulate_dx: bool = False, dW=None, db=None, accumulate: bool = False, workspace=None):
    """Backward of Y = X W^T (+ b): returns (dX bf16, dW float32, db float32), None where not asked.

    X [..., K] and dY [..., N] may be views with strided rows (e.g. column slices of a wider
    activation); W is [N, K] contiguous bf16.  ``dX`` may be given (and is accumulated into
    when ``accumulate_dx``); so may ``dW`` and ``db`` (accumulated into when ``accumulate``).
    """
    N, K = W.shape
    _need(W.dtype == torch.bfloat16 and W.is_contiguous(), "W must be contiguous bf16 [N, K]")
    M, n2, lddy = _matrix(dY, "dY")
    _need(n2 == N, "dY's last dim must be W's rows")
    ldx = 0
    if need_dw:
        mx, k2, ldx = _matrix(X, "X")
        _need(mx == M and k2 == K, "X must be [M, K]")
    dev = dY.device
    lddx = 0
    if need_dx:
        if dX is None:
            _need(not accumulate_dx, "accumulate_dx needs dX")
            dX = torch.empty(tuple(dY.shape[:-1]) + (K,), dtype=torch.bfloat16, device=dev)
        mx, k2, lddx = _matrix(dX, "dX")
        _need(mx == M and k2 == K, "dX must be [M, K]")
    else:
        dX = None
    _need(not accumulate or ((dW is not None or not need_dw) and (db is not None or not need_db)),
          "accumulate needs the dW / db buffers")
    if need_dw:
        dW = torch.empty((N, K), dtype=torch.float32, device=dev) if dW is None else dW
        _need(dW.shape == (N, K) and dW.dtype == torch.float32 and dW.is_contiguous(), "dW must be float32 [N, K]")
    else:
        dW = None
    if need_db:
        db = torch.empty((N,), dtype=torch.float32, device=dev) if db is None else db
        _need(db.shape == (N,) and db.dtype == torch.float32 and db.is_contiguous(), "db must be float32 [N]")
    else:
        db = None
    flags = (SSM_BWD_ACCUMULATE_DX if accumulate_dx else 0) | (SSM_BWD_ACCUMULATE if accumulate else 0)
    nbytes = int(lib().linear_bwd_workspace_size(M, K, N))
    ws, wsb = _workspace(nbytes, dev, workspace)
    _check("linear_bwd", lib().linear_bwd(_ptr(X) if need_dw else None, ldx, _ptr(W), _ptr(dY), lddy, _ptr(dX),
                                         lddx, flags, _ptr(dW), _ptr(db), M, K, N, _ptr(ws), wsb,
                                         SSM_BF16, _stream(dY)))
    return dX, dW, db


def linear_fwd(X, W, *, Y=None, workspace=None):
    """Y = X W^T in bf16 (float accumulation); X [..., K] with contiguous rows, W [N, K]."""
    N, K = W.shape
    _need(W.dtype == torch.bfloat16 and W.is_contiguous(), "W must be contiguous bf16 [N, K]")
    M, k2, ldx = _matrix(X, "X")
    _need(k2 == K, "X's last dim must be W's columns")
    if Y is None:
        Y = torch.empty(tuple(X.shape[:-1]) + (N,), dtype=torch.bfloat16, device=X.device)
    my, n2, ldy = _matrix(Y, "Y")
    _need(my == M and n2 == N, "Y must be [M, N]")
    nbytes = int(lib().linear_fwd_workspace_size(M, K, N))
    ws, wsb = _workspace(nbytes, X.device, workspace)
    _check("linear_fwd", lib().linear_fwd(_ptr(X), ldx, _ptr(W), None, _ptr(Y), ldy, M, K, N, _ptr(ws), wsb,
                                         SSM_BF16, _stream(X)))
    return Y


# ---- the whole layer -------------------------------------------------------------
_LAYER_BF16 = ("W_in", "W_x", "W_dt", "W_out")


def layer_dims(x, weights: dict, *, eps: float = 1e-5, seg_len: int = 0) -> ssm_layer_dims:
    batch, seqlen, d_model = x.shape
    d_inner, d_state = weights["A_log"].shape
    return ssm_layer_dims(batch, seqlen, d_model, d_inner, d_state, weights["W_dt"].shape[1],
                          weights["conv_w"].shape[1], seg_len, eps)


def _layer_weights(weights: dict, dims: ssm_layer_dims):
    di, dm, R, N, K = dims.d_inner, dims.d_model, dims.dt_rank, dims.d_state, dims.d_conv
    shapes = {"norm_w": (dm,), "W_in": (2 * di, dm), "conv_w": (di, K), "conv_b": (di,), "W_x": (R + 2 * N, di),
              "W_dt": (di, R), "b_dt": (di,), "A_log": (di, N), "D": (di,), "W_out": (dm, di)}
    for k, shp in shapes.items():
        t = weights.get(k)
        if t is None and k in ("conv_b", "b_dt"):
            continue
        _need(t is not None and tuple(t.shape) == shp and t.is_contiguous(), f"{k} must be contiguous {shp}")
        _need(t.dtype == (torch.bfloat16 if k in _LAYER_BF16 else torch.float32),
              f"{k} must be {'bfloat16' if k in _LAYER_BF16 else 'float32'}")
    return ssm_layer_weights(*[ctypes.c_void_p(weights[k].data_ptr()) if weights.get(k) is not None else None
                               for k in LAYER_WEIGHTS])


def mamba_layer_fwd(x, weights: dict, *, eps: float = 1e-5, seg_len: int = 0, keep_scan_states: bool = False,
                    keep_gemm_inputs: bool = False, workspace=None):
    """Layer forward on bf16 activations: returns (out, saved) with saved = {xz, xdbl, delta, y}
    (and h_ckpt, the scan's chunk states, with ``keep_scan_states``: the backward then skips rebuilding them;
    with ``keep_gemm_inputs``, gated, u and xn in place of y: the backward then skips recomputing them)."""
    _need(x.dtype == torch.bfloat16 and x.dim() == 3 and x.is_contiguous(), "x must be contiguous bf16 [B, T, d_model]")
    dims = layer_dims(x, weights, eps=eps, seg_len=seg_len)
    w = _layer_weights(weights, dims)
    B_, T_, di = dims.batch, dims.seqlen, dims.d_inner
    saved = _new_saved(B_, T_, dims, x.device, keep_gemm_inputs)
    if keep_scan_states:
        saved["h_ckpt"] = _scan_states(B_, T_, dims.d_state, di, x.device)
    out = torch.empty_like(x)
    sv = _saved_struct(saved)
    nbytes = int(lib().mamba_layer_fwd_workspace_size(ctypes.byref(dims)))
    _need(nbytes > 0, "unsupported layer shape: " + (lib().ssm_last_error() or b"").decode())
    ws, wsb = _workspace(nbytes, x.device, workspace)
    _check("mamba_layer_fwd", lib().mamba_layer_fwd(_ptr(x), ctypes.byref(w), _ptr(out), ctypes.byref(sv), _ptr(ws),
                                                   wsb, ctypes.byref(dims), _stream(x)))
    return out, saved


def mamba_layer_bwd_workspace_size(x, weights: dict, **kw) -> int:
    return int(lib().mamba_layer_bwd_workspace_size(ctypes.byref(layer_dims(x, weights, **kw))))


def mamba_layer_bwd(x, weights: dict, saved: dict, d_out, *, eps: float = 1e-5, seg_len: int = 0, workspace=None,
                    out: dict | None = None, accumulate: bool = False, stage_events=None) -> dict:
    """Layer backward (Phases B1-B8): returns d_x (bf16) and every parameter gradient (float32).
    ``accumulate`` adds the parameter gradients into the buffers given in ``out``."""
    _need(x.dtype == torch.bfloat16 and x.dim() == 3 and x.is_contiguous(), "x must be contiguous bf16 [B, T, d_model]")
    _need(d_out.shape == x.shape and d_out.dtype == x.dtype and d_out.is_contiguous(), "d_out must match x")
    dims = layer_dims(x, weights, eps=eps, seg_len=seg_len)
    w = _layer_weights(weights, dims)
    _check_saved(saved, dims)
    sv = _saved_struct(saved)
    o = dict(out or {})
    _need(not accumulate or all(k in o for k in LAYER_GRADS), "accumulate needs every gradient buffer in out")
    o.setdefault("d_x", torch.empty_like(x))
    for k in LAYER_WEIGHTS:
        ref = weights.get(k)
        if ref is None:
            ref = weights["D"]
        o.setdefault("d_" + k, torch.empty(ref.shape, dtype=torch.float32, device=x.device))
    g = ssm_layer_grads(*[ctypes.c_void_p(o[k].data_ptr()) for k in LAYER_GRADS], int(bool(accumulate)))
    nbytes = int(lib().mamba_layer_bwd_workspace_size(ctypes.byref(dims)))
    _need(nbytes > 0, "unsupported layer shape: " + (lib().ssm_last_error() or b"").decode())
    ws, wsb = _workspace(nbytes, x.device, workspace)
    args = (_ptr(x), ctypes.byref(w), ctypes.byref(sv), _ptr(d_out), _ptr(o["d_x"]), ctypes.byref(g), _ptr(ws), wsb,
            ctypes.byref(dims), _stream(x))
    if stage_events is None:
        rc = lib().mamba_layer_bwd(*args)
    else:
        ev = (ctypes.c_void_p * 11)(*[ctypes.c_void_p(e) if e else None for e in stage_events])
        rc = lib().mamba_layer_bwd_timed(*args, ev)
    _check("mamba_layer_bwd", rc)
    return o


# ---------------------------------------------------------------------------
# backbone: input projection, the layers, final RMSNorm (mamba_backbone_* in include/ssmbwd.h)

def backbone_dims(inp, W_ip, layers: list, *, eps: float = 1e-5, seg_len: int = 0,
                  keep: str = "all") -> ssm_backbone_dims:
    """keep: "all" (every layer's saved activations, SSM_KEEP_ALL) or "inputs" (only the layer
    inputs, SSM_KEEP_INPUTS: the backward recomputes each layer's activations)."""
    batch, seqlen, input_dim = inp.shape
    _need(len(layers) >= 1, "at least one layer")
    _need(keep in ("all", "inputs"), 'keep is "all" or "inputs"')
    d_model = W_ip.shape[0]
    x_like = torch.empty((batch, seqlen, d_model), device="meta")
    return ssm_backbone_dims(layer_dims(x_like, layers[0], eps=eps, seg_len=seg_len), len(layers), input_dim,
                             SSM_KEEP_ALL if keep == "all" else SSM_KEEP_INPUTS)


def _check_saved(saved: dict, dims: ssm_layer_dims):
    """Shapes of a layer's saved activations: xz, xdbl, delta always; y unless gated is kept; gated, u, xn
    and h_ckpt when present."""
    B_, T_, di, R2 = dims.batch, dims.seqlen, dims.d_inner, dims.dt_rank + 2 * dims.d_state
    want = {"xz": (B_, T_, 2 * di), "xdbl": (B_, T_, R2), "delta": (B_, T_, di), "y": (B_, T_, di),
            "gated": (B_, T_, di), "u": (B_, T_, di), "xn": (B_, T_, dims.d_model)}
    _need(saved.get("y") is not None or saved.get("gated") is not None, "saved needs y or gated")
    for k, shp in want.items():
        t = saved.get(k)
        if t is None:
            _need(k not in ("xz", "xdbl", "delta"), f"saved {k} is required")
            continue
        _need(tuple(t.shape) == shp and t.dtype == torch.bfloat16 and t.is_contiguous(), f"saved {k} must be {shp}")
    _check_scan_states(saved, dims)


def _check_scan_states(saved: dict, dims: ssm_layer_dims):
    h = saved.get("h_ckpt")
    if h is not None:
        shp = (dims.batch, (dims.seqlen + 7) // 8, dims.d_state, dims.d_inner)
        _need(tuple(h.shape) == shp and h.dtype == torch.float32 and h.is_contiguous(),
              f"saved h_ckpt must be float32 {shp}")


def _backbone_arrays(bd, layers, xs, saved):
    L = bd.n_layers
    W = (ssm_layer_weights * L)(*[_layer_weights(p, bd.layer) for p in layers])
    X = (ctypes.c_void_p * (L + 1))(*[ctypes.c_void_p(x.data_ptr()) for x in xs])
    if saved is None:
        return W, X, None
    for sv in saved:
        _check_saved(sv, bd.layer)
    S = (ssm_layer_saved * L)(*[_saved_struct(sv) for sv in saved])
    return W, X, S


def mamba_backbone_fwd(inp, W_ip, b_ip, norm_f_w, layers: list, *, eps: float = 1e-5, seg_len: int = 0,
                       keep: str = "all", keep_scan_states: bool = False, keep_gemm_inputs: bool = False,
                       workspace=None):
    """Backbone forward on bf16 activations: returns (out, kept) with kept = {"xs": [n_layers + 1 tensors],
    "saved": [per-layer {xz, xdbl, delta, y}] (None with keep="inputs"), "keep": keep}, what the backward reads.
    ``keep_scan_states`` and ``keep_gemm_inputs`` add to every layer's saved set as in mamba_layer_fwd."""
    _need(inp.dtype == torch.bfloat16 and inp.dim() == 3 and inp.is_contiguous(), "inp must be contiguous bf16")
    _need(W_ip.dtype == torch.bfloat16 and W_ip.is_contiguous() and W_ip.shape[1] == inp.shape[2], "W_ip [d_model, in]")
    _need(keep == "all" or not (keep_scan_states or keep_gemm_inputs),
          "scan states and product inputs are kept only with keep=\"all\"")
    bd = backbone_dims(inp, W_ip, layers, eps=eps, seg_len=seg_len, keep=keep)
    d = bd.layer
    dev = inp.device
    B_, T_, dm, di = d.batch, d.seqlen, d.d_model, d.d_inner
    xs = [torch.empty((B_, T_, dm), dtype=torch.bfloat16, device=dev) for _ in range(bd.n_layers + 1)]
    saved = [_new_saved(B_, T_, d, dev, keep_gemm_inputs) for _ in range(bd.n_layers)]
    if keep_scan_states:
        for sv in saved:
            sv["h_ckpt"] = _scan_states(B_, T_, d.d_state, di, dev)
    if keep == "inputs":
        saved = None
    out = torch.empty((B_, T_, dm), dtype=torch.bfloat16, device=dev)
    W, X, S = _backbone_arrays(bd, layers, xs, saved)
    nbytes = int(lib().mamba_backbone_fwd_workspace_size(ctypes.byref(bd)))
    _need(nbytes > 0, "unsupported backbone shape: " + (lib().ssm_last_error() or b"").decode())
    ws, wsb = _workspace(nbytes, dev, workspace)
    _check("mamba_backbone_fwd", lib().mamba_backbone_fwd(_ptr(inp), _ptr(W_ip), _ptr(b_ip), _ptr(norm_f_w), W, X, S,
                                                         _ptr(out), _ptr(ws), wsb, ctypes.byref(bd), _stream(inp)))
    return out, {"xs": xs, "saved": saved, "keep": keep}


def mamba_backbone_fwd_workspace_size(inp, W_ip, layers: list, **kw) -> int:
    return int(lib().mamba_backbone_fwd_workspace_size(ctypes.byref(backbone_dims(inp, W_ip, layers, **kw))))


def mamba_backbone_bwd_workspace_size(inp, W_ip, layers: list, **kw) -> int:
    return int(lib().mamba_backbone_bwd_workspace_size(ctypes.byref(backbone_dims(inp, W_ip, layers, **kw))))


def mamba_backbone_bwd(inp, W_ip, norm_f_w, layers: list, kept: dict, d_out, *, need_d_inp: bool = False,
                       accumulate: bool = False, out: dict | None = None, eps: float = 1e-5, seg_len: int = 0,
                       workspace=None) -> dict:
    """Backbone backward: returns {"d_W_ip", "d_b_ip", "d_norm_f_w", "layers": [per-layer gradient dicts]}
    (and "d_inp" if asked).  ``accumulate`` adds every parameter gradient into the buffers given in ``out``.
    ``kept`` as mamba_backbone_fwd returns it (its "keep" plan decides whether the layers' activations are
    read or recomputed)."""
    bd = backbone_dims(inp, W_ip, layers, eps=eps, seg_len=seg_len, keep=kept.get("keep", "all"))
    d = bd.layer
    dev = inp.device
    _need(d_out.dtype == torch.bfloat16 and d_out.is_contiguous() and tuple(d_out.shape) == (d.batch, d.seqlen,
                                                                                             d.d_model), "d_out")
    o = dict(out or {})
    if accumulate:
        _need(all(k in o for k in ("d_W_ip", "d_b_ip", "d_norm_f_w", "layers")), "accumulate needs the buffers in out")
    o.setdefault("d_W_ip", torch.empty(W_ip.shape, dtype=torch.float32, device=dev))
    o.setdefault("d_b_ip", torch.empty((d.d_model,), dtype=torch.float32, device=dev))
    o.setdefault("d_norm_f_w", torch.empty((d.d_model,), dtype=torch.float32, device=dev))
    if "layers" not in o:
        o["layers"] = [{"d_" + k: torch.empty((p[k] if p.get(k) is not None else p["D"]).shape, dtype=torch.float32,
                                              device=dev) for k in LAYER_WEIGHTS} for p in layers]
    if need_d_inp:
        o.setdefault("d_inp", torch.empty_like(inp))
    W, X, S = _backbone_arrays(bd, layers, kept["xs"], kept["saved"])
    G = (ssm_layer_grads * bd.n_layers)(*[ssm_layer_grads(*[ctypes.c_void_p(g[k].data_ptr()) for k in LAYER_GRADS], 0)
                                          for g in o["layers"]])
    nbytes = int(lib().mamba_backbone_bwd_workspace_size(ctypes.byref(bd)))
    _need(nbytes > 0, "unsupported backbone shape: " + (lib().ssm_last_error() or b"").decode())
    ws, wsb = _workspace(nbytes, dev, workspace)
    _check("mamba_backbone_bwd", lib().mamba_backbone_bwd(
        _ptr(inp), _ptr(W_ip), _ptr(norm_f_w), W, X, S, _ptr(d_out), _ptr(o.get("d_inp")), G, _ptr(o["d_W_ip"]),
        _ptr(o["d_b_ip"]), _ptr(o["d_norm_f_w"]), SSM_BWD_ACCUMULATE if accumulate else 0, _ptr(ws), wsb,
        ctypes.byref(bd), _stream(inp)))
    return o
