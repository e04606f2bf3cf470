"""Seeded input generators for the selective-scan workloads.

Recipe (the same for every consumer):
  * generator: NumPy PCG64, ``numpy.random.default_rng(seed)``;
  * scan workloads draw, in this order, u, delta_raw, B, C, z, d_out, each
    ``standard_normal`` in float64; delta = softplus(-2 + 0.5 * delta_raw) so that
    delta = softplus(N(-2, 0.5)); A_log[d, n] = log(n + 1) (the real S4D
    initialisation, A = -(n + 1)); D = 1;
  * every value is then rounded to its storage dtype: float64 -> float32
    (round to nearest even), and for bf16 storage float32 -> bf16 (round to
    nearest even).  Arrays are returned as float32 holding exactly the stored
    values, so ``torch.from_numpy(x).to(torch.bfloat16)`` is exact;
  * the full-layer workload draws x, d_out, then the random weights in the order
    W_in, conv_w, W_x, W_dt, W_out, each N(0, 0.02); biases are 0, the norm
    weight is 1, A_log and D as above.  The "perturbed" variant then draws
    conv_b, b_dt ~ N(0, 0.1) and norm_w = 1 + N(0, 0.1) so that a kernel that
    ignores a bias or the norm weight cannot pass.

Variants of the scan recipe (stress cases for the cross-chunk carries):
  * ``long_memory``: delta = softplus(N(-6, 0.5)) (about 0.0025), so a 64-step
    chunk keeps 0.85 (n = 0) down to 0.08 (n = 15) of its carry;
  * ``random_A``: A_log = N(0, 1) + log(n + 1), drawn after d_out;
  * ``last_chunk``: d_out is zero outside the last ``last_steps`` steps, so every
    earlier gradient arrives through the adjoint carry;
  * ``zero_delta``: delta = 0 exactly (the state stays zero).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def round_bf16(x) -> np.ndarray:
    """Round to bfloat16 (nearest even) via float32; returns float32 values."""
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = x32.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    nan = np.isnan(x32)
    out = rounded.view(np.float32).copy()
    if nan.any():
        out[nan] = np.nan
    return out


def round_storage(x, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


@dataclass(frozen=True)
class ScanConfig:
    name: str
    batch: int
    seqlen: int
    d_inner: int
    d_state: int
    dtype: str  # storage of the [B, T, *] tensors: "f32" or "bf16"
    seed: int

    @property
    def state_elements(self) -> int:
        return self.batch * self.seqlen * self.d_inner * self.d_state


@dataclass(frozen=True)
class LayerConfig:
    name: str
    batch: int
    seqlen: int
    d_model: int
    d_inner: int
    d_state: int
    dt_rank: int
    d_conv: int
    dtype: str
    seed: int
    eps: float = 1e-5

    @property
    def state_elements(self) -> int:
        return self.batch * self.seqlen * self.d_inner * self.d_state


@dataclass(frozen=True)
class BackboneConfig:
    name: str
    n_layers: int
    input_dim: int
    batch: int
    seqlen: int
    d_model: int
    d_inner: int
    d_state: int
    dt_rank: int
    d_conv: int
    dtype: str
    seed: int
    eps: float = 1e-5

    @property
    def state_elements(self) -> int:
        return self.n_layers * self.batch * self.seqlen * self.d_inner * self.d_state


@dataclass(frozen=True)
class RecurrenceConfig:
    name: str
    batch: int
    seqlen: int
    channels: int
    dtype: str
    seed: int

    @property
    def elements(self) -> int:
        return self.batch * self.seqlen * self.channels


CONFIGS = {
    "tiny": ScanConfig("tiny B1 T64 Di32 N8 f32", 1, 64, 32, 8, "f32", 0),
    "mamba130m": ScanConfig("mamba-130m-shaped B8 T1024 Di1536 N16 f32", 8, 1024, 1536, 16, "f32", 1),
    "mamba370m": ScanConfig("mamba-370m-shaped B8 T2048 Di2048 N16 f32", 8, 2048, 2048, 16, "f32", 2),
    "mamba2p8b": ScanConfig("mamba-2.8b-shaped B2 T8192 Di5120 N16 bf16", 2, 8192, 5120, 16, "bf16", 3),
    "layer": LayerConfig("full layer B8 T2048 dm1536 di3072 N16 r96 k4 bf16",
                         8, 2048, 1536, 3072, 16, 96, 4, "bf16", 4),
    "backbone": BackboneConfig("backbone L4 B8 T2048 in512 dm1536 di3072 N16 r96 k4 bf16",
                               4, 512, 8, 2048, 1536, 3072, 16, 96, 4, "bf16", 6),
    "revscan": RecurrenceConfig("reverse linear scan B8 T2048 C2048 f32", 8, 2048, 2048, "f32", 5),
}


def backbone_inputs(n_layers: int, input_dim: int, batch: int, seqlen: int, d_model: int, d_inner: int,
                    d_state: int, dt_rank: int, d_conv: int, dtype: str = "bf16", seed: int = 6,
                    weight_std: float = 0.02) -> tuple:
    """Inputs of one backbone backward call: (bp, layers).

    bp: the input embedding inp [B, T, input_dim] ~ N(0, 1) and d_out [B, T, d_model]
    ~ N(0, 1) (rounded to ``dtype``), the input projection W_ip [d_model, input_dim]
    ~ N(0, 1 / input_dim) (rounded to ``dtype``) with bias b_ip ~ N(0, 0.01) and the
    final norm weight norm_f_w = 1 (float32).  layers: one parameter dict per layer
    as ``layer_inputs`` draws them (seed 1000 seed + l), without its x and d_out.
    """
    rng = np.random.default_rng(seed)
    bp = {
        "inp": round_storage(rng.standard_normal((batch, seqlen, input_dim)), dtype),
        "W_ip": round_storage(rng.standard_normal((d_model, input_dim)) / np.sqrt(input_dim), dtype),
        "b_ip": (0.1 * rng.standard_normal(d_model)).astype(np.float32),
        "norm_f_w": np.ones(d_model, dtype=np.float32),
        "d_out": round_storage(rng.standard_normal((batch, seqlen, d_model)), dtype),
    }
    layers = []
    for l in range(n_layers):
        p = layer_inputs(1, 1, d_model, d_inner, d_state, dt_rank, d_conv, dtype, seed=1000 * seed + l,
                         weight_std=weight_std)
        layers.append({k: v for k, v in p.items() if k not in ("x", "d_out")})
    return bp, layers


def recurrence_inputs(batch: int, seqlen: int, channels: int, dtype: str = "f32", seed: int = 5,
                      decay: str | None = "ssm") -> dict:
    """b ~ N(0, 1) [B, T, C] and the decay a: None (a = 1, the cumsum backward),
    "uniform" (U(0.2, 1.0)) or "ssm" (exp(-delta) with delta = softplus(N(-2, 0.5)),
    the decay of one state of the mamba-370m-shaped scan inputs); rounded to ``dtype``."""
    rng = np.random.default_rng(seed)
    b = rng.standard_normal((batch, seqlen, channels))
    if decay is None:
        a = None
    elif decay == "uniform":
        a = rng.uniform(0.2, 1.0, (batch, seqlen, channels))
    elif decay == "ssm":
        a = np.exp(-_softplus(-2.0 + 0.5 * rng.standard_normal((batch, seqlen, channels))))
    else:
        raise ValueError(f"unknown decay {decay!r}")
    return {"a": None if a is None else round_storage(a, dtype), "b": round_storage(b, dtype)}


def scan_inputs(batch: int, seqlen: int, d_inner: int, d_state: int, dtype: str = "f32",
                seed: int = 0, variant: str = "default", last_steps: int = 64) -> dict:
    """Inputs of one selective-scan backward call, rounded to ``dtype`` storage.

    Returns float32 arrays u, delta, z, d_out [B, T, Di]; B, C [B, T, N];
    A_log [Di, N] and D [Di] (parameters are always float32).
    """
    rng = np.random.default_rng(seed)
    shp = (batch, seqlen, d_inner)
    shs = (batch, seqlen, d_state)
    u = rng.standard_normal(shp)
    draw = rng.standard_normal(shp)
    Bm = rng.standard_normal(shs)
    Cm = rng.standard_normal(shs)
    z = rng.standard_normal(shp)
    d_out = rng.standard_normal(shp)
    A_log = np.broadcast_to(np.log(np.arange(1, d_state + 1, dtype=np.float64)),
                            (d_inner, d_state)).copy()
    if variant == "long_memory":
        delta = _softplus(-6.0 + 0.5 * draw)
    elif variant == "zero_delta":
        delta = np.zeros(shp)
    else:
        delta = _softplus(-2.0 + 0.5 * draw)
    del draw
    if variant == "random_A":
        A_log = A_log + rng.standard_normal((d_inner, d_state))
    if variant == "last_chunk":
        d_out[:, : max(seqlen - last_steps, 0), :] = 0.0
    elif variant not in ("default", "long_memory", "zero_delta", "random_A"):
        raise ValueError(f"unknown variant {variant!r}")
    out = {
        "u": round_storage(u, dtype),
        "delta": round_storage(delta, dtype),
        "B": round_storage(Bm, dtype),
        "C": round_storage(Cm, dtype),
        "z": round_storage(z, dtype),
        "d_out": round_storage(d_out, dtype),
        "A_log": np.asarray(A_log, dtype=np.float32),
        "D": np.ones(d_inner, dtype=np.float32),
    }
    return out


def layer_inputs(batch: int, seqlen: int, d_model: int, d_inner: int, d_state: int,
                 dt_rank: int, d_conv: int, dtype: str = "bf16", seed: int = 4,
                 variant: str = "default", weight_std: float = 0.02) -> dict:
    """Inputs and parameters of one full-layer backward call.

    Activations x, d_out [B, T, d_model] are rounded to ``dtype``; matrices are
    stored [out_features, in_features] and rounded to ``dtype``; the conv
    weight is [d_inner, d_conv]; biases, the norm weight, A_log and D are float32.
    Weight matrices and the conv weight are N(0, weight_std).
    """
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((batch, seqlen, d_model))
    d_out = rng.standard_normal((batch, seqlen, d_model))
    w_in = weight_std * rng.standard_normal((2 * d_inner, d_model))
    conv_w = weight_std * rng.standard_normal((d_inner, d_conv))
    w_x = weight_std * rng.standard_normal((dt_rank + 2 * d_state, d_inner))
    w_dt = weight_std * rng.standard_normal((d_inner, dt_rank))
    w_out = weight_std * rng.standard_normal((d_model, d_inner))
    conv_b = np.zeros(d_inner)
    b_dt = np.zeros(d_inner)
    norm_w = np.ones(d_model)
    if variant == "perturbed":
        conv_b = 0.1 * rng.standard_normal(d_inner)
        b_dt = 0.1 * rng.standard_normal(d_inner)
        norm_w = 1.0 + 0.1 * rng.standard_normal(d_model)
    elif variant != "default":
        raise ValueError(f"unknown variant {variant!r}")
    A_log = np.broadcast_to(np.log(np.arange(1, d_state + 1, dtype=np.float64)),
                            (d_inner, d_state)).copy()
    return {
        "x": round_storage(x, dtype),
        "d_out": round_storage(d_out, dtype),
        "norm_w": np.asarray(norm_w, np.float32),
        "W_in": round_storage(w_in, dtype),
        "conv_w": round_storage(conv_w, dtype),
        "conv_b": np.asarray(conv_b, np.float32),
        "W_x": round_storage(w_x, dtype),
        "W_dt": round_storage(w_dt, dtype),
        "b_dt": np.asarray(b_dt, np.float32),
        "A_log": np.asarray(A_log, np.float32),
        "D": np.ones(d_inner, np.float32),
        "W_out": round_storage(w_out, dtype),
    }
