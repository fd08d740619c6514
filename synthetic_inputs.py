"""Seeded synthetic inputs for the Gated DeltaNet workloads.

This module is shared by the tests, the smoke check and the benchmark. It holds
no step of the token mixer itself: it only draws random numbers and shapes them
into the input distributions of the five workloads. Two distribution recipes
need a transform of the draws, and both are applied here in float64 only to
define the inputs of the core kernels (they never stand in for the front-end
kernel or for the oracle's front end):

* q and k of the core-only workloads are "L2-normalised Gaussians": Gaussian
  draws divided by their norm (a uniform direction on the sphere).
* g of the core-only workloads is the log-decay "-exp(A_log) * softplus(a +
  dt_bias)" with A_log ~ U(0, 2.7) per V head, a ~ N(0, 1), dt_bias ~ N(0, 0.1);
  beta is "sigmoid(N(0, 1))".

Every value is drawn with ``numpy.random.default_rng(seed)`` (PCG64), rounded
to the workload dtype with round-to-nearest-even (through torch), and returned
as CPU tensors. The oracle reads back exactly the rounded values.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

# ---------------------------------------------------------------------------
# Workloads (sizes of the Qwen3.5 GDN layers the source pages describe).
# ---------------------------------------------------------------------------
WORKLOADS = {
    1: dict(name="tiny_fp32_d32", kind="core", num_seqs=1, seqlen=256, hqk=1, hv=1, dk=32, dv=32,
            dtype="f32", gate="uniform", g_low=-0.1, h0_std=0.0),
    2: dict(name="prefill_35b_a3b_1x4096", kind="core", num_seqs=1, seqlen=4096, hqk=16, hv=32,
            dk=128, dv=128, dtype="bf16", gate="model", h0_std=0.0),
    3: dict(name="prefill_long_4x32768", kind="core", num_seqs=4, seqlen=32768, hqk=16, hv=32,
            dk=128, dv=128, dtype="bf16", gate="model", h0_std=0.02),
    4: dict(name="decode_256x1", kind="decode", num_seqs=256, seqlen=1, hqk=16, hv=32, dk=128,
            dv=128, dtype="bf16", gate="model", h0_std=0.02),
    5: dict(name="prefill_397b_packed_8xU512_8192", kind="front", num_seqs=8, len_low=512,
            len_high=8192, hqk=16, hv=64, dk=128, dv=128, dtype="bf16", h0_std=0.02,
            conv_w_std=0.5),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _round(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """Round float64/float32 numpy values to ``dtype`` (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype)


def _normal(rng: np.random.Generator, shape, std=1.0, chunk=1 << 24) -> np.ndarray:
    """N(0, std) in float64, drawn in bounded pieces (same stream as one draw)."""
    total = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(total, dtype=np.float64)
    for s in range(0, total, chunk):
        e = min(total, s + chunk)
        out[s:e] = rng.standard_normal(e - s)
    out *= std
    return out.reshape(shape)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    """Divide each last-axis vector by its Euclidean norm (distribution recipe)."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


@dataclass
class CoreCase:
    """Inputs of the chunked core / decode step (CPU tensors)."""

    q: torch.Tensor            # [T, Hqk, dk]  dtype
    k: torch.Tensor            # [T, Hqk, dk]  dtype
    v: torch.Tensor            # [T, Hv, dv]   dtype
    g: torch.Tensor            # [T, Hv]       float32 (log-decay, <= 0)
    beta: torch.Tensor         # [T, Hv]       float32
    cu_seqlens: torch.Tensor   # [N+1]         int32
    h0: Optional[torch.Tensor]  # [N, Hv, dk, dv] float32 or None
    meta: dict = field(default_factory=dict)


@dataclass
class FrontCase:
    """Inputs of the front end + core (CPU tensors)."""

    mixed_qkv: torch.Tensor    # [T, 2*Hqk*dk + Hv*dv] dtype
    conv_weight: torch.Tensor  # [conv_dim, 4] dtype
    a: torch.Tensor            # [T, Hv] dtype
    b: torch.Tensor            # [T, Hv] dtype
    A_log: torch.Tensor        # [Hv] float32
    dt_bias: torch.Tensor      # [Hv] float32
    cu_seqlens: torch.Tensor   # [N+1] int32
    h0: Optional[torch.Tensor]  # [N, Hv, dk, dv] float32 or None
    meta: dict = field(default_factory=dict)


def _gates(rng, T, hv, gate, g_low=-0.1, g_high=0.0):
    """Draw (g, beta) as float64 arrays [T, Hv]."""
    if gate == "model":
        A_log = rng.uniform(0.0, 2.7, size=hv)
        dt_bias = rng.normal(0.0, 0.1, size=hv)
        a = rng.standard_normal((T, hv))
        g = -np.exp(A_log)[None, :] * _softplus(a + dt_bias[None, :])
        beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, hv))))
    elif gate == "uniform":
        g = rng.uniform(g_low, g_high, size=(T, hv))
        beta = rng.uniform(0.0, 1.0, size=(T, hv))
    else:
        raise ValueError(gate)
    return g, beta


def make_core_case(lengths, hqk, hv, dk, dv, dtype="bf16", gate="model", h0_std=0.0,
                   seed=0, g_low=-0.1, g_high=0.0, qk_normalize=True, meta=None) -> CoreCase:
    """Packed variable-length core inputs. Draw order: q, k, v, gates, initial state."""
    lengths = [int(x) for x in lengths]
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    n = len(lengths)
    td = torch_dtype(dtype)
    q = _normal(rng, (T, hqk, dk))
    k = _normal(rng, (T, hqk, dk))
    if qk_normalize and T > 0:
        q, k = _unit_rows(q), _unit_rows(k)
    v = _normal(rng, (T, hv, dv))
    g, beta = _gates(rng, T, hv, gate, g_low, g_high)
    h0 = None
    if h0_std > 0:
        h0 = _round(_normal(rng, (n, hv, dk, dv), std=h0_std), torch.float32)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))
    return CoreCase(q=_round(q, td), k=_round(k, td), v=_round(v, td),
                    g=_round(g, torch.float32), beta=_round(beta, torch.float32),
                    cu_seqlens=cu, h0=h0, meta=dict(meta or {}, dtype=dtype, hqk=hqk, hv=hv,
                                                    dk=dk, dv=dv, lengths=lengths))


def make_front_case(lengths, hqk, hv, dk, dv, dtype="bf16", h0_std=0.02, conv_w_std=0.5,
                    seed=0, meta=None) -> FrontCase:
    """Projected inputs for the front end. Draw order: mixed_qkv, conv weight, a, b,
    A_log, dt_bias, initial state."""
    lengths = [int(x) for x in lengths]
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    n = len(lengths)
    td = torch_dtype(dtype)
    conv_dim = 2 * hqk * dk + hv * dv
    x = _normal(rng, (T, conv_dim))
    w = _normal(rng, (conv_dim, 4), std=conv_w_std)
    a = _normal(rng, (T, hv))
    b = _normal(rng, (T, hv))
    A_log = rng.uniform(0.0, 2.7, size=hv)
    dt_bias = rng.normal(0.0, 0.1, size=hv)
    h0 = None
    if h0_std > 0:
        h0 = _round(_normal(rng, (n, hv, dk, dv), std=h0_std), torch.float32)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))
    return FrontCase(mixed_qkv=_round(x, td), conv_weight=_round(w, td), a=_round(a, td),
                     b=_round(b, td), A_log=_round(A_log, torch.float32),
                     dt_bias=_round(dt_bias, torch.float32), cu_seqlens=cu, h0=h0,
                     meta=dict(meta or {}, dtype=dtype, hqk=hqk, hv=hv, dk=dk, dv=dv,
                               lengths=lengths))


@dataclass
class GateCase:
    """Inputs of the output gate (CPU tensors)."""

    o: torch.Tensor        # [T, Hv, dv] dtype (stands in for the core output)
    z: torch.Tensor        # [T, Hv, dv] dtype (gate projection)
    weight: torch.Tensor   # [dv] float32
    meta: dict = field(default_factory=dict)


def make_gate_case(T, hv, dv, dtype="bf16", seed=0, meta=None) -> GateCase:
    """Draw order: o ~ N(0, 1), z ~ N(0, 1), weight ~ N(0, 0.1) (used with offset 1)."""
    rng = np.random.default_rng(seed)
    td = torch_dtype(dtype)
    o = _normal(rng, (T, hv, dv))
    z = _normal(rng, (T, hv, dv))
    w = _normal(rng, (dv,), std=0.1)
    return GateCase(o=_round(o, td), z=_round(z, td), weight=_round(w, torch.float32),
                    meta=dict(meta or {}, dtype=dtype, T=T, hv=hv, dv=dv))


@dataclass
class DecodeFrontCase:
    """Inputs of one decode token per sequence from projected inputs (CPU tensors)."""

    mixed_qkv: torch.Tensor    # [N, conv_dim] dtype
    window: torch.Tensor       # [N, conv_dim, 3] dtype, oldest first
    conv_weight: torch.Tensor  # [conv_dim, 4] dtype
    a: torch.Tensor            # [N, Hv] dtype
    b: torch.Tensor            # [N, Hv] dtype
    A_log: torch.Tensor        # [Hv] float32
    dt_bias: torch.Tensor      # [Hv] float32
    h0: torch.Tensor           # [N, Hv, dk, dv] float32
    meta: dict = field(default_factory=dict)


def make_decode_front_case(N, hqk, hv, dk, dv, dtype="bf16", h0_std=0.02, conv_w_std=0.5,
                           seed=0, meta=None) -> DecodeFrontCase:
    """Draw order: mixed_qkv, window, conv weight, a, b, A_log, dt_bias, state."""
    rng = np.random.default_rng(seed)
    td = torch_dtype(dtype)
    conv_dim = 2 * hqk * dk + hv * dv
    x = _normal(rng, (N, conv_dim))
    win = _normal(rng, (N, conv_dim, 3))
    w = _normal(rng, (conv_dim, 4), std=conv_w_std)
    a = _normal(rng, (N, hv))
    b = _normal(rng, (N, hv))
    A_log = rng.uniform(0.0, 2.7, size=hv)
    dt_bias = rng.normal(0.0, 0.1, size=hv)
    h0 = _round(_normal(rng, (N, hv, dk, dv), std=h0_std), torch.float32)
    return DecodeFrontCase(mixed_qkv=_round(x, td), window=_round(win, td),
                           conv_weight=_round(w, td), a=_round(a, td), b=_round(b, td),
                           A_log=_round(A_log, torch.float32),
                           dt_bias=_round(dt_bias, torch.float32), h0=h0,
                           meta=dict(meta or {}, dtype=dtype, N=N, hqk=hqk, hv=hv, dk=dk, dv=dv))


def workload_lengths(cfg_id: int, seed: Optional[int] = None):
    w = WORKLOADS[cfg_id]
    if "seqlen" in w:
        return [w["seqlen"]] * w["num_seqs"]
    rng = np.random.default_rng((1000 + cfg_id) if seed is None else seed)
    return [int(x) for x in rng.integers(w["len_low"], w["len_high"], size=w["num_seqs"],
                                         endpoint=True)]


def workload_case(cfg_id: int, seed: Optional[int] = None):
    """Inputs of workload ``cfg_id`` (1..5) with seed 1000 + cfg_id by default.

    Workload 5's lengths come from their own generator (seed 1000 + 5 + 100000 unless
    given) so that the front-end draws keep one fixed order."""
    w = WORKLOADS[cfg_id]
    s = (1000 + cfg_id) if seed is None else seed
    meta = dict(workload=w["name"], cfg_id=cfg_id, seed=s)
    if w["kind"] in ("core", "decode"):
        return make_core_case(workload_lengths(cfg_id), w["hqk"], w["hv"], w["dk"], w["dv"],
                              dtype=w["dtype"], gate=w["gate"], h0_std=w["h0_std"], seed=s,
                              g_low=w.get("g_low", -0.1), meta=meta)
    lengths = workload_lengths(cfg_id, seed=s + 100000)
    return make_front_case(lengths, w["hqk"], w["hv"], w["dk"], w["dv"], dtype=w["dtype"],
                           h0_std=w["h0_std"], conv_w_std=w["conv_w_std"], seed=s, meta=meta)


def slow_decay_case(lengths, hqk, hv, dk, dv, dtype="bf16", seed=7) -> CoreCase:
    """Slow-decay set: g ~ U(-0.01, 0), beta ~ U(0, 1), nonzero initial state, so that
    state carried across hundreds of chunks and the initial state stay visible."""
    return make_core_case(lengths, hqk, hv, dk, dv, dtype=dtype, gate="uniform", g_low=-0.01,
                          h0_std=0.02, seed=seed, meta=dict(workload="slow_decay"))
