"""Gated DeltaNet token mixer core for MI355X (gfx950): Python binding of ``libgdn.so``.

Argument marshalling only. Every step of the computation runs in the library's HIP kernels;
torch provides device memory and the current HIP stream. Calls are asynchronous on
``torch.cuda.current_stream()``. There is no CPU fallback: if ``libgdn.so`` is missing or a
tensor is not on the GPU, the call raises.

Entry points (same names as the C ABI in ``include/gdn.h``):
  prepare(...)         conv(4) + SiLU, split, q/k L2 norm, gates
  chunk_forward(...)   chunked prefill (chunk 64), optional initial/final states, varlen
  chunk_intra(...), chunk_scan(...)  the two stages of chunk_forward
  recurrent_step(...)  one decode token per sequence, state updated in place
  decode_prepare(...)  front end of one decode token per sequence with a cached conv window
  gated_rmsnorm(...)   output gate RMSNorm(o) * SiLU(z) per V-head vector
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = ["prepare", "chunk_forward", "chunk_intra", "chunk_scan", "recurrent_step",
           "recurrent_step_gated", "decode_step", "decode_step_gated",
           "decode_prepare", "gated_rmsnorm", "workspace_size", "library_path", "GdnError",
           "CHUNK"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libgdn.so")
CHUNK = 64

ABI_VERSION = 3  # GDN_ABI_VERSION of include/gdn.h that GdnShape and the signatures follow
GDN_DTYPE_F32, GDN_DTYPE_BF16, GDN_DTYPE_F32_SPLIT = 0, 1, 2
_DT = {torch.float32: GDN_DTYPE_F32, torch.bfloat16: GDN_DTYPE_BF16}


class GdnError(RuntimeError):
    pass


class GdnShape(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("total_tokens", ctypes.c_int32),
                ("num_qk_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
                ("head_dim_k", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
                ("qkv_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("in_dtype", ctypes.c_int32), ("scale", ctypes.c_float),
                ("state_dtype", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise GdnError(f"{_LIB_PATH} is not built; run `python -m gated_deltanet_linear_amd.build` "
                       "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(_LIB_PATH)
    sp = ctypes.POINTER(GdnShape)
    lib.gdn_prepare.restype = ctypes.c_int
    lib.gdn_prepare.argtypes = [sp, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P, _P,
                                _P, _P]
    lib.gdn_chunk_forward_workspace_size.restype = ctypes.c_size_t
    lib.gdn_chunk_forward_workspace_size.argtypes = [sp]
    lib.gdn_chunk_forward.restype = ctypes.c_int
    lib.gdn_chunk_forward.argtypes = [sp, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.gdn_chunk_forward_noalloc.restype = ctypes.c_int
    lib.gdn_chunk_forward_noalloc.argtypes = [sp, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.gdn_chunk_intra.restype = ctypes.c_int
    lib.gdn_chunk_intra.argtypes = [sp, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.gdn_chunk_scan.restype = ctypes.c_int
    lib.gdn_chunk_scan.argtypes = [sp, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    lib.gdn_chunk_backward_workspace_size.restype = ctypes.c_size_t
    lib.gdn_chunk_backward_workspace_size.argtypes = [sp]
    lib.gdn_chunk_backward.restype = ctypes.c_int
    lib.gdn_chunk_backward.argtypes = [sp, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       _P, _P, _P, ctypes.c_size_t, _P]
    lib.gdn_recurrent_step.restype = ctypes.c_int
    lib.gdn_recurrent_step.argtypes = [sp, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.gdn_decode_prepare.restype = ctypes.c_int
    lib.gdn_decode_prepare.argtypes = [sp, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P,
                                       _P, _P, _P, _P]
    lib.gdn_decode_step.restype = ctypes.c_int
    lib.gdn_decode_step.argtypes = [sp, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P,
                                    _P]
    lib.gdn_recurrent_step_gated.restype = ctypes.c_int
    lib.gdn_recurrent_step_gated.argtypes = [sp, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                             ctypes.c_float, _P, _P]
    lib.gdn_decode_step_gated.restype = ctypes.c_int
    lib.gdn_decode_step_gated.argtypes = [sp, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P,
                                          _P, _P, ctypes.c_float, ctypes.c_float, _P, _P]
    lib.gdn_gated_rmsnorm.restype = ctypes.c_int
    lib.gdn_gated_rmsnorm.argtypes = [sp, _P, _P, _P, ctypes.c_float, ctypes.c_float, _P, _P]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_abi_version.restype = ctypes.c_int
    lib.gdn_abi_version.argtypes = []
    if lib.gdn_abi_version() != ABI_VERSION:
        raise GdnError(f"{_LIB_PATH} has ABI version {lib.gdn_abi_version()}, this binding "
                       f"expects {ABI_VERSION}; rebuild the library")
    _lib = lib
    return lib


def _check(rc: int, what: str):
    if rc != 0:
        raise GdnError(f"{what}: {_load().gdn_status_string(rc).decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise GdnError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise GdnError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise GdnError(f"{name} must be contiguous")
    return t


def _out(t, shape, dtype, device, name):
    """An output buffer: a new tensor, or the caller's, which must be a contiguous GPU tensor of
    exactly this shape and dtype (the kernels write shape x dtype bytes through its pointer)."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _dev(t, name, dtype)
    if tuple(t.shape) != tuple(shape):
        raise GdnError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _out_dtype(out_dtype, o, default):
    """Output dtype: the one asked for, else that of a given output buffer, else the default."""
    if out_dtype is not None:
        return out_dtype
    return o.dtype if isinstance(o, torch.Tensor) else default


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(dt: torch.dtype, name: str) -> int:
    if dt not in _DT:
        raise GdnError(f"{name}: dtype {dt} not supported (float32 or bfloat16)")
    return _DT[dt]


def _shape(num_seqs, total_tokens, hqk, hv, dk, dv, qkv_dtype, out_dtype, in_dtype=None,
           scale=1.0, state_dtype=None, split_f32=False) -> GdnShape:
    qc = _dtype_code(qkv_dtype, "q/k/v")
    if split_f32:
        if qc != GDN_DTYPE_F32:
            raise GdnError("split_f32 takes float32 q/k/v")
        qc = GDN_DTYPE_F32_SPLIT
    return GdnShape(int(num_seqs), int(total_tokens), int(hqk), int(hv), int(dk), int(dv),
                    qc, _dtype_code(out_dtype, "o"),
                    _dtype_code(in_dtype or torch.bfloat16, "front-end input"), float(scale),
                    _dtype_code(state_dtype or torch.float32, "state"))


def _state_dtype(*states, default=None):
    """The one dtype of the given state tensors (None entries skipped)."""
    dts = {t.dtype for t in states if t is not None}
    if len(dts) > 1:
        raise GdnError("initial and final states must have the same dtype")
    return dts.pop() if dts else (default or torch.float32)


def _core_shape(q, k, g, beta, cu_seqlens, hv, dv, scale, out_dtype, state_dtype=None,
                split_f32=False):
    _dev(q, "q")
    _dev(k, "k", q.dtype)
    _dev(g, "g", torch.float32)
    _dev(beta, "beta", torch.float32)
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    if q.dim() != 3 or k.shape != q.shape:
        raise GdnError("q and k must be [T, H_qk, d_k]")
    T, hqk, dk = q.shape
    if g.shape != (T, hv) or beta.shape != (T, hv):
        raise GdnError("g and beta must be [T, H_v]")
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise GdnError("cu_seqlens must be [N + 1]")
    n = cu_seqlens.numel() - 1
    return _shape(n, T, hqk, hv, dk, dv, q.dtype, out_dtype or q.dtype, scale=scale,
                  state_dtype=state_dtype, split_f32=split_f32), n


def _v_shape(v, q):
    _dev(v, "v", q.dtype)
    if v.dim() != 3 or v.shape[0] != q.shape[0]:
        raise GdnError("v must be [T, H_v, d_v]")
    return v.shape[1], v.shape[2]


def workspace_size(total_tokens: int, num_seqs: int, num_qk_heads: int, num_v_heads: int,
                   head_dim: int, dtype=torch.bfloat16) -> int:
    s = _shape(num_seqs, total_tokens, num_qk_heads, num_v_heads, head_dim, head_dim, dtype, dtype)
    return int(_load().gdn_chunk_forward_workspace_size(ctypes.byref(s)))


def backward_workspace_size(total_tokens: int, num_seqs: int, num_qk_heads: int,
                            num_v_heads: int, head_dim: int) -> int:
    s = _shape(num_seqs, total_tokens, num_qk_heads, num_v_heads, head_dim, head_dim,
               torch.bfloat16, torch.bfloat16)
    return int(_load().gdn_chunk_backward_workspace_size(ctypes.byref(s)))


def _workspace(s: GdnShape, device, workspace):
    nbytes = int(_load().gdn_chunk_forward_workspace_size(ctypes.byref(s)))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    _dev(workspace, "workspace", torch.uint8)
    return workspace


def chunk_forward(q, k, v, g, beta, cu_seqlens, initial_state=None, output_final_state=True,
                  scale=1.0, out_dtype=None, workspace=None, final_state=None, o=None,
                  state_dtype=None,
                  split_f32=False) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked prefill. Returns (o [T, H_v, d_v], final_state [N, H_v, d_k, d_v] or None).

    ``final_state`` may be passed (and may be ``initial_state`` itself for an in-place update).
    States are fp32 or bf16 (one dtype for both: ``state_dtype``, else the given states' dtype,
    else fp32). ``split_f32``: float32 q/k/v taken on the split-bf16 MFMA path
    (GDN_DTYPE_F32_SPLIT) instead of the fp32 one.
    """
    hv, dv = _v_shape(v, q)
    sd = _state_dtype(initial_state, final_state, default=state_dtype)
    od = _out_dtype(out_dtype, o, q.dtype)
    s, n = _core_shape(q, k, g, beta, cu_seqlens, hv, dv, scale, od, sd, split_f32)
    T, dk = s.total_tokens, s.head_dim_k
    if initial_state is not None:
        _dev(initial_state, "initial_state", sd)
        if initial_state.shape != (n, hv, dk, dv):
            raise GdnError("initial_state must be [N, H_v, d_k, d_v]")
    o = _out(o, (T, hv, dv), od, q.device, "o")
    if output_final_state or final_state is not None:
        final_state = _out(final_state, (n, hv, dk, dv), sd, q.device, "final_state")
    ws = _workspace(s, q.device, workspace)
    rc = _load().gdn_chunk_forward(ctypes.byref(s), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(o),
                                   _ptr(final_state), _ptr(ws), ws.numel(), _stream())
    _check(rc, "gdn_chunk_forward")
    return o, final_state


def chunk_forward_noalloc(q, k, v, g, beta, cu_seqlens, initial_state=None,
                          output_final_state=True, scale=1.0, out_dtype=None, final_state=None,
                          o=None, state_dtype=None, split_f32=False):
    """chunk_forward through gdn_chunk_forward_noalloc: the same result, with the workspace in the
    library's own device array (no device allocation by the library; this wrapper still creates
    o and final_state unless they are given)."""
    hv, dv = _v_shape(v, q)
    sd = _state_dtype(initial_state, final_state, default=state_dtype)
    od = _out_dtype(out_dtype, o, q.dtype)
    s, n = _core_shape(q, k, g, beta, cu_seqlens, hv, dv, scale, od, sd, split_f32)
    T, dk = s.total_tokens, s.head_dim_k
    if initial_state is not None:
        _dev(initial_state, "initial_state", sd)
        if initial_state.shape != (n, hv, dk, dv):
            raise GdnError("initial_state must be [N, H_v, d_k, d_v]")
    o = _out(o, (T, hv, dv), od, q.device, "o")
    if output_final_state or final_state is not None:
        final_state = _out(final_state, (n, hv, dk, dv), sd, q.device, "final_state")
    rc = _load().gdn_chunk_forward_noalloc(ctypes.byref(s), _ptr(cu_seqlens), _ptr(q), _ptr(k),
                                           _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                           _ptr(o), _ptr(final_state), _stream())
    _check(rc, "gdn_chunk_forward_noalloc")
    return o, final_state


def chunk_intra(q, k, g, beta, cu_seqlens, num_v_heads, workspace, scale=1.0, split_f32=False):
    """Stage 1 of chunk_forward (state-independent in-chunk work) into ``workspace``."""
    s, n = _core_shape(q, k, g, beta, cu_seqlens, int(num_v_heads), q.shape[2], scale, None,
                       split_f32=split_f32)
    _dev(workspace, "workspace", torch.uint8)
    rc = _load().gdn_chunk_intra(ctypes.byref(s), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(g),
                                 _ptr(beta), _ptr(workspace), workspace.numel(), _stream())
    _check(rc, "gdn_chunk_intra")


def chunk_scan(q, k, v, g, beta, cu_seqlens, workspace, initial_state=None, o=None,
               final_state=None, scale=1.0, out_dtype=None, split_f32=False):
    """Stage 2 of chunk_forward (sequential cross-chunk recurrence) from ``workspace``."""
    hv, dv = _v_shape(v, q)
    sd = _state_dtype(initial_state, final_state)
    od = _out_dtype(out_dtype, o, q.dtype)
    s, n = _core_shape(q, k, g, beta, cu_seqlens, hv, dv, scale, od, sd, split_f32)
    for t, name in ((initial_state, "initial_state"), (final_state, "final_state")):
        if t is not None:
            _dev(t, name, sd)
            if t.shape != (n, hv, s.head_dim_k, dv):
                raise GdnError(f"{name} must be [N, H_v, d_k, d_v]")
    _dev(workspace, "workspace", torch.uint8)
    o = _out(o, (s.total_tokens, s.num_v_heads, s.head_dim_v), od, q.device, "o")
    rc = _load().gdn_chunk_scan(ctypes.byref(s), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(initial_state), _ptr(o), _ptr(final_state), _ptr(workspace),
                                workspace.numel(), _stream())
    _check(rc, "gdn_chunk_scan")
    return o, final_state


def chunk_backward(q, k, v, g, beta, cu_seqlens, dout, initial_state=None, dht=None, scale=1.0,
                   workspace=None, state_dtype=None):
    """Gradients of sum(o * dout) + sum(final_state * dht) for the chunked prefill with these
    inputs. Returns (dq, dk [T, H_qk, d_k], dv [T, H_v, d_v] in the q/k/v dtype, dg, dbeta
    [T, H_v] fp32, dh0 [N, H_v, d_k, d_v] in the state dtype)."""
    hv, dv_ = _v_shape(v, q)
    _dev(dout, "dout")
    sd = _state_dtype(initial_state, dht, default=state_dtype)
    s, n = _core_shape(q, k, g, beta, cu_seqlens, hv, dv_, scale, dout.dtype, sd)
    T, hqk, dk_ = s.total_tokens, s.num_qk_heads, s.head_dim_k
    if dout.shape != (T, hv, dv_):
        raise GdnError("dout must be [T, H_v, d_v]")
    for t, name in ((initial_state, "initial_state"), (dht, "dht")):
        if t is not None:
            _dev(t, name, sd)
            if t.shape != (n, hv, dk_, dv_):
                raise GdnError(f"{name} must be [N, H_v, d_k, d_v]")
    lib = _load()
    nbytes = int(lib.gdn_chunk_backward_workspace_size(ctypes.byref(s)))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace", torch.uint8)
    dev = q.device
    dq = torch.empty((T, hqk, dk_), dtype=q.dtype, device=dev)
    dk = torch.empty((T, hqk, dk_), dtype=q.dtype, device=dev)
    dv = torch.empty((T, hv, dv_), dtype=q.dtype, device=dev)
    dg = torch.empty((T, hv), dtype=torch.float32, device=dev)
    dbeta = torch.empty((T, hv), dtype=torch.float32, device=dev)
    dh0 = torch.empty((n, hv, dk_, dv_), dtype=sd, device=dev)
    rc = lib.gdn_chunk_backward(ctypes.byref(s), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(dout), _ptr(dht),
                                _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0),
                                _ptr(workspace), workspace.numel(), _stream())
    _check(rc, "gdn_chunk_backward")
    return dq, dk, dv, dg, dbeta, dh0


def recurrent_step(q, k, v, g, beta, state, scale=1.0, out_dtype=None, o=None) -> torch.Tensor:
    """One decode token per sequence: q, k [N, H_qk, d_k], v [N, H_v, d_v], g, beta [N, H_v],
    state [N, H_v, d_k, d_v] fp32 or bf16 (updated in place). Returns o [N, H_v, d_v]."""
    _dev(q, "q")
    _dev(k, "k", q.dtype)
    _dev(v, "v", q.dtype)
    _dev(g, "g", torch.float32)
    _dev(beta, "beta", torch.float32)
    _dev(state, "state")
    N, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    if k.shape != q.shape or v.shape[0] != N or g.shape != (N, hv) or beta.shape != (N, hv) \
            or state.shape != (N, hv, dk, dv):
        raise GdnError("recurrent_step: inconsistent shapes")
    od = _out_dtype(out_dtype, o, q.dtype)
    s = _shape(N, N, hqk, hv, dk, dv, q.dtype, od, scale=scale, state_dtype=state.dtype)
    o = _out(o, (N, hv, dv), od, q.device, "o")
    rc = _load().gdn_recurrent_step(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                    _ptr(beta), _ptr(state), _ptr(o), _stream())
    _check(rc, "gdn_recurrent_step")
    return o


def _gate_args(z, weight, n, hv, dv, name):
    _dev(z, "z")
    if z.shape != (n, hv, dv):
        raise GdnError(f"{name}: z must be [N, H_v, d_v]")
    if weight is not None:
        _dev(weight, "weight", torch.float32)
        if weight.shape != (dv,):
            raise GdnError(f"{name}: weight must be [d_v]")


def recurrent_step_gated(q, k, v, g, beta, state, z, weight=None, weight_offset=0.0, eps=1e-6,
                         scale=1.0, out_dtype=None, out=None) -> torch.Tensor:
    """recurrent_step with the output gate fused into the same kernel: returns
    RMSNorm(o) * (weight + weight_offset) * SiLU(z) per V-head row, [N, H_v, d_v] (out_dtype,
    default q's dtype); z [N, H_v, d_v] (its dtype is the shape's in_dtype), weight [d_v] fp32
    or None (factor 1). The state is updated in place as by recurrent_step."""
    _dev(q, "q")
    _dev(k, "k", q.dtype)
    _dev(v, "v", q.dtype)
    _dev(g, "g", torch.float32)
    _dev(beta, "beta", torch.float32)
    _dev(state, "state")
    N, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    if k.shape != q.shape or v.shape[0] != N or g.shape != (N, hv) or beta.shape != (N, hv) \
            or state.shape != (N, hv, dk, dv):
        raise GdnError("recurrent_step_gated: inconsistent shapes")
    _gate_args(z, weight, N, hv, dv, "recurrent_step_gated")
    od = _out_dtype(out_dtype, out, q.dtype)
    s = _shape(N, N, hqk, hv, dk, dv, q.dtype, od, in_dtype=z.dtype, scale=scale,
               state_dtype=state.dtype)
    out = _out(out, (N, hv, dv), od, q.device, "out")
    rc = _load().gdn_recurrent_step_gated(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                          _ptr(beta), _ptr(state), _ptr(z), _ptr(weight),
                                          float(weight_offset), float(eps), _ptr(out), _stream())
    _check(rc, "gdn_recurrent_step_gated")
    return out


def prepare(mixed_qkv, conv_weight, a, b, A_log, dt_bias, cu_seqlens, num_qk_heads, head_dim_k,
            num_v_heads, head_dim_v, conv_bias=None, l2norm_eps=1e-6, qkv_dtype=None):
    """Front end: returns q, k [T, H_qk, d_k], v [T, H_v, d_v] (qkv_dtype, default the input
    dtype) and g, beta [T, H_v] fp32."""
    _dev(mixed_qkv, "mixed_qkv")
    dt = mixed_qkv.dtype
    _dev(conv_weight, "conv_weight", dt)
    _dev(a, "a", dt)
    _dev(b, "b", dt)
    _dev(A_log, "A_log", torch.float32)
    _dev(dt_bias, "dt_bias", torch.float32)
    _dev(cu_seqlens, "cu_seqlens", torch.int32)
    if conv_bias is not None:
        _dev(conv_bias, "conv_bias", dt)
    T, conv_dim = mixed_qkv.shape
    hqk, dk, hv, dv = int(num_qk_heads), int(head_dim_k), int(num_v_heads), int(head_dim_v)
    if conv_dim != 2 * hqk * dk + hv * dv or conv_weight.shape != (conv_dim, 4):
        raise GdnError("mixed_qkv must be [T, 2*H_qk*d_k + H_v*d_v] and conv_weight [conv_dim, 4]")
    if a.shape != (T, hv) or b.shape != (T, hv) or A_log.shape != (hv,) or dt_bias.shape != (hv,):
        raise GdnError("a, b must be [T, H_v]; A_log, dt_bias [H_v]")
    qd = qkv_dtype or dt
    n = cu_seqlens.numel() - 1
    s = _shape(n, T, hqk, hv, dk, dv, qd, qd, in_dtype=dt)
    dev = mixed_qkv.device
    q = torch.empty((T, hqk, dk), dtype=qd, device=dev)
    k = torch.empty((T, hqk, dk), dtype=qd, device=dev)
    v = torch.empty((T, hv, dv), dtype=qd, device=dev)
    g = torch.empty((T, hv), dtype=torch.float32, device=dev)
    beta = torch.empty((T, hv), dtype=torch.float32, device=dev)
    rc = _load().gdn_prepare(ctypes.byref(s), _ptr(cu_seqlens), _ptr(mixed_qkv), _ptr(conv_weight),
                             _ptr(conv_bias), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
                             float(l2norm_eps), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _stream())
    _check(rc, "gdn_prepare")
    return q, k, v, g, beta


def decode_prepare(mixed_qkv, conv_window, conv_weight, a, b, A_log, dt_bias, num_qk_heads,
                   head_dim_k, num_v_heads, head_dim_v, conv_bias=None, l2norm_eps=1e-6,
                   qkv_dtype=None):
    """Front end of one decode token per sequence with a cached conv window.

    mixed_qkv [N, conv_dim]; conv_window [N, conv_dim, 3] (previous inputs, oldest first; updated
    in place to the last three). Returns q, k [N, H_qk, d_k], v [N, H_v, d_v] (qkv_dtype, default
    the input dtype) and g, beta [N, H_v] fp32.
    """
    _dev(mixed_qkv, "mixed_qkv")
    dt = mixed_qkv.dtype
    _dev(conv_window, "conv_window", dt)
    _dev(conv_weight, "conv_weight", dt)
    _dev(a, "a", dt)
    _dev(b, "b", dt)
    _dev(A_log, "A_log", torch.float32)
    _dev(dt_bias, "dt_bias", torch.float32)
    if conv_bias is not None:
        _dev(conv_bias, "conv_bias", dt)
    N, conv_dim = mixed_qkv.shape
    hqk, dk, hv, dv = int(num_qk_heads), int(head_dim_k), int(num_v_heads), int(head_dim_v)
    if conv_dim != 2 * hqk * dk + hv * dv or conv_weight.shape != (conv_dim, 4):
        raise GdnError("mixed_qkv must be [N, 2*H_qk*d_k + H_v*d_v] and conv_weight [conv_dim, 4]")
    if conv_window.shape != (N, conv_dim, 3):
        raise GdnError("conv_window must be [N, conv_dim, 3]")
    if a.shape != (N, hv) or b.shape != (N, hv) or A_log.shape != (hv,) or dt_bias.shape != (hv,):
        raise GdnError("a, b must be [N, H_v]; A_log, dt_bias [H_v]")
    qd = qkv_dtype or dt
    s = _shape(N, N, hqk, hv, dk, dv, qd, qd, in_dtype=dt)
    dev = mixed_qkv.device
    q = torch.empty((N, hqk, dk), dtype=qd, device=dev)
    k = torch.empty((N, hqk, dk), dtype=qd, device=dev)
    v = torch.empty((N, hv, dv), dtype=qd, device=dev)
    g = torch.empty((N, hv), dtype=torch.float32, device=dev)
    beta = torch.empty((N, hv), dtype=torch.float32, device=dev)
    rc = _load().gdn_decode_prepare(ctypes.byref(s), _ptr(mixed_qkv), _ptr(conv_window),
                                    _ptr(conv_weight), _ptr(conv_bias), _ptr(a), _ptr(b),
                                    _ptr(A_log), _ptr(dt_bias), float(l2norm_eps), _ptr(q),
                                    _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _stream())
    _check(rc, "gdn_decode_prepare")
    return q, k, v, g, beta


def decode_step(mixed_qkv, conv_window, conv_weight, a, b, A_log, dt_bias, state, num_qk_heads,
                head_dim, num_v_heads, conv_bias=None, l2norm_eps=1e-6, scale=1.0, out_dtype=None,
                o=None):
    """One decode token per sequence from projected inputs, fused (front end + gated delta step).

    mixed_qkv [N, conv_dim]; conv_window [N, conv_dim, 3] (updated in place); conv_weight
    [conv_dim, 4]; a, b [N, H_v]; A_log, dt_bias [H_v] fp32; state [N, H_v, d, d] fp32 or bf16
    (updated in place). Returns o [N, H_v, d] (out_dtype, default the input dtype).
    """
    _dev(mixed_qkv, "mixed_qkv")
    dt = mixed_qkv.dtype
    _dev(conv_window, "conv_window", dt)
    _dev(conv_weight, "conv_weight", dt)
    _dev(a, "a", dt)
    _dev(b, "b", dt)
    _dev(A_log, "A_log", torch.float32)
    _dev(dt_bias, "dt_bias", torch.float32)
    _dev(state, "state")
    if conv_bias is not None:
        _dev(conv_bias, "conv_bias", dt)
    N, conv_dim = mixed_qkv.shape
    hqk, d, hv = int(num_qk_heads), int(head_dim), int(num_v_heads)
    if conv_dim != (2 * hqk + hv) * d or conv_weight.shape != (conv_dim, 4):
        raise GdnError("mixed_qkv must be [N, (2*H_qk + H_v)*d] and conv_weight [conv_dim, 4]")
    if conv_window.shape != (N, conv_dim, 3):
        raise GdnError("conv_window must be [N, conv_dim, 3]")
    if a.shape != (N, hv) or b.shape != (N, hv) or A_log.shape != (hv,) or dt_bias.shape != (hv,):
        raise GdnError("a, b must be [N, H_v]; A_log, dt_bias [H_v]")
    if state.shape != (N, hv, d, d):
        raise GdnError("state must be [N, H_v, d, d]")
    od = _out_dtype(out_dtype, o, dt)
    s = _shape(N, N, hqk, hv, d, d, torch.float32, od, in_dtype=dt, scale=scale,
               state_dtype=state.dtype)
    o = _out(o, (N, hv, d), od, mixed_qkv.device, "o")
    rc = _load().gdn_decode_step(ctypes.byref(s), _ptr(mixed_qkv), _ptr(conv_window),
                                 _ptr(conv_weight), _ptr(conv_bias), _ptr(a), _ptr(b), _ptr(A_log),
                                 _ptr(dt_bias), float(l2norm_eps), _ptr(state), _ptr(o), _stream())
    _check(rc, "gdn_decode_step")
    return o


def decode_step_gated(mixed_qkv, conv_window, conv_weight, a, b, A_log, dt_bias, state, z,
                      num_qk_heads, head_dim, num_v_heads, weight=None, weight_offset=0.0,
                      norm_eps=1e-6, conv_bias=None, l2norm_eps=1e-6, scale=1.0, out_dtype=None,
                      out=None):
    """decode_step with the output gate fused into the same kernel: one decode token per
    sequence from projected inputs to RMSNorm(o) * (weight + weight_offset) * SiLU(z), [N, H_v, d]
    (out_dtype, default the input dtype). z [N, H_v, d] in the input dtype; the window and the
    state are updated in place as by decode_step."""
    _dev(mixed_qkv, "mixed_qkv")
    dt = mixed_qkv.dtype
    _dev(conv_window, "conv_window", dt)
    _dev(conv_weight, "conv_weight", dt)
    _dev(a, "a", dt)
    _dev(b, "b", dt)
    _dev(A_log, "A_log", torch.float32)
    _dev(dt_bias, "dt_bias", torch.float32)
    _dev(state, "state")
    if conv_bias is not None:
        _dev(conv_bias, "conv_bias", dt)
    N, conv_dim = mixed_qkv.shape
    hqk, d, hv = int(num_qk_heads), int(head_dim), int(num_v_heads)
    if conv_dim != (2 * hqk + hv) * d or conv_weight.shape != (conv_dim, 4):
        raise GdnError("mixed_qkv must be [N, (2*H_qk + H_v)*d] and conv_weight [conv_dim, 4]")
    if conv_window.shape != (N, conv_dim, 3):
        raise GdnError("conv_window must be [N, conv_dim, 3]")
    if a.shape != (N, hv) or b.shape != (N, hv) or A_log.shape != (hv,) or dt_bias.shape != (hv,):
        raise GdnError("a, b must be [N, H_v]; A_log, dt_bias [H_v]")
    if state.shape != (N, hv, d, d):
        raise GdnError("state must be [N, H_v, d, d]")
    _gate_args(z, weight, N, hv, d, "decode_step_gated")
    if z.dtype != dt:
        raise GdnError("decode_step_gated: z must have the input dtype")
    od = _out_dtype(out_dtype, out, dt)
    s = _shape(N, N, hqk, hv, d, d, torch.float32, od, in_dtype=dt, scale=scale,
               state_dtype=state.dtype)
    out = _out(out, (N, hv, d), od, mixed_qkv.device, "out")
    rc = _load().gdn_decode_step_gated(ctypes.byref(s), _ptr(mixed_qkv), _ptr(conv_window),
                                       _ptr(conv_weight), _ptr(conv_bias), _ptr(a), _ptr(b),
                                       _ptr(A_log), _ptr(dt_bias), float(l2norm_eps), _ptr(state),
                                       _ptr(z), _ptr(weight), float(weight_offset),
                                       float(norm_eps), _ptr(out), _stream())
    _check(rc, "gdn_decode_step_gated")
    return out


def gated_rmsnorm(o, z, weight=None, weight_offset=0.0, eps=1e-6, out=None):
    """Output gate: RMSNorm(o) * SiLU(z) per V-head vector (last axis, d_v).

    o [T, H_v, d_v] (the core output's dtype), z [T, H_v, d_v]; weight [d_v] fp32 or None
    (factor weight + weight_offset, 1 without a weight). Returns out (a new tensor, or `out`,
    which may be `o`).
    """
    _dev(o, "o")
    _dev(z, "z")
    if o.dim() != 3 or z.shape != o.shape:
        raise GdnError("o and z must be [T, H_v, d_v] of the same shape")
    if weight is not None:
        _dev(weight, "weight", torch.float32)
        if weight.shape != (o.shape[2],):
            raise GdnError("weight must be [d_v]")
    if out is None:
        out = torch.empty_like(o)
    else:
        _dev(out, "out", o.dtype)
        if out.shape != o.shape:
            raise GdnError("out must have the shape of o")
    T, hv, dv = o.shape
    s = _shape(1, T, 1, hv, dv, dv, o.dtype, o.dtype, in_dtype=z.dtype)
    rc = _load().gdn_gated_rmsnorm(ctypes.byref(s), _ptr(o), _ptr(z), _ptr(weight),
                                   float(weight_offset), float(eps), _ptr(out), _stream())
    _check(rc, "gdn_gated_rmsnorm")
    return out
