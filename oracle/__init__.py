"""float64 CPU oracle for the Gated DeltaNet token mixer (ctypes binding).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The GPU library does
not depend on it and this package does not import the GPU library.

The arithmetic lives in ``gdn_oracle.c`` (plain C, float64, token by token,
OpenMP over independent (sequence, V head) chains). This module only builds the
shared object and marshals numpy arrays.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc (-O2, OpenMP). Always recompiles."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           _SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    dp = ctypes.POINTER(ctypes.c_double)
    lp = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.gdn_oracle_recurrent.restype = ctypes.c_int
    lib.gdn_oracle_recurrent.argtypes = [i64, lp, i64, i64, i64, i64, dp, dp, dp, dp, dp, dp,
                                         ctypes.c_double, dp, dp]
    lib.gdn_oracle_prepare.restype = ctypes.c_int
    lib.gdn_oracle_prepare.argtypes = [i64, lp, i64, i64, i64, i64, dp, dp, dp, dp, dp, dp, dp,
                                       ctypes.c_double, dp, dp, dp, dp, dp]
    lib.gdn_oracle_gated_rmsnorm.restype = ctypes.c_int
    lib.gdn_oracle_gated_rmsnorm.argtypes = [i64, i64, dp, dp, dp, ctypes.c_double,
                                             ctypes.c_double, dp]
    lib.gdn_oracle_decode_prepare.restype = ctypes.c_int
    lib.gdn_oracle_decode_prepare.argtypes = [i64, i64, i64, i64, i64, dp, dp, dp, dp, dp, dp,
                                              dp, dp, ctypes.c_double, dp, dp, dp, dp, dp]
    lib.gdn_oracle_recurrent_backward.restype = ctypes.c_int
    lib.gdn_oracle_recurrent_backward.argtypes = [i64, lp, i64, i64, i64, i64, dp, dp, dp, dp,
                                                  dp, dp, ctypes.c_double, dp, dp, dp, dp, dp,
                                                  dp, dp, dp]
    lib.gdn_oracle_num_threads.restype = ctypes.c_int
    lib.gdn_oracle_num_threads.argtypes = []
    _lib = lib
    return lib


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS or all visible cores)."""
    return int(_load().gdn_oracle_num_threads())


def recurrent(q, k, v, g, beta, cu_seqlens, initial_state=None, scale=1.0,
              output_final_state=True):
    """Token-by-token gated delta rule in float64.

    q, k: [T, Hqk, dk]; v: [T, Hv, dv]; g, beta: [T, Hv]; cu_seqlens: [N+1];
    initial_state: [N, Hv, dk, dv] or None. Returns (o [T, Hv, dv], final [N, Hv, dk, dv]
    or None).
    """
    lib = _load()
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    T, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    n = cu.shape[0] - 1
    assert k.shape == q.shape and v.shape[0] == T and g.shape == (T, hv) and beta.shape == (T, hv)
    assert int(cu[-1]) == T
    h0 = _f64(initial_state)
    if h0 is not None:
        assert h0.shape == (n, hv, dk, dv)
    o = np.zeros((T, hv, dv), dtype=np.float64)
    ht = np.zeros((n, hv, dk, dv), dtype=np.float64) if output_final_state else None
    rc = lib.gdn_oracle_recurrent(n, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), hqk, hv,
                                  dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                  _ptr(h0), float(scale), _ptr(o), _ptr(ht))
    if rc != 0:
        raise ValueError("gdn_oracle_recurrent rejected its arguments")
    return o, ht


def recurrent_backward(q, k, v, g, beta, cu_seqlens, dout, initial_state=None, dht=None,
                       scale=1.0):
    """Gradients of sum(o * dout) + sum(ht * dht) through the token recurrence, float64.

    Returns (dq, dk [T, Hqk, dk], dv [T, Hv, dv], dg, dbeta [T, Hv], dh0 [N, Hv, dk, dv]).
    """
    lib = _load()
    q, k, v, g, beta, dout = (_f64(a) for a in (q, k, v, g, beta, dout))
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    T, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    n = cu.shape[0] - 1
    assert dout.shape == (T, hv, dv) and int(cu[-1]) == T
    h0, dh = _f64(initial_state), _f64(dht)
    for st in (h0, dh):
        if st is not None:
            assert st.shape == (n, hv, dk, dv)
    dq = np.zeros((T, hqk, dk))
    dkk = np.zeros((T, hqk, dk))
    dvv = np.zeros((T, hv, dv))
    dg = np.zeros((T, hv))
    dbeta = np.zeros((T, hv))
    dh0 = np.zeros((n, hv, dk, dv))
    rc = lib.gdn_oracle_recurrent_backward(
        n, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), hqk, hv, dk, dv, _ptr(q), _ptr(k),
        _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), float(scale), _ptr(dout), _ptr(dh), _ptr(dq),
        _ptr(dkk), _ptr(dvv), _ptr(dg), _ptr(dbeta), _ptr(dh0))
    if rc != 0:
        raise ValueError("gdn_oracle_recurrent_backward rejected its arguments")
    return dq, dkk, dvv, dg, dbeta, dh0


def prepare(mixed_qkv, conv_weight, a, b, A_log, dt_bias, cu_seqlens, num_qk_heads,
            head_dim_k, num_v_heads, head_dim_v, conv_bias=None, l2_eps=1e-6):
    """Front end in float64: conv(4) + SiLU, split, q/k L2 norm, gates.

    Returns q [T,Hqk,dk], k [T,Hqk,dk], v [T,Hv,dv], g [T,Hv], beta [T,Hv].
    """
    lib = _load()
    x, w, a, b = (_f64(t) for t in (mixed_qkv, conv_weight, a, b))
    A_log, dt_bias, bias = _f64(A_log), _f64(dt_bias), _f64(conv_bias)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    T = x.shape[0]
    hqk, dk, hv, dv = int(num_qk_heads), int(head_dim_k), int(num_v_heads), int(head_dim_v)
    assert x.shape[1] == 2 * hqk * dk + hv * dv and w.shape == (x.shape[1], 4)
    assert a.shape == (T, hv) and b.shape == (T, hv) and int(cu[-1]) == T
    q = np.zeros((T, hqk, dk))
    k = np.zeros((T, hqk, dk))
    v = np.zeros((T, hv, dv))
    g = np.zeros((T, hv))
    beta = np.zeros((T, hv))
    rc = lib.gdn_oracle_prepare(cu.shape[0] - 1, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                hqk, hv, dk, dv, _ptr(x), _ptr(w), _ptr(bias), _ptr(a), _ptr(b),
                                _ptr(A_log), _ptr(dt_bias), float(l2_eps), _ptr(q), _ptr(k),
                                _ptr(v), _ptr(g), _ptr(beta))
    if rc != 0:
        raise ValueError("gdn_oracle_prepare rejected its arguments")
    return q, k, v, g, beta


def gated_rmsnorm(o, z, weight=None, weight_offset=0.0, eps=1e-6):
    """Output gate in float64: RMSNorm(o) * SiLU(z) over the last axis.

    o, z: [..., dv]; weight: [dv] or None (factor 1); factor = weight + weight_offset.
    """
    lib = _load()
    o, z, w = _f64(o), _f64(z), _f64(weight)
    assert o.shape == z.shape and o.ndim >= 1
    dv = o.shape[-1]
    rows = o.size // dv if dv else 0
    if w is not None:
        assert w.shape == (dv,)
    out = np.zeros_like(o)
    rc = lib.gdn_oracle_gated_rmsnorm(rows, dv, _ptr(o), _ptr(z), _ptr(w), float(weight_offset),
                                      float(eps), _ptr(out))
    if rc != 0:
        raise ValueError("gdn_oracle_gated_rmsnorm rejected its arguments")
    return out


def decode_prepare(x, window, conv_weight, a, b, A_log, dt_bias, num_qk_heads, head_dim_k,
                   num_v_heads, head_dim_v, conv_bias=None, l2_eps=1e-6):
    """Decode-side front end in float64 for one token per sequence with a conv window.

    x: [N, conv_dim]; window: [N, conv_dim, 3] (previous inputs, oldest first).
    Returns q [N,Hqk,dk], k [N,Hqk,dk], v [N,Hv,dv], g [N,Hv], beta [N,Hv], new window.
    """
    lib = _load()
    x, w, a, b = (_f64(t) for t in (x, conv_weight, a, b))
    win = np.array(window, dtype=np.float64, order="C", copy=True)
    A_log, dt_bias, bias = _f64(A_log), _f64(dt_bias), _f64(conv_bias)
    N = x.shape[0]
    hqk, dk, hv, dv = int(num_qk_heads), int(head_dim_k), int(num_v_heads), int(head_dim_v)
    assert x.shape[1] == 2 * hqk * dk + hv * dv and w.shape == (x.shape[1], 4)
    assert win.shape == (N, x.shape[1], 3) and a.shape == (N, hv) and b.shape == (N, hv)
    q = np.zeros((N, hqk, dk))
    k = np.zeros((N, hqk, dk))
    v = np.zeros((N, hv, dv))
    g = np.zeros((N, hv))
    beta = np.zeros((N, hv))
    rc = lib.gdn_oracle_decode_prepare(N, hqk, hv, dk, dv, _ptr(x), _ptr(win), _ptr(w),
                                       _ptr(bias), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
                                       float(l2_eps), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                       _ptr(beta))
    if rc != 0:
        raise ValueError("gdn_oracle_decode_prepare rejected its arguments")
    return q, k, v, g, beta, win
