"""Helpers shared by the GPU parity tests: oracle runs on whole cases or on sampled
(sequence, V head) chains, and the tolerance check max|err| <= tol * RMS(reference)."""

from __future__ import annotations

import numpy as np
import torch

import oracle

# Tolerances: fp32 inputs 1e-4 * RMS, bf16 inputs 2e-2 * RMS, on outputs and final states.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def f64(t):
    return None if t is None else t.detach().double().cpu().numpy()


def rel_err(got, ref) -> float:
    got = f64(got) if isinstance(got, torch.Tensor) else np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return err / rms if rms > 0 else err


def assert_rms_close(got, ref, tol, what):
    e = rel_err(got, ref)
    print(f"  {what}: max|err| = {e:.3e} x RMS (tol {tol:g})", flush=True)
    assert e <= tol, f"{what}: max|err| = {e:.3e} x RMS > {tol:g}"


def assert_rms_close_rounded_out(got, ref, tol, what):
    """For bf16 outputs: the output format's own rounding (one bf16 unit in the last place,
    2^-8 |ref|, covering a rounding decision flipped by fp32 arithmetic) is allowed on top of
    tol * RMS(ref)."""
    g = f64(got) if isinstance(got, torch.Tensor) else np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(r * r)))
    excess = np.abs(g - r) - 2.0 ** -8 * np.abs(r)
    e = float(np.max(excess)) / rms if r.size and rms > 0 else 0.0
    print(f"  {what}: max(|err| - ulp_bf16) = {max(e, 0.0):.3e} x RMS (tol {tol:g})", flush=True)
    assert e <= tol, f"{what}: max(|err| - ulp_bf16) = {e:.3e} x RMS > {tol:g}"


def oracle_case(case):
    """float64 oracle on a whole CoreCase."""
    return oracle.recurrent(f64(case.q), f64(case.k), f64(case.v), f64(case.g), f64(case.beta),
                            case.cu_seqlens.numpy(), initial_state=f64(case.h0))


def oracle_chains(case, chains):
    """float64 oracle on chosen (sequence n, V head h) chains only.

    Returns {(n, h): (o [L, d_v], final [d_k, d_v])}."""
    cu = case.cu_seqlens.numpy().astype(np.int64)
    hv = case.v.shape[1]
    G = hv // case.q.shape[1]
    out = {}
    for n, h in chains:
        s, e = int(cu[n]), int(cu[n + 1])
        m = h // G
        q = f64(case.q[s:e, m:m + 1])
        k = f64(case.k[s:e, m:m + 1])
        v = f64(case.v[s:e, h:h + 1])
        g = f64(case.g[s:e, h:h + 1])
        b = f64(case.beta[s:e, h:h + 1])
        h0 = None if case.h0 is None else f64(case.h0[n:n + 1, h:h + 1])
        o, ht = oracle.recurrent(q, k, v, g, b, [0, e - s], initial_state=h0)
        out[(n, h)] = (o[:, 0], ht[0, 0])
    return out


def to_dev(case, dev="cuda"):
    return {k: (None if getattr(case, k) is None else getattr(case, k).to(dev))
            for k in ("q", "k", "v", "g", "beta", "cu_seqlens", "h0")}


def bf16_store(x, rounding):
    """Store float64 values as bf16 and read them back: round to nearest even ("rne", torch's
    cast of the fp32 value) or truncate toward zero ("trunc", the top 16 bits of the fp32 value),
    or keep them ("none")."""
    if rounding == "none":
        return x
    x32 = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if rounding == "rne":
        return x32.to(torch.bfloat16).double().numpy()
    if rounding == "trunc":
        return (x32.view(torch.int32) & ~0xFFFF).view(torch.float32).double().numpy()
    raise ValueError(rounding)


def decode_state_storage_model(case, h0, N, T, rounding):
    """Error model of a stored bf16 decode state: T decode steps of N sequences (token t of
    sequence n at row t * N + n) in float64 arithmetic, with the state written back through
    bf16_store(rounding) after every step and each output formed before that store, as the decode
    kernel does. Returns (o [N, T, H_v, d_v], final state [N, H_v, d_k, d_v]). With rounding
    "none" it is the plain token recurrence (pinned against the oracle)."""
    q, k, v, g, b = (f64(getattr(case, a)) for a in ("q", "k", "v", "g", "beta"))
    G = v.shape[1] // q.shape[1]
    H = f64(h0).copy()
    outs = []
    for t in range(T):
        sl = slice(t * N, (t + 1) * N)
        qt, kt = np.repeat(q[sl], G, axis=1), np.repeat(k[sl], G, axis=1)
        H = np.exp(g[sl])[:, :, None, None] * H
        u = b[sl][:, :, None] * (v[sl] - np.einsum("nhij,nhi->nhj", H, kt))
        H = H + kt[:, :, :, None] * u[:, :, None, :]
        outs.append(np.einsum("nhij,nhi->nhj", H, qt))
        H = bf16_store(H, rounding)
    return np.stack(outs, 1), H
