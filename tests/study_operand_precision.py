"""Operand-precision study of the chunked form (CPU only; not collected by pytest).

Emulates the scan kernels' chunk formulas ([MoE report] §3.7 Steps 3-6 in the Y form the scan
uses: Y = V - diag(gamma) K H, V' = (T diag(beta)) Y, O = diag(gamma) Q H + P V',
H <- gamma_C H + K^T diag(delta) V') in float64, with chosen operands rounded once to bf16
(single), to fp16, or carried as a hi + lo pair of bf16 values (split), and reports the max
error / RMS of the outputs and final states against the float64 token-recurrence oracle. T, P,
gamma and delta are formed in float64 from the same inputs (the intra kernel forms them in fp32).

Operands: H (the state in K H and Q H; "HQ" only in Q H), T (T diag(beta)), P, Y (in T Y),
V (V' in P V'), D (diag(delta) V' in the update), KQ (q and k rows: "h" converts them to fp16).
Modes: "p" split, "s" bf16, "h" fp16, "f" fp32.

Usage: python tests/study_operand_precision.py   (a few minutes on 8 cores)
"""
import os
import sys
import time

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import oracle  # noqa: E402
import synthetic_inputs as si  # noqa: E402


def r32(x):
    return x.astype(np.float32).astype(np.float64)


def rbf16(x):
    t = torch.from_numpy(np.ascontiguousarray(x.astype(np.float32)))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def rf16(x):
    return r32(x).astype(np.float16).astype(np.float64)


def operand(x, mode):
    if mode == "f":
        return r32(x)
    if mode == "h":
        return rf16(x)
    if mode == "s":
        return rbf16(x)
    hi = rbf16(x)
    return hi + rbf16(r32(x) - hi)


def emulate(case, modes, C=64):
    q, k, v = (getattr(case, n).double().numpy() for n in ("q", "k", "v"))
    g, be = case.g.double().numpy(), case.beta.double().numpy()
    T_, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    G = hv // hqk
    cu = case.cu_seqlens.numpy()
    O = np.zeros((T_, hv, dv))
    HT = np.zeros((len(cu) - 1, hv, dk, dv))
    low = np.tril(np.ones((C, C)), -1).astype(bool)
    lowi = np.tril(np.ones((C, C))).astype(bool)
    for n in range(len(cu) - 1):
        s0, s1 = cu[n], cu[n + 1]
        H = np.zeros((hv, dk, dv)) if case.h0 is None else case.h0[n].double().numpy().copy()
        for c0 in range(s0, s1, C):
            L = min(C, s1 - c0)
            Kc, Qc = np.zeros((hv, C, dk)), np.zeros((hv, C, dk))
            Vc, gc, bc = np.zeros((hv, C, dv)), np.zeros((hv, C)), np.zeros((hv, C))
            Kc[:, :L] = np.repeat(k[c0:c0 + L], G, axis=1).transpose(1, 0, 2)
            Qc[:, :L] = np.repeat(q[c0:c0 + L], G, axis=1).transpose(1, 0, 2)
            if modes.get("KQ") == "h":
                Kc, Qc = rf16(Kc), rf16(Qc)
            Vc[:, :L] = v[c0:c0 + L].transpose(1, 0, 2)
            gc[:, :L], bc[:, :L] = g[c0:c0 + L].T, be[c0:c0 + L].T
            b = np.cumsum(gc, axis=1)
            gam, dl = np.exp(b), np.exp(b[:, -1:] - b)
            diff = b[:, :, None] - b[:, None, :]
            Gm = np.where(lowi[None], np.exp(np.where(lowi[None], diff, 0.0)), 0.0)
            A = np.where(low[None], bc[:, :, None] * Gm * (Kc @ Kc.transpose(0, 2, 1)), 0.0)
            TB = operand(np.linalg.inv(np.eye(C)[None] + A) * bc[:, None, :], modes["T"])
            P = operand(np.where(lowi[None], (Qc @ Kc.transpose(0, 2, 1)) * Gm, 0.0), modes["P"])
            HK = operand(H, modes["H"])
            HQ = operand(H, modes.get("HQ", modes["H"]))
            Y = Vc - gam[:, :, None] * (Kc @ HK)
            Vp = TB @ operand(Y, modes["Y"])
            Oc = gam[:, :, None] * (Qc @ HQ) + P @ operand(Vp, modes["V"])
            H = r32(np.exp(b[:, -1])[:, None, None] * H +
                    Kc.transpose(0, 2, 1) @ operand(dl[:, :, None] * Vp, modes["D"]))
            O[c0:c0 + L] = r32(Oc[:, :L]).transpose(1, 0, 2)
        HT[n] = H
    return O, HT


def err(a, r):
    return float(np.max(np.abs(a - r)) / np.sqrt(np.mean(r * r)))


SPLIT = dict(H="p", T="p", P="p", Y="p", V="p", D="p")
CONFIGS = {
    "all split": SPLIT,
    "all bf16": dict(H="s", T="s", P="s", Y="s", V="s", D="s"),
    "T bf16": dict(SPLIT, T="s"),
    "P bf16": dict(SPLIT, P="s"),
    "Y bf16": dict(SPLIT, Y="s"),
    "V' bf16": dict(SPLIT, V="s"),
    "V'' bf16": dict(SPLIT, D="s"),
    "H bf16": dict(SPLIT, H="s"),
    "all fp16": dict(H="h", T="h", P="h", Y="h", V="h", D="h", KQ="h"),
    "H fp16 (K, Q fp16): the kernels": dict(SPLIT, H="h", KQ="h"),
    "H, V'' fp16 (K, Q fp16)": dict(SPLIT, H="h", D="h", KQ="h"),
    "V'' fp16": dict(SPLIT, D="h"),
    "T, P fp16": dict(SPLIT, T="h", P="h"),
}


def main():
    cases = {
        "workload 2 (1x4096, 32 V heads)": si.workload_case(2),
        "slow decay 1x4096, 8 V heads": si.slow_decay_case([4096], 4, 8, 128, 128, seed=11),
        "model gates + h0, 1x16384, 4 V heads": si.make_core_case(
            [16384], 2, 4, 128, 128, gate="model", h0_std=0.02, seed=12),
        "slow decay 1x16384, 4 V heads": si.slow_decay_case([16384], 2, 4, 128, 128, seed=13),
    }
    for cname, case in cases.items():
        t0 = time.time()
        f = lambda t: None if t is None else t.double().numpy()  # noqa: E731
        o_ref, h_ref = oracle.recurrent(f(case.q), f(case.k), f(case.v), f(case.g), f(case.beta),
                                        case.cu_seqlens.numpy(), initial_state=f(case.h0))
        rms = np.sqrt(np.mean(o_ref ** 2))
        print(f"== {cname} (oracle {time.time() - t0:.1f} s), max|o|/RMS "
              f"{np.max(np.abs(o_ref)) / rms:.1f}", flush=True)
        for name, modes in CONFIGS.items():
            O, HT = emulate(case, modes)
            print(f"  {name:34s} o {err(O, o_ref):.2e}  final state {err(HT, h_ref):.2e}",
                  flush=True)


if __name__ == "__main__":
    main()
