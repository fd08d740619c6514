"""Benchmark of the Gated DeltaNet core on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--only NAME]

Prints ONE JSON line. The headline ``value`` is prefill tokens/s of the 35B-A3B-shaped GDN
layer (1 x 4096 tokens, 16 QK / 32 V heads, d = 128, bf16 q/k/v): one step is one
gdn_chunk_forward (its two kernels, gdn_chunk_intra then gdn_chunk_scan) over inputs already
resident in HBM. The same line carries decode tokens/s (256 sequences x 1 token, 537 MB fp32
state updated in place), the long-context and packed front-end workloads, per-kernel HIP-event
timings, the roofline of each workload's dominant kernel and the float64 CPU oracle timed on
a bounded sample on this host.

Roofline conventions (algorithmic work, not what the kernels happen to issue):
  prefill FLOPs per token per V head = (4/G) C d_k + 2 C d_k + 4 C d_v + 6 d_k d_v   (C = 64)
    of which the scan kernel's share is 4 C d_v + 6 d_k d_v (state products, T diag(beta) Y
    and the masked intra-chunk product); peak = 2500 TFLOP/s dense bf16 MFMA.
  decode bytes = 2 N H_v d_k d_v 4 + N [H_qk 2 d_k e + H_v (2 d_v e + 8)];  peak 8000 GB/s.
  front-end bytes = T [2 conv_dim e + 2 H_v e + 8 H_v] (+ q/k/v written at their dtype).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
C = 64


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None,
                    help="run one workload: prefill, decode, long, front")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 3 times (the known-size kernel that "
                         "scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings to bytes)")
    return ap.parse_args()


def prefill_flops_per_token_head(hqk, hv, dk, dv):
    G = hv // hqk
    return (4 / G) * C * dk + 2 * C * dk + 4 * C * dv + 6 * dk * dv


def scan_flops_per_token_head(dk, dv):
    return 4 * C * dv + 6 * dk * dv


def prefill_bytes(lengths, hqk, hv, dk, dv, e, h0_given, state_out=True):
    T = sum(lengths)
    n = len(lengths)
    b = T * (hqk * 2 * dk * e + hv * (2 * dv * e + 8))
    b += n * hv * dk * dv * 4 * ((1 if state_out else 0) + (1 if h0_given else 0))
    return b


def _traffic(kernel_key):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was taken on the
    current source of that kernel; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_key}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(ROOT, rec["source"])
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest() if os.path.exists(src) else None
    if sha != rec.get("source_sha256"):
        return None
    return rec.get("hbm_bytes_per_launch")


class Timer:
    """HIP events recorded on the stream the kernels are launched on (torch's current
    stream; the library launches on it)."""

    def __init__(self, torch, names, steps):
        self.torch = torch
        self.names = names
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
                   for _ in range(steps)]

    def mark(self, step, i):
        self.ev[step][i].record(self.torch.cuda.current_stream())

    def per_kernel_ms(self):
        out = {}
        for i, nm in enumerate(self.names):
            out[nm] = sum(e[i].elapsed_time(e[i + 1]) for e in self.ev) / len(self.ev)
        return out


def run_prefill(torch, gdn, si, cfg_id, steps, warmup, with_h0):
    case = si.workload_case(cfg_id)
    dev = "cuda"
    d = {k: (None if getattr(case, k) is None else getattr(case, k).to(dev))
         for k in ("q", "k", "v", "g", "beta", "cu_seqlens", "h0")}
    T, hqk, dk = case.q.shape
    hv, dv = case.v.shape[1], case.v.shape[2]
    n = case.cu_seqlens.numel() - 1
    ws = torch.empty(gdn.workspace_size(T, n, hqk, hv, dk), dtype=torch.uint8, device=dev)
    o = torch.empty((T, hv, dv), dtype=torch.bfloat16, device=dev)
    ht = torch.empty((n, hv, dk, dv), dtype=torch.float32, device=dev)
    h0 = d["h0"] if with_h0 else None

    def step(tm=None, i=0):
        if tm:
            tm.mark(i, 0)
        gdn.chunk_intra(d["q"], d["k"], d["g"], d["beta"], d["cu_seqlens"], hv, ws)
        if tm:
            tm.mark(i, 1)
        gdn.chunk_scan(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], ws,
                       initial_state=h0, o=o, final_state=ht)
        if tm:
            tm.mark(i, 2)

    for _ in range(warmup):
        step()
    tm = Timer(torch, ["gdn_chunk_intra", "gdn_chunk_scan"], steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(tm, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = tm.per_kernel_ms()
    lengths = case.meta["lengths"]
    F = prefill_flops_per_token_head(hqk, hv, dk, dv) * T * hv
    Fscan = scan_flops_per_token_head(dk, dv) * T * hv
    B = prefill_bytes(lengths, hqk, hv, dk, dv, 2, with_h0)
    ms = wall * 1e3 / steps
    scan_ms = kms["gdn_chunk_scan"]
    return dict(case=case, T=T, ms_per_step=ms, tokens_per_s=T / (ms / 1e3), kernels_ms=kms,
                path_tflops=F / (ms / 1e3) / 1e12, path_mfma_frac=F / (ms / 1e3) / 1e12 /
                PEAK_BF16_TFLOPS, path_hbm_gbs=B / (ms / 1e3) / 1e9,
                roofline=dict(kernel="gdn_chunk_scan", bound="mfma",
                              achieved=round(Fscan / (scan_ms / 1e3) / 1e12, 3),
                              peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                              frac=round(Fscan / (scan_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 5),
                              traffic=_traffic(f"gdn_chunk_scan_{case.meta['workload']}"),
                              algorithmic_flops_per_launch=Fscan),
                algorithmic=dict(flops=F, bytes=B))


def run_decode(torch, gdn, si, steps, warmup):
    case = si.workload_case(4)
    dev = "cuda"
    d = {k: getattr(case, k).to(dev) for k in ("q", "k", "v", "g", "beta", "h0")}
    state = d["h0"]
    o = torch.empty_like(d["v"])
    N, hqk, dk = case.q.shape
    hv, dv = case.v.shape[1], case.v.shape[2]

    def step(tm=None, i=0):
        if tm:
            tm.mark(i, 0)
        gdn.recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state, o=o)
        if tm:
            tm.mark(i, 1)

    for _ in range(warmup):
        step()
    tm = Timer(torch, ["gdn_recurrent_step"], steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(tm, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = tm.per_kernel_ms()
    B = 2 * N * hv * dk * dv * 4 + N * (hqk * 2 * dk * 2 + hv * (2 * dv * 2 + 8))
    kt = kms["gdn_recurrent_step"] / 1e3
    ms = wall * 1e3 / steps
    return dict(ms_per_step=ms, tokens_per_s=N / (ms / 1e3), kernels_ms=kms,
                roofline=dict(kernel="gdn_recurrent_step", bound="hbm",
                              achieved=round(B / kt / 1e9, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                              frac=round(B / kt / 1e9 / PEAK_HBM_GBS, 4),
                              traffic=_traffic("gdn_recurrent_step_decode_256x1"),
                              algorithmic_bytes_per_launch=B))


def run_front(torch, gdn, si, steps, warmup):
    fc = si.workload_case(5)
    dev = "cuda"
    x, w, a, b = (t.to(dev) for t in (fc.mixed_qkv, fc.conv_weight, fc.a, fc.b))
    A_log, dt_bias, cu, h0 = (t.to(dev) for t in (fc.A_log, fc.dt_bias, fc.cu_seqlens, fc.h0))
    m = fc.meta
    T = x.shape[0]
    n = len(m["lengths"])
    hqk, hv, dk, dv = m["hqk"], m["hv"], m["dk"], m["dv"]
    ws = torch.empty(gdn.workspace_size(T, n, hqk, hv, dk), dtype=torch.uint8, device=dev)
    o = torch.empty((T, hv, dv), dtype=torch.bfloat16, device=dev)
    ht = torch.empty((n, hv, dk, dv), dtype=torch.float32, device=dev)

    def step(tm=None, i=0):
        if tm:
            tm.mark(i, 0)
        q, k, v, g, beta = gdn.prepare(x, w, a, b, A_log, dt_bias, cu, hqk, dk, hv, dv)
        if tm:
            tm.mark(i, 1)
        gdn.chunk_intra(q, k, g, beta, cu, hv, ws)
        if tm:
            tm.mark(i, 2)
        gdn.chunk_scan(q, k, v, g, beta, cu, ws, initial_state=h0, o=o, final_state=ht)
        if tm:
            tm.mark(i, 3)

    for _ in range(warmup):
        step()
    tm = Timer(torch, ["gdn_prepare", "gdn_chunk_intra", "gdn_chunk_scan"], steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(tm, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = tm.per_kernel_ms()
    conv_dim = 2 * hqk * dk + hv * dv
    Bprep = T * (2 * conv_dim * 2 + 2 * hv * 2 + 8 * hv)
    Fscan = scan_flops_per_token_head(dk, dv) * T * hv
    F = prefill_flops_per_token_head(hqk, hv, dk, dv) * T * hv
    ms = wall * 1e3 / steps
    return dict(T=T, lengths=m["lengths"], ms_per_step=ms, tokens_per_s=T / (ms / 1e3),
                kernels_ms=kms, path_tflops=F / (ms / 1e3) / 1e12,
                prepare=dict(bound="hbm", achieved=round(Bprep / (kms["gdn_prepare"] / 1e3) / 1e9, 1),
                             peak=PEAK_HBM_GBS, unit="GB/s",
                             frac=round(Bprep / (kms["gdn_prepare"] / 1e3) / 1e9 / PEAK_HBM_GBS, 4)),
                roofline=dict(kernel="gdn_chunk_scan", bound="mfma",
                              achieved=round(Fscan / (kms["gdn_chunk_scan"] / 1e3) / 1e12, 3),
                              peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                              frac=round(Fscan / (kms["gdn_chunk_scan"] / 1e3) / 1e12 /
                                         PEAK_BF16_TFLOPS, 5)))


def cpu_baseline(case, budget_s=20.0, min_s=3.0):
    """The float64 oracle as it stands on this host, on whole (sequence, V head) chains of the
    prefill workload: whole passes over all V heads are repeated until ~min_s of work (a
    partial pass is scaled if the budget runs out first); tokens/s for the whole layer."""
    import numpy as np  # noqa: F401

    import oracle

    f64 = lambda t: t.double().numpy()  # noqa: E731
    T, hqk, dk = case.q.shape
    hv = case.v.shape[1]
    G = hv // hqk
    threads = oracle.num_threads()
    heads_total, t_spent, passes = 0, 0.0, 0
    while t_spent < min_s and t_spent < budget_s:
        # One oracle call over a group of V heads (threads chains at once).
        heads_done = 0
        while heads_done < hv and t_spent < budget_s:
            hs = list(range(heads_done, min(hv, heads_done + max(1, threads))))
            ms = sorted({h // G for h in hs})
            # keep the h -> h // G mapping by taking whole QK groups
            q = f64(case.q[:, ms[0]:ms[-1] + 1])
            k = f64(case.k[:, ms[0]:ms[-1] + 1])
            h_lo, h_hi = ms[0] * G, (ms[-1] + 1) * G
            v = f64(case.v[:, h_lo:h_hi])
            g = f64(case.g[:, h_lo:h_hi])
            b = f64(case.beta[:, h_lo:h_hi])
            t0 = time.perf_counter()
            oracle.recurrent(q, k, v, g, b, case.cu_seqlens.numpy(), output_final_state=True)
            t_spent += time.perf_counter() - t0
            heads_done = h_hi
        heads_total += heads_done
        passes += 1
    per_layer_s = t_spent * hv / heads_total
    return dict(value=round(T / per_layer_s, 2), unit="tokens/s", cores=threads, kind="oracle",
                sample=f"workload prefill_35b_a3b_1x4096: {heads_total} V-head chains of {T} "
                       f"tokens ({passes} pass(es) over the {hv} heads) in {t_spent:.1f} s on "
                       f"{threads} threads, scaled to one layer of {hv} heads",
                wall_s=round(t_spent, 2),
                host_cpu_count=os.cpu_count(),
                affinity=len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None)


def main():
    args = _parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the Gated DeltaNet core "
                          "has no cross-GPU step here; run with --gpus 1"}))
        sys.exit(2)
    import torch

    import gated_deltanet_linear_amd as gdn
    import synthetic_inputs as si

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}))
        return
    out = {}
    only = args.only
    pre = None
    if only in (None, "prefill"):
        pre = run_prefill(torch, gdn, si, 2, args.steps, args.warmup, with_h0=False)
    if only in (None, "decode"):
        out["decode"] = run_decode(torch, gdn, si, args.steps, args.warmup)
    if only in (None, "long"):
        lg = run_prefill(torch, gdn, si, 3, max(3, args.steps // 10), 2, with_h0=True)
        lg.pop("case")
        out["long_context_4x32768"] = lg
    if only in (None, "front"):
        out["front_end_packed_8_seqs"] = run_front(torch, gdn, si, max(3, args.steps // 5), 2)

    line = {"metric": "GDN prefill tokens/s (1 MI355X; decode tokens/s alongside)",
            "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic"}
    if pre is not None:
        case = pre.pop("case")
        line.update(value=round(pre["tokens_per_s"], 1), ms_per_step=round(pre["ms_per_step"], 5),
                    config={"workload": "prefill_35b_a3b_1x4096", "num_seqs": 1, "seq_len": 4096,
                            "num_qk_heads": 16, "num_v_heads": 32, "head_dim": 128, "chunk": 64,
                            "qkv_dtype": "bf16", "out_dtype": "bf16", "state_dtype": "f32",
                            "initial_state": False, "final_state": True},
                    roofline=pre["roofline"], kernels_ms=pre["kernels_ms"],
                    path=dict(tflops=round(pre["path_tflops"], 3),
                              mfma_frac=round(pre["path_mfma_frac"], 5),
                              hbm_gbs=round(pre["path_hbm_gbs"], 1), **pre["algorithmic"]))
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline(case)
    else:
        k0 = next(iter(out))
        line.update(value=round(out[k0]["tokens_per_s"], 1), ms_per_step=out[k0]["ms_per_step"],
                    config={"workload": k0}, roofline=out[k0]["roofline"])
    line.update(out)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
