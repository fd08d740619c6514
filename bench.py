"""Benchmark of the Gated DeltaNet core on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--only NAME]

Prints ONE JSON line. The headline ``value`` is prefill tokens/s of the long-context workload,
the largest single-GPU configuration: 4 sequences x 32768 tokens of the 35B-A3B-shaped GDN layer
(16 QK / 32 V heads, d = 128, bf16 q/k/v, fp32 initial states given and final states returned).
One step is one gdn_chunk_forward (its two kernels, gdn_chunk_intra then gdn_chunk_scan) over
inputs already resident in HBM; W untimed steps, then exactly K timed steps. The same line
carries, as extra keys: the 1 x 4096 prefill, decode tokens/s (256 sequences x 1 token, 537 MB
fp32 state updated in place), the packed front-end workload, the output gate (1 x 4096 shape), a
decode step from projected inputs (fused front end + recurrent step, 256 sequences), the
backward of the 1 x 4096 prefill, per-kernel HIP-event timings, the roofline of each workload's
dominant kernel and the float64 CPU oracle timed on a bounded sample of the headline workload
on this host.

Roofline conventions (algorithmic work, not what the kernels happen to issue):
  prefill FLOPs per token per V head = (4/G) C d_k + 2 C d_k + 4 C d_v + 6 d_k d_v   (C = 64)
    of which the scan kernel's share is 4 C d_v + 6 d_k d_v (state products, T diag(beta) Y
    and the masked intra-chunk product); peak = 2500 TFLOP/s dense bf16 MFMA.
  decode bytes = 2 N H_v d_k d_v s + N [H_qk 2 d_k e + H_v (2 d_v e + 8)];  peak 8000 GB/s
    (s = 4 for the fp32 state, 2 for the bf16 state).
  front-end bytes = T [conv_dim e + 2 H_v e + 8 H_v + conv_dim e_qkv]  (mixed_qkv and a, b
    read, g and beta written, q / k / v written at their dtype e_qkv).
  output-gate bytes = 3 T H_v d_v e + 4 d_v   (o and z read, out written, fp32 weight).
  decode front-end bytes = N [8 conv_dim e + H_v (2 e + 8)] + 4 conv_dim e   (x, window read
    and rewritten, q/k/v written; a, b in, g, beta out; taps once).
  fused decode-step bytes = 2 N H_v d_k d_v 4 + N [7 conv_dim e + H_v (2 e + d_v e)]
    + 4 conv_dim e   (state read and written; x, window read and rewritten; a, b; o; taps).
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
PEAK_F32_TFLOPS = 157.3  # dense fp32 MFMA
PEAK_HBM_GBS = 8000.0
C = 64


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None,
                    help="run one workload: prefill, decode, long, front, gate, decode_front, backward")
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


def scan_bytes(lengths, hqk, hv, dk, dv, e, h0_given, state_out=True, eo=None):
    """Algorithmic HBM bytes of one scan launch: q and k (each unique byte once), v (e bytes an
    element), the workspace records the intra kernel wrote (20992 bytes per chunk and V head),
    the initial states, o (eo bytes an element, e unless given) and the final states."""
    T = sum(lengths)
    n = len(lengths)
    chunks = sum((L + C - 1) // C for L in lengths)
    eo = e if eo is None else eo
    b = T * (hqk * 2 * dk * e + hv * dv * (e + eo)) + chunks * hv * 20992
    b += n * hv * dk * dv * 4 * ((1 if state_out else 0) + (1 if h0_given else 0))
    return b


def _sha(rel):
    path = os.path.join(ROOT, rel)
    return hashlib.sha256(open(path, "rb").read()).hexdigest() if os.path.exists(path) else None


def _traffic(kernel_key):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was taken on the
    current sources of that kernel (every file the record lists, by SHA-256); else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_key}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if "sources" in rec:
        if any(_sha(f) != h for f, h in rec["sources"].items()):
            return None
    elif _sha(rec["source"]) != rec.get("source_sha256"):
        return None
    return rec.get("hbm_bytes_per_launch")


def _measure(torch, kernels, steps, warmup):
    """Time one leg. ``kernels`` lists (name, launch) in step order; a step launches each once.

    Step time: W untimed steps, then K steps between two HIP events on the launch stream
    (torch's current stream; the library launches on it), bracketed by synchronizes.
    Per-kernel average launch duration: for each kernel, K launches back to back between two
    HIP events on the same stream, divided by K. A spin kernel placed before the first event
    keeps the GPU busy until the host has queued all K launches, so that the host's own call
    overhead (which exceeds the run time of the smaller kernels) is not timed. (An event pair
    around every single launch would add the dispatch latency of the event markers, several
    microseconds, to each launch.) The kernels' inputs stay valid across repeated launches;
    in-place state is updated each time."""
    stream = torch.cuda.current_stream()

    def step():
        for _, fn in kernels:
            fn()

    for _ in range(warmup):
        step()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    a.record(stream)
    for _ in range(steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    step_ms = a.elapsed_time(b) / steps
    # cycles of the spin kernel per millisecond
    torch.cuda.synchronize()
    a.record(stream)
    torch.cuda._sleep(1_000_000)
    b.record(stream)
    torch.cuda.synchronize()
    cycles_per_ms = 1_000_000 / max(a.elapsed_time(b), 1e-3)
    kms = {}
    for name, fn in kernels:
        # host time to queue K launches (queuing does not wait for the GPU), then a hold just
        # longer than that: a long idle hold lets the clocks drop before the timed launches
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        queue_ms = (time.perf_counter() - t0) * 1e3
        torch.cuda.synchronize()
        torch.cuda._sleep(int(cycles_per_ms * (1.5 * queue_ms + 0.05)))
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        kms[name] = a.elapsed_time(b) / steps
    return step_ms, wall_ms, kms


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

    kernels = [
        ("gdn_chunk_intra",
         lambda: gdn.chunk_intra(d["q"], d["k"], d["g"], d["beta"], d["cu_seqlens"], hv, ws)),
        ("gdn_chunk_scan",
         lambda: gdn.chunk_scan(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], ws,
                                initial_state=h0, o=o, final_state=ht)),
    ]
    ev_ms, ms, kms = _measure(torch, kernels, steps, warmup)
    lengths = case.meta["lengths"]
    F = prefill_flops_per_token_head(hqk, hv, dk, dv) * T * hv
    Fscan = scan_flops_per_token_head(dk, dv) * T * hv
    B = prefill_bytes(lengths, hqk, hv, dk, dv, 2, with_h0)
    Bscan = scan_bytes(lengths, hqk, hv, dk, dv, 2, with_h0)
    scan_ms = kms["gdn_chunk_scan"]
    return dict(case=case, T=T, ms_per_step=ms, step_ms_events=ev_ms,
                tokens_per_s=T / (ms / 1e3), kernels_ms=kms,
                path_tflops=F / (ms / 1e3) / 1e12, path_mfma_frac=F / (ms / 1e3) / 1e12 /
                PEAK_BF16_TFLOPS, path_hbm_gbs=B / (ms / 1e3) / 1e9,
                roofline=dict(kernel="gdn_chunk_scan", bound="mfma",
                              achieved=round(Fscan / (scan_ms / 1e3) / 1e12, 3),
                              peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                              frac=round(Fscan / (scan_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 5),
                              traffic=_traffic(f"gdn_chunk_scan_{case.meta['workload']}"),
                              algorithmic_flops_per_launch=Fscan,
                              algorithmic_bytes_per_launch=Bscan,
                              hbm_gbs=round(Bscan / (scan_ms / 1e3) / 1e9, 1),
                              hbm_frac=round(Bscan / (scan_ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4)),
                algorithmic=dict(flops=F, bytes=B))


def run_decode(torch, gdn, si, steps, warmup):
    case = si.workload_case(4)
    dev = "cuda"
    d = {k: getattr(case, k).to(dev) for k in ("q", "k", "v", "g", "beta", "h0")}
    state = d["h0"]
    o = torch.empty_like(d["v"])
    N, hqk, dk = case.q.shape
    hv, dv = case.v.shape[1], case.v.shape[2]

    kernels = [("gdn_recurrent_step",
                lambda: gdn.recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state,
                                           o=o))]
    ev_ms, ms, kms = _measure(torch, kernels, steps, warmup)
    B = 2 * N * hv * dk * dv * 4 + N * (hqk * 2 * dk * 2 + hv * (2 * dv * 2 + 8))
    kt = kms["gdn_recurrent_step"] / 1e3
    # the same step on a bf16 state (half the state bytes)
    state16 = state.to(torch.bfloat16)
    del state
    ev16, ms16, kms16 = _measure(
        torch, [("gdn_recurrent_step",
                 lambda: gdn.recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state16,
                                            o=o))], steps, warmup)
    B16 = 2 * N * hv * dk * dv * 2 + N * (hqk * 2 * dk * 2 + hv * (2 * dv * 2 + 8))
    bf16_state = dict(ms_per_step=ms16, tokens_per_s=N / (ms16 / 1e3), kernels_ms=kms16,
                      roofline=_hbm("gdn_recurrent_step", B16, kms16["gdn_recurrent_step"],
                                    "gdn_recurrent_step_decode_256x1_bf16_state"))
    del state16
    return dict(ms_per_step=ms, step_ms_events=ev_ms, tokens_per_s=N / (ms / 1e3),
                kernels_ms=kms, bf16_state=bf16_state,
                roofline=dict(kernel="gdn_recurrent_step", bound="hbm",
                              achieved=round(B / kt / 1e9, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                              frac=round(B / kt / 1e9 / PEAK_HBM_GBS, 4),
                              traffic=_traffic("gdn_recurrent_step_decode_256x1"),
                              algorithmic_bytes_per_launch=B))


def run_front(torch, gdn, si, steps, warmup, split=True):
    """Workload 5 (8 packed sequences, 16 QK / 64 V heads, d = 128, bf16 projected inputs,
    initial states): gdn_prepare then the chunked core, exactly the call sequence the end-to-end
    parity test checks. q, k and v cross from the front end to the core in fp32: rounding them
    to bf16 there moves the result ~15% x RMS away from the float64 front end + core on this
    workload (its conv makes neighbouring keys nearly collinear), so the bf16 intermediates do
    not meet the bf16 bar. ``split``: the core takes them on the split-bf16 MFMA path
    (split_f32); else on the fp32-MFMA path."""
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
    qkv_dtype = torch.float32

    qkv = {}

    def prep():
        qkv["t"] = gdn.prepare(x, w, a, b, A_log, dt_bias, cu, hqk, dk, hv, dv,
                               qkv_dtype=qkv_dtype)

    def intra():
        q, k, v, g, beta = qkv["t"]
        gdn.chunk_intra(q, k, g, beta, cu, hv, ws, split_f32=split)

    def scan():
        q, k, v, g, beta = qkv["t"]
        gdn.chunk_scan(q, k, v, g, beta, cu, ws, initial_state=h0, o=o, final_state=ht,
                       split_f32=split)

    ev_ms, ms, kms = _measure(
        torch, [("gdn_prepare", prep), ("gdn_chunk_intra", intra), ("gdn_chunk_scan", scan)],
        steps, warmup)
    conv_dim = 2 * hqk * dk + hv * dv
    eq = 4 if qkv_dtype == torch.float32 else 2
    # mixed_qkv read, a and b read, g and beta written, q / k / v written at their dtype
    Bprep = T * (conv_dim * 2 + 2 * hv * 2 + 8 * hv + conv_dim * eq)
    Fscan = scan_flops_per_token_head(dk, dv) * T * hv
    F = prefill_flops_per_token_head(hqk, hv, dk, dv) * T * hv
    peak = PEAK_F32_TFLOPS if qkv_dtype == torch.float32 and not split else PEAK_BF16_TFLOPS
    Bscan = scan_bytes(m["lengths"], hqk, hv, dk, dv, eq, True, eo=2)
    return dict(T=T, lengths=m["lengths"], ms_per_step=ms, step_ms_events=ev_ms,
                tokens_per_s=T / (ms / 1e3), qkv_dtype=str(qkv_dtype).replace("torch.", ""),
                core_products="split-bf16 MFMA" if split else "fp32 MFMA",
                kernels_ms=kms, path_tflops=F / (ms / 1e3) / 1e12,
                prepare=_hbm("gdn_prepare", Bprep, kms["gdn_prepare"],
                             "gdn_prepare_prefill_397b_packed_8xU512_8192_f32qkv"),
                roofline=dict(kernel="gdn_chunk_scan", bound="mfma",
                              achieved=round(Fscan / (kms["gdn_chunk_scan"] / 1e3) / 1e12, 3),
                              peak=peak, unit="TFLOP/s",
                              frac=round(Fscan / (kms["gdn_chunk_scan"] / 1e3) / 1e12 / peak, 5),
                              traffic=_traffic("gdn_chunk_scan_prefill_397b_packed_8xU512_8192"
                                               + ("_f32qkv" if eq == 4 else "")
                                               + ("_split" if split else "")),
                              algorithmic_flops_per_launch=Fscan,
                              algorithmic_bytes_per_launch=Bscan,
                              hbm_gbs=round(Bscan / (kms["gdn_chunk_scan"] / 1e3) / 1e9, 1)))


def _hbm(kernel, nbytes, ms, traffic_key=None):
    gbs = nbytes / (ms / 1e3) / 1e9
    return dict(kernel=kernel, bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS,
                unit="GB/s", frac=round(gbs / PEAK_HBM_GBS, 4),
                traffic=_traffic(traffic_key) if traffic_key else None,
                algorithmic_bytes_per_launch=nbytes)


def run_gate(torch, gdn, si, steps, warmup):
    """Output gate over the 1 x 4096 prefill shape (4096 tokens x 32 V heads x 128, bf16)."""
    gc = si.make_gate_case(4096, 32, 128, seed=1006, meta=dict(workload="output_gate_1x4096"))
    o, z, w = gc.o.cuda(), gc.z.cuda(), gc.weight.cuda()
    out = torch.empty_like(o)
    T, hv, dv = o.shape

    ev_ms, ms, kms = _measure(
        torch, [("gdn_gated_rmsnorm", lambda: gdn.gated_rmsnorm(o, z, w, 1.0, 1e-6, out=out))],
        steps, warmup)
    B = T * hv * dv * 2 * 3 + dv * 4
    return dict(ms_per_step=ms, step_ms_events=ev_ms, tokens_per_s=T / (ms / 1e3),
                kernels_ms=kms, roofline=_hbm("gdn_gated_rmsnorm", B, kms["gdn_gated_rmsnorm"],
                              "gdn_gated_rmsnorm_output_gate_1x4096"))


def run_decode_front(torch, gdn, si, steps, warmup):
    """One decode token for 256 sequences from projected inputs (35B-A3B layer shape, bf16
    inputs, fp32 state updated in place): the fused gdn_decode_step, and for comparison the
    two-call path gdn_decode_prepare then gdn_recurrent_step; with the layer's output gate,
    gdn_decode_step_gated (one kernel) against gdn_decode_step then gdn_gated_rmsnorm."""
    dc = si.make_decode_front_case(256, 16, 32, 128, 128, seed=1007,
                                   meta=dict(workload="decode_front_256x1"))
    dev = "cuda"
    x, win, w, a, b = (t.to(dev) for t in (dc.mixed_qkv, dc.window, dc.conv_weight, dc.a, dc.b))
    A_log, dt_bias, state = dc.A_log.to(dev), dc.dt_bias.to(dev), dc.h0.to(dev)
    m = dc.meta
    N, hqk, hv, dk, dv = m["N"], m["hqk"], m["hv"], m["dk"], m["dv"]
    o = torch.empty((N, hv, dv), dtype=torch.bfloat16, device=dev)

    ev_ms, ms, kms = _measure(
        torch, [("gdn_decode_step", lambda: gdn.decode_step(x, win, w, a, b, A_log, dt_bias,
                                                            state, hqk, dk, hv, o=o))],
        steps, warmup)

    qkv = {}

    def prep():
        qkv["t"] = gdn.decode_prepare(x, win, w, a, b, A_log, dt_bias, hqk, dk, hv, dv)

    def rstep():
        q, k, v, g, beta = qkv["t"]
        gdn.recurrent_step(q, k, v, g, beta, state, o=o)

    ev2, ms2, kms2 = _measure(
        torch, [("gdn_decode_prepare", prep), ("gdn_recurrent_step", rstep)], steps, warmup)
    # the layer's output gate: fused into the step (one kernel) and as the step + gate kernel
    gen = torch.Generator().manual_seed(1008)
    z = torch.randn((N, hv, dv), generator=gen).to(torch.bfloat16).to(dev)
    gw = (0.1 * torch.randn((dv,), generator=gen)).to(dev)
    out = torch.empty_like(o)
    ev4, ms4, kms4 = _measure(
        torch, [("gdn_decode_step_gated",
                 lambda: gdn.decode_step_gated(x, win, w, a, b, A_log, dt_bias, state, z, hqk, dk,
                                               hv, weight=gw, weight_offset=1.0, out=out))],
        steps, warmup)
    ev5, ms5, kms5 = _measure(
        torch, [("gdn_decode_step", lambda: gdn.decode_step(x, win, w, a, b, A_log, dt_bias,
                                                            state, hqk, dk, hv, o=o)),
                ("gdn_gated_rmsnorm", lambda: gdn.gated_rmsnorm(o, z, gw, 1.0, 1e-6, out=out))],
        steps, warmup)
    del z, gw, out
    state16 = state.to(torch.bfloat16)
    del state
    ev3, ms3, kms3 = _measure(
        torch, [("gdn_decode_step", lambda: gdn.decode_step(x, win, w, a, b, A_log, dt_bias,
                                                            state16, hqk, dk, hv, o=o))],
        steps, warmup)
    del state16
    conv_dim = 2 * hqk * dk + hv * dv
    e = 2
    Bfused = (2 * N * hv * dk * dv * 4 + N * (conv_dim * e * 7 + hv * (2 * e + dv * e))
              + conv_dim * 4 * e)
    Bfused16 = Bfused - N * hv * dk * dv * 4
    Bprep = N * (conv_dim * e * 8 + hv * (2 * e + 8)) + conv_dim * 4 * e
    Bstep = 2 * N * hv * dk * dv * 4 + N * (hqk * 2 * dk * e + hv * (2 * dv * e + 8))
    return dict(ms_per_step=ms, step_ms_events=ev_ms, tokens_per_s=N / (ms / 1e3),
                kernels_ms=kms,
                roofline=_hbm("gdn_decode_step", Bfused, kms["gdn_decode_step"],
                              "gdn_decode_step_decode_front_256x1"),
                bf16_state=dict(ms_per_step=ms3, tokens_per_s=N / (ms3 / 1e3), kernels_ms=kms3,
                                roofline=_hbm("gdn_decode_step", Bfused16, kms3["gdn_decode_step"],
                                              "gdn_decode_step_decode_front_256x1_bf16_state")),
                gated=dict(ms_per_step=ms4, tokens_per_s=N / (ms4 / 1e3), kernels_ms=kms4,
                           roofline=_hbm("gdn_decode_step_gated", Bfused + N * hv * dv * e + dv * 4,
                                         kms4["gdn_decode_step_gated"],
                                         "gdn_decode_step_gated_decode_front_256x1"),
                           unfused=dict(ms_per_step=ms5, tokens_per_s=N / (ms5 / 1e3),
                                        kernels_ms=kms5)),
                two_call=dict(ms_per_step=ms2, tokens_per_s=N / (ms2 / 1e3), kernels_ms=kms2,
                              decode_prepare=_hbm("gdn_decode_prepare", Bprep,
                                                  kms2["gdn_decode_prepare"],
                                                  "gdn_decode_prepare_decode_front_256x1"),
                              recurrent_step=_hbm("gdn_recurrent_step", Bstep,
                                                  kms2["gdn_recurrent_step"],
                                                  "gdn_recurrent_step_decode_256x1")))


def backward_flops_per_token_head(dk, dv):
    """Algorithmic MACs x 2 of the backward per token per V head (d = d_k = d_v, C = 64): the
    intra products (K K^T, Q K^T: 2 C d), the state recomputation (K H, T Y, K^T V': 2 d^2 + C d),
    the reverse scan (K dH', P^T dO, T^T dV', Q^T dO, K^T dY: 3 d^2 + 2 C d) and the gradient
    products (dO H^T, dY H^T, V' dH'^T: 3 d^2; dO V'^T, Z V'^T, (dP o G) K, (dP o G)^T Q,
    (dS + dS^T) K: 5 C d)."""
    d = dk
    return 2 * (8 * d * d + 10 * C * d)


def backward_bytes(T, hqk, hv, dk, dv, e):
    """Algorithmic HBM bytes of one backward call without initial or final states: q, k, v and
    dout read and dq, dk, dv written once (e bytes an element), g and beta read and dg, dbeta
    written in fp32."""
    return T * (2 * (hqk * 2 * dk * e + hv * 2 * dv * e) + 16 * hv)


def run_backward(torch, gdn, si, steps, warmup):
    """Backward of the 1 x 4096 prefill (gdn_chunk_backward: dq, dk, dv, dg, dbeta and dh0 from a
    bf16 output gradient), inputs resident in HBM, workspace preallocated."""
    case = si.workload_case(2)
    dev = "cuda"
    d = {k: getattr(case, k).to(dev) for k in ("q", "k", "v", "g", "beta", "cu_seqlens")}
    T, hqk, dk = case.q.shape
    hv, dv = case.v.shape[1], case.v.shape[2]
    gen = torch.Generator(device="cpu").manual_seed(1008)
    dout = torch.randn((T, hv, dv), generator=gen).to(torch.bfloat16).to(dev)
    nbytes = gdn.backward_workspace_size(T, 1, hqk, hv, dk)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def step():
        gdn.chunk_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], dout,
                           workspace=ws)

    ev_ms, ms, kms = _measure(torch, [("gdn_chunk_backward", step)], steps, warmup)
    F = backward_flops_per_token_head(dk, dv) * T * hv
    Bb = backward_bytes(T, hqk, hv, dk, dv, 2)
    tf = F / (kms["gdn_chunk_backward"] / 1e3) / 1e12
    return dict(ms_per_step=ms, step_ms_events=ev_ms, tokens_per_s=T / (ms / 1e3),
                kernels_ms=kms, workspace_bytes=nbytes,
                roofline=dict(kernel="gdn_chunk_backward (3 launches)", bound="mfma",
                              achieved=round(tf, 3), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                              frac=round(tf / PEAK_BF16_TFLOPS, 5),
                              traffic=_traffic("gdn_chunk_backward_backward_1x4096"),
                              algorithmic_flops_per_launch=F,
                              algorithmic_bytes_per_launch=Bb,
                              note="bf16 inputs: most products on bf16 MFMA (computed operands "
                                   "as hi + lo pairs), the C x C dP and dA products on fp32 "
                                   "MFMA; priced against the bf16 dense peak"))


def cpu_baseline(case, budget_s=30.0, min_s=10.0):
    """The float64 oracle as it stands on this host, on whole (sequence, V head) chains of a
    prefill workload: chains are taken in order (sequence-major, all V heads of a sequence with
    their QK heads) in groups of one per thread until about min_s of work (or the budget) is
    spent; tokens/s for the whole layer is scaled from the chain-tokens done."""
    import numpy as np

    import oracle

    f64 = lambda t: t.double().numpy()  # noqa: E731
    T, hqk, dk = case.q.shape
    hv = case.v.shape[1]
    G = hv // hqk
    cu = case.cu_seqlens.numpy().astype(np.int64)
    n_seqs = len(cu) - 1
    threads = oracle.num_threads()
    chain_tokens_total = int(sum((cu[n + 1] - cu[n]) * hv for n in range(n_seqs)))
    done_tokens, chains, t_spent = 0, 0, 0.0
    n, h0 = 0, 0
    while t_spent < min_s and t_spent < budget_s and n < n_seqs:
        # one oracle call over up to `threads` V heads of sequence n (whole QK groups)
        h1 = min(hv, h0 + max(G, (threads // G) * G))
        s0, s1 = int(cu[n]), int(cu[n + 1])
        q = f64(case.q[s0:s1, h0 // G:h1 // G])
        k = f64(case.k[s0:s1, h0 // G:h1 // G])
        v = f64(case.v[s0:s1, h0:h1])
        g = f64(case.g[s0:s1, h0:h1])
        b = f64(case.beta[s0:s1, h0:h1])
        init = None if case.h0 is None else f64(case.h0[n:n + 1, h0:h1])
        t0 = time.perf_counter()
        oracle.recurrent(q, k, v, g, b, [0, s1 - s0], initial_state=init,
                         output_final_state=True)
        t_spent += time.perf_counter() - t0
        done_tokens += (s1 - s0) * (h1 - h0)
        chains += h1 - h0
        h0 = h1
        if h0 >= hv:
            n, h0 = n + 1, 0
    per_layer_s = t_spent * chain_tokens_total / done_tokens
    return dict(value=round(T / per_layer_s, 2), unit="tokens/s", cores=threads, kind="oracle",
                sample=f"workload {case.meta['workload']}: {chains} (sequence, V head) chains, "
                       f"{done_tokens} chain-tokens of the layer's {chain_tokens_total}, in "
                       f"{t_spent:.1f} s on {threads} threads, scaled to the whole layer",
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
    lg = None
    if only in (None, "long"):
        lg = run_prefill(torch, gdn, si, 3, args.steps, args.warmup, with_h0=True)
    if only in (None, "prefill"):
        pre = run_prefill(torch, gdn, si, 2, args.steps, args.warmup, with_h0=False)
        pre.pop("case")
        out["prefill_35b_a3b_1x4096"] = pre
    if only in (None, "decode"):
        out["decode"] = run_decode(torch, gdn, si, args.steps, args.warmup)
    if only in (None, "front"):
        out["front_end_packed_8_seqs"] = run_front(torch, gdn, si, max(3, args.steps // 5), 2)
        f32 = run_front(torch, gdn, si, max(3, args.steps // 5), 2, split=False)
        out["front_end_packed_8_seqs"]["fp32_mfma_core"] = {
            k: f32[k] for k in ("ms_per_step", "kernels_ms", "roofline")}
    if only in (None, "gate"):
        out["output_gate_1x4096"] = run_gate(torch, gdn, si, args.steps, args.warmup)
    if only in (None, "backward"):
        out["backward_1x4096"] = run_backward(torch, gdn, si, max(3, args.steps // 5), 2)
    if only in (None, "decode_front"):
        out["decode_front_256x1"] = run_decode_front(torch, gdn, si, args.steps, args.warmup)

    line = {"metric": "GDN prefill tokens/s (1 MI355X; decode tokens/s alongside)",
            "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic"}
    if lg is not None:
        case = lg.pop("case")
        line.update(value=round(lg["tokens_per_s"], 1), ms_per_step=round(lg["ms_per_step"], 5),
                    config={"workload": "prefill_long_4x32768", "num_seqs": 4, "seq_len": 32768,
                            "num_qk_heads": 16, "num_v_heads": 32, "head_dim": 128, "chunk": 64,
                            "qkv_dtype": "bf16", "out_dtype": "bf16", "state_dtype": "f32",
                            "initial_state": True, "final_state": True},
                    roofline=lg["roofline"], kernels_ms=lg["kernels_ms"],
                    path=dict(tflops=round(lg["path_tflops"], 3),
                              mfma_frac=round(lg["path_mfma_frac"], 5),
                              hbm_gbs=round(lg["path_hbm_gbs"], 1), **lg["algorithmic"]))
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
