"""GPU parity of gdn_chunk_forward (chunked prefill) against the float64 oracle.

Every case compares the fp32 output and the final states element by element with
max|err| <= tol * RMS(reference), tol = 1e-4 for fp32 inputs and 2e-2 for bf16 inputs.
"""

import numpy as np
import pytest
import torch

import gated_deltanet_linear_amd as gdn
import synthetic_inputs as si
from gdn_testutil import TOL, assert_rms_close, f64, oracle_case, to_dev

pytestmark = pytest.mark.gpu


def _run(case, out_dtype=torch.float32, scale=1.0, with_h0=True):
    d = to_dev(case)
    o, ht = gdn.chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                              initial_state=d["h0"] if with_h0 else None, scale=scale,
                              out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o, ht


def _check(case, label, scale=1.0):
    tol = TOL[case.meta["dtype"]]
    print(f"[chunk] {label} lengths={case.meta['lengths'][:8]} dtype={case.meta['dtype']}",
          flush=True)
    o, ht = _run(case, scale=scale)
    o_ref, h_ref = oracle_case(case)
    assert_rms_close(o, scale * o_ref if scale != 1.0 else o_ref, tol, f"{label} o")
    assert_rms_close(ht, h_ref, tol, f"{label} final state")


def test_tiny_fp32_workload():
    """Workload 1: 1 x 256 tokens, 1/1 heads, d = 32, fp32."""
    _check(si.workload_case(1), "tiny_fp32")


@pytest.mark.parametrize("T", [1, 63, 64, 65, 127, 130, 300])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_ragged_lengths_bf16(T, d):
    case = si.make_core_case([T], 2, 4, d, d, dtype="bf16", gate="model", h0_std=0.02,
                             seed=10 * T + d)
    _check(case, f"bf16 T={T} d={d}")


@pytest.mark.parametrize("T", [1, 65, 200])
@pytest.mark.parametrize("d", [32, 128])
def test_ragged_lengths_fp32(T, d):
    case = si.make_core_case([T], 1, 2, d, d, dtype="f32", gate="uniform", g_low=-0.1,
                             h0_std=0.5, seed=3 * T + d)
    _check(case, f"fp32 T={T} d={d}")


def test_varlen_with_empty_sequences_and_states():
    case = si.make_core_case([0, 1, 64, 100, 257, 5, 0, 130], 2, 4, 128, 128, dtype="bf16",
                             gate="model", h0_std=0.05, seed=77)
    _check(case, "varlen")


def test_gqa_four_v_heads_per_qk_head():
    case = si.make_core_case([200, 77], 2, 8, 128, 128, dtype="bf16", gate="model", h0_std=0.02,
                             seed=5)
    _check(case, "gqa G=4")


def test_slow_decay_state_propagation():
    """Slow decay (g ~ U(-0.01, 0)) keeps the initial state and state from hundreds of chunks
    back visible in the output, unlike the fast model gates."""
    case = si.slow_decay_case([1500, 700], 2, 4, 128, 128, dtype="bf16", seed=9)
    _check(case, "slow decay")


def test_slow_decay_fp32():
    case = si.slow_decay_case([600], 1, 1, 32, 32, dtype="f32", seed=19)
    _check(case, "slow decay fp32")


def test_scale_is_linear():
    case = si.make_core_case([150], 1, 2, 128, 128, dtype="bf16", gate="model", h0_std=0.02,
                             seed=8)
    _check(case, "scale 0.37", scale=0.37)


def test_bf16_output_is_rounded_fp32_output():
    case = si.make_core_case([300, 64], 2, 4, 128, 128, dtype="bf16", gate="model", h0_std=0.02,
                             seed=12)
    o32, h32 = _run(case, out_dtype=torch.float32)
    o16, h16 = _run(case, out_dtype=torch.bfloat16)
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.equal(h16, h32)


def test_state_handoff_split_prefill():
    """chunk_forward(T1) -> final -> chunk_forward(rest, initial=final) ~ chunk_forward(T)."""
    case = si.slow_decay_case([333], 2, 4, 128, 128, dtype="bf16", seed=21)
    T1 = 150
    d = to_dev(case)
    cu1 = torch.tensor([0, T1], dtype=torch.int32, device="cuda")
    cu2 = torch.tensor([0, 333 - T1], dtype=torch.int32, device="cuda")
    sl1, sl2 = slice(0, T1), slice(T1, 333)
    o1, h1 = gdn.chunk_forward(d["q"][sl1].contiguous(), d["k"][sl1].contiguous(),
                               d["v"][sl1].contiguous(), d["g"][sl1].contiguous(),
                               d["beta"][sl1].contiguous(), cu1, initial_state=d["h0"],
                               out_dtype=torch.float32)
    o2, h2 = gdn.chunk_forward(d["q"][sl2].contiguous(), d["k"][sl2].contiguous(),
                               d["v"][sl2].contiguous(), d["g"][sl2].contiguous(),
                               d["beta"][sl2].contiguous(), cu2, initial_state=h1,
                               out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle_case(case)
    assert_rms_close(torch.cat([o1, o2]), o_ref, TOL["bf16"], "handoff o")
    assert_rms_close(h2, h_ref, TOL["bf16"], "handoff final state")


def test_final_state_in_place():
    case = si.make_core_case([190, 3], 2, 4, 128, 128, dtype="bf16", gate="model", h0_std=0.02,
                             seed=31)
    d = to_dev(case)
    state = d["h0"].clone()
    o, ht = gdn.chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                              initial_state=state, final_state=state, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle_case(case)
    assert ht.data_ptr() == state.data_ptr()
    assert_rms_close(o, o_ref, TOL["bf16"], "in-place o")
    assert_rms_close(state, h_ref, TOL["bf16"], "in-place state")


def test_no_final_state_and_zero_initial_state():
    case = si.make_core_case([129], 1, 2, 128, 128, dtype="bf16", gate="model", seed=41)
    d = to_dev(case)
    o, ht = gdn.chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                              output_final_state=False, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert ht is None
    o_ref, _ = oracle_case(case)
    assert_rms_close(o, o_ref, TOL["bf16"], "no-final o")


def test_all_sequences_empty():
    case = si.make_core_case([0, 0], 1, 2, 128, 128, dtype="bf16", gate="model", h0_std=0.1,
                             seed=2)
    o, ht = _run(case)
    assert o.shape[0] == 0
    assert torch.equal(ht.cpu(), case.h0)


def test_stages_equal_chunk_forward():
    """gdn_chunk_intra + gdn_chunk_scan == gdn_chunk_forward bit for bit."""
    case = si.make_core_case([260, 70], 2, 4, 128, 128, dtype="bf16", gate="model", h0_std=0.02,
                             seed=51)
    d = to_dev(case)
    o_ref, h_ref = _run(case)
    T, n = case.q.shape[0], 2
    ws = torch.empty(gdn.workspace_size(T, n, 2, 4, 128), dtype=torch.uint8, device="cuda")
    gdn.chunk_intra(d["q"], d["k"], d["g"], d["beta"], d["cu_seqlens"], 4, ws)
    ht = torch.empty_like(d["h0"])
    o, _ = gdn.chunk_scan(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], ws,
                          initial_state=d["h0"], final_state=ht, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(ht, h_ref)


def test_prefill_then_decode_equals_longer_prefill():
    """chunk_forward(T) then recurrent_step(token T) ~ chunk_forward(T + 1) (both vs oracle)."""
    case = si.slow_decay_case([97], 2, 4, 128, 128, dtype="bf16", seed=61)
    d = to_dev(case)
    T = 96
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    o1, h1 = gdn.chunk_forward(d["q"][:T].contiguous(), d["k"][:T].contiguous(),
                               d["v"][:T].contiguous(), d["g"][:T].contiguous(),
                               d["beta"][:T].contiguous(), cu, initial_state=d["h0"],
                               out_dtype=torch.float32)
    o_last = gdn.recurrent_step(d["q"][T:].contiguous(), d["k"][T:].contiguous(),
                                d["v"][T:].contiguous(), d["g"][T:].contiguous(),
                                d["beta"][T:].contiguous(), h1, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle_case(case)
    assert_rms_close(torch.cat([o1, o_last]), o_ref, TOL["bf16"], "prefill+decode o")
    assert_rms_close(h1, h_ref, TOL["bf16"], "prefill+decode state")


_LAYOUT_CONFIGS = [(dt, d) for dt in ("bf16", "f32") for d in (32, 64, 128)]


def _concat_cases(a, b):
    """Case a followed by the sequences of case b (same heads and dtypes)."""
    cu = torch.cat([a.cu_seqlens, a.cu_seqlens[-1] + b.cu_seqlens[1:]])
    h0 = None if a.h0 is None else torch.cat([a.h0, b.h0])
    return si.CoreCase(q=torch.cat([a.q, b.q]), k=torch.cat([a.k, b.k]), v=torch.cat([a.v, b.v]),
                       g=torch.cat([a.g, b.g]), beta=torch.cat([a.beta, b.beta]), cu_seqlens=cu,
                       h0=h0, meta=dict(a.meta))


@pytest.mark.parametrize("dt,dd", _LAYOUT_CONFIGS)
def test_scan_batch_invariance_across_layouts(dt, dd):
    """A sequence's outputs and final state do not depend on what else is in the batch. The scan
    picks its workgroup layout from the number of (chain, 16-column tile) pairs, a chain being a
    (sequence, V head): three sequences alone (12 chains) run the row-split layout; the same three
    followed by 70 filler sequences (292 chains) run a one-wave-per-tile layout at every head size
    (for bf16 q/k/v the many-chain kernel with separate chain and output waves), and followed by
    20 (92 chains) at d = 128 as well. All three must agree bit for bit, for fp32 and bf16
    outputs, the bf16 output must be the fp32 output rounded, and the small run must meet the
    oracle."""
    base = si.make_core_case([300, 64, 5], 2, 4, dd, dd, dtype=dt, gate="model", h0_std=0.02,
                             seed=91 + dd)
    T0 = int(base.cu_seqlens[-1])
    runs = {}
    for fill in (0, 20, 70):
        case = base if fill == 0 else _concat_cases(
            base, si.make_core_case([64] * fill, 2, 4, dd, dd, dtype=dt, gate="model",
                                    h0_std=0.02, seed=500 + fill + dd))
        d = to_dev(case)
        for od in (torch.float32, torch.bfloat16):
            print(f"layout case {dt} d={dd} fillers={fill} out={od}", flush=True)
            o, h = gdn.chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                     initial_state=d["h0"], out_dtype=od)
            torch.cuda.synchronize()
            runs[(fill, od)] = (o[:T0].cpu(), h[:3].cpu())
    for od in (torch.float32, torch.bfloat16):
        o_a, h_a = runs[(0, od)]
        for fill in (20, 70):
            o_b, h_b = runs[(fill, od)]
            assert torch.equal(o_a, o_b) and torch.equal(h_a, h_b), (dt, dd, fill, od)
    (o32, h32), (o16, h16) = runs[(0, torch.float32)], runs[(0, torch.bfloat16)]
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(h16, h32), (dt, dd)
    o_ref, h_ref = oracle_case(base)
    assert_rms_close(o32, o_ref, TOL[dt], f"{dt} d={dd} o")
    assert_rms_close(h32, h_ref, TOL[dt], f"{dt} d={dd} final state")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_scale_across_layouts(dt):
    """The output scale (folded into the workspace's masked Q K^T and into the Q H term) on both
    scan layouts: three sequences alone (row-split layout) and followed by 70 fillers (one wave
    per tile; for bf16 q/k/v the many-chain kernel) agree bit for bit at scale 0.37, and the
    small run meets the oracle's scaled output; the final states do not depend on the scale."""
    base = si.make_core_case([300, 64, 5], 2, 4, 128, 128, dtype=dt, gate="model", h0_std=0.02,
                             seed=131)
    T0 = int(base.cu_seqlens[-1])
    runs = {}
    for fill in (0, 70):
        case = base if fill == 0 else _concat_cases(
            base, si.make_core_case([64] * fill, 2, 4, 128, 128, dtype=dt, gate="model",
                                    h0_std=0.02, seed=600 + fill))
        d = to_dev(case)
        print(f"scale case {dt} fillers={fill}", flush=True)
        o, h = gdn.chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                 initial_state=d["h0"], scale=0.37, out_dtype=torch.float32)
        torch.cuda.synchronize()
        runs[fill] = (o[:T0].cpu(), h[:3].cpu())
    assert torch.equal(runs[0][0], runs[70][0]) and torch.equal(runs[0][1], runs[70][1]), dt
    o_ref, h_ref = oracle_case(base)
    assert_rms_close(runs[0][0], 0.37 * o_ref, TOL[dt], f"{dt} scale 0.37 o")
    assert_rms_close(runs[0][1], h_ref, TOL[dt], f"{dt} scale 0.37 final state")


def test_binding_output_buffers_follow_the_given_tensor():
    """A caller-provided o decides the output dtype when out_dtype is not given (fp32 q/k/v with
    a bf16 o writes bf16, the rounded fp32 result); an o, final state or workspace that does not
    match the call is refused on the host before any launch."""
    case = si.make_core_case([70, 5], 2, 4, 64, 64, dtype="f32", gate="model", h0_std=0.02,
                             seed=71)
    d = to_dev(case)
    T = case.q.shape[0]
    o32, h32 = gdn.chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                 initial_state=d["h0"])
    o16 = torch.empty((T, 4, 64), dtype=torch.bfloat16, device="cuda")
    o_ret, _ = gdn.chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                 initial_state=d["h0"], o=o16)
    ws = torch.empty(gdn.workspace_size(T, 2, 2, 4, 64), dtype=torch.uint8, device="cuda")
    gdn.chunk_intra(d["q"], d["k"], d["g"], d["beta"], d["cu_seqlens"], 4, ws)
    o16s = torch.empty_like(o16)
    gdn.chunk_scan(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], ws,
                   initial_state=d["h0"], o=o16s)
    torch.cuda.synchronize()
    assert o_ret.data_ptr() == o16.data_ptr()
    assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(o16s, o16)
    bad = [
        dict(o=torch.empty((T, 4, 64), dtype=torch.bfloat16, device="cuda"),
             out_dtype=torch.float32),                                     # dtype mismatch
        dict(o=torch.empty((T - 1, 4, 64), dtype=torch.float32, device="cuda")),  # short
        dict(o=torch.empty((T, 4, 64), dtype=torch.float32, device="cuda")[:, :, ::1].transpose(0, 1)),
        dict(final_state=torch.empty((1, 4, 64, 64), dtype=torch.float32, device="cuda")),
    ]
    for kw in bad:
        with pytest.raises(gdn.GdnError):
            gdn.chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                              initial_state=d["h0"], **kw)
        if "o" in kw:
            with pytest.raises(gdn.GdnError):
                gdn.chunk_scan(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], ws,
                               initial_state=d["h0"], **kw)
    with pytest.raises(gdn.GdnError):
        gdn.recurrent_step(d["q"][:2], d["k"][:2], d["v"][:2], d["g"][:2], d["beta"][:2],
                           d["h0"].clone(), o=torch.empty((2, 4, 32), device="cuda"))
