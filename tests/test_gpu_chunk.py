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


def test_scan_layouts_are_bit_identical():
    """The scan layouts (row-split: 4 waves per d_v tile; tile-per-wave with 4 tiles per
    workgroup; tile-per-wave with all 8 tiles of a d = 128 chain per workgroup, bf16 in and out)
    for every input dtype, output dtype and head size: identical bits, the tile layout within
    tolerance of the oracle, and bf16 outputs equal to the fp32 outputs rounded. Each layout runs
    in a process of its own (the layout is chosen once per process)."""
    import os
    import subprocess
    import sys
    import tempfile
    code = (
        "import sys, torch; sys.path.insert(0, '.'); import synthetic_inputs as si;"
        "import gated_deltanet_linear_amd as gdn;"
        "res = [];"
        f"cfgs = {_LAYOUT_CONFIGS!r};\n"
        "for dt, dd in cfgs:\n"
        "    c = si.make_core_case([300, 64, 5], 2, 4, dd, dd, dtype=dt, gate='model',"
        " h0_std=0.02, seed=91 + dd);\n"
        "    d = {k: getattr(c, k).cuda() for k in ('q','k','v','g','beta','cu_seqlens','h0')};\n"
        "    for od in (torch.float32, torch.bfloat16):\n"
        "        print('layout case', dt, dd, od, flush=True);\n"
        "        o, h = gdn.chunk_forward(d['q'], d['k'], d['v'], d['g'], d['beta'],"
        " d['cu_seqlens'], initial_state=d['h0'], out_dtype=od);\n"
        "        res.append((o.cpu(), h.cpu()))\n"
        "torch.save(res, sys.argv[1])\n")
    outs = {}
    with tempfile.TemporaryDirectory() as td:
        for layout in ("rows", "tiles", "tiles8"):
            path = os.path.join(td, layout + ".pt")
            env = dict(os.environ, GDN_SCAN_LAYOUT=layout)
            print(f"[layout] {layout}", flush=True)
            subprocess.run([sys.executable, "-c", code, path], check=True, env=env,
                           cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           timeout=300)
            outs[layout] = torch.load(path, weights_only=True)
    for i, (dt, dd) in enumerate(_LAYOUT_CONFIGS):
        for j, od in enumerate(("f32", "bf16")):
            (o_r, h_r), (o_t, h_t) = outs["rows"][2 * i + j], outs["tiles"][2 * i + j]
            assert torch.equal(o_r, o_t) and torch.equal(h_r, h_t), (dt, dd, od)
            o_8, h_8 = outs["tiles8"][2 * i + j]
            assert torch.equal(o_r, o_8) and torch.equal(h_r, h_8), (dt, dd, od, "tiles8")
        (o32, h32), (o16, h16) = outs["tiles"][2 * i], outs["tiles"][2 * i + 1]
        assert torch.equal(o16, o32.to(torch.bfloat16)) and torch.equal(h16, h32), (dt, dd)
        case = si.make_core_case([300, 64, 5], 2, 4, dd, dd, dtype=dt, gate="model",
                                 h0_std=0.02, seed=91 + dd)
        o_ref, h_ref = oracle_case(case)
        assert_rms_close(o32, o_ref, TOL[dt], f"tiles {dt} d={dd} o")
        assert_rms_close(h32, h_ref, TOL[dt], f"tiles {dt} d={dd} final state")
