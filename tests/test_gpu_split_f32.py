"""GPU parity of the chunked prefill on fp32 q/k/v taken on the split-bf16 MFMA path
(qkv_dtype GDN_DTYPE_F32_SPLIT: every product but the intra kernel's inverse on bf16 MFMA with
both operands as hi + lo bf16 pairs).

Such q/k/v stand for values derived from bf16 inputs (the front end's fp32 output), so the bar
is the bf16 one, 2e-2 x RMS, against the float64 oracle on the same fp32 values. Both scan
layouts are covered: few chains (four waves per 16-column tile) and many chains (one wave per
tile)."""

import dataclasses

import pytest
import torch

import gated_deltanet_linear_amd as gdn
import synthetic_inputs as si
from gdn_testutil import (TOL, assert_rms_close, assert_rms_close_rounded_out, oracle_case,
                          rel_err)

pytestmark = pytest.mark.gpu


def _run(case, split, out_dtype=torch.float32, final=True):
    dev = "cuda"
    d = {k: getattr(case, k) for k in ("q", "k", "v", "g", "beta", "cu_seqlens", "h0")}
    d = {k: (t.to(dev) if t is not None else None) for k, t in d.items()}
    o, ht = gdn.chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                              initial_state=d["h0"], output_final_state=final,
                              out_dtype=out_dtype, split_f32=split)
    torch.cuda.synchronize()
    return o.cpu(), (ht.cpu() if ht is not None else None)


# (layout, d): lengths and head counts that put the launch in that layout (many chains: more
# than 512 (sequence, V head, 16-column tile) units)
CASES = {
    ("few", 32): dict(lengths=[1, 63, 0, 64, 65, 130, 300], hqk=2, hv=4),
    ("few", 64): dict(lengths=[127, 0, 200, 5], hqk=1, hv=4),
    ("few", 128): dict(lengths=[300, 64, 1, 129], hqk=2, hv=4),
    ("many", 32): dict(lengths=[(37 * i) % 150 for i in range(33)], hqk=4, hv=8),
    ("many", 64): dict(lengths=[(53 * i) % 190 for i in range(17)], hqk=4, hv=8),
    ("many", 128): dict(lengths=[(71 * i) % 210 for i in range(9)], hqk=2, hv=8),
}


@pytest.mark.parametrize("layout,d", sorted(CASES))
def test_split_f32_against_oracle(layout, d):
    c = CASES[(layout, d)]
    case = si.make_core_case(c["lengths"], c["hqk"], c["hv"], d, d, dtype="f32", gate="model",
                             h0_std=0.02, seed=900 + d + (layout == "many"))
    print(f"[split_f32] layout={layout} d={d} lengths={c['lengths']}", flush=True)
    o, ht = _run(case, split=True)
    ref_o, ref_h = oracle_case(case)
    assert_rms_close(o, ref_o, TOL["bf16"], "split o")
    assert_rms_close(ht, ref_h, TOL["bf16"], "split final state")
    # the fp32-MFMA path on the same inputs, for the record
    o32, h32 = _run(case, split=False)
    print(f"  fp32 path: o {rel_err(o32, ref_o):.3e}, final state {rel_err(h32, ref_h):.3e} x RMS",
          flush=True)
    # bf16 output = the round-to-nearest-even cast of the fp32 output; no final state requested
    ob, hb = _run(case, split=True, out_dtype=torch.bfloat16, final=False)
    assert hb is None
    assert torch.equal(ob, o.to(torch.bfloat16))


def test_split_f32_slow_decay():
    """Slow decay (g ~ U(-0.01, 0)): a long memory, the state's rounding and the split operands'
    errors survive many chunks."""
    case = si.slow_decay_case([1000, 333], 2, 4, 128, 128, dtype="f32", seed=931)
    o, ht = _run(case, split=True)
    ref_o, ref_h = oracle_case(case)
    assert_rms_close(o, ref_o, TOL["bf16"], "split slow-decay o")
    assert_rms_close(ht, ref_h, TOL["bf16"], "split slow-decay final state")


def test_split_f32_stages_equal_forward():
    """gdn_chunk_intra + gdn_chunk_scan with split_f32 give gdn_chunk_forward's bits."""
    case = si.make_core_case([(71 * i) % 210 for i in range(9)], 2, 8, 128, 128, dtype="f32",
                             gate="model", h0_std=0.02, seed=932)
    o, ht = _run(case, split=True)
    dev = "cuda"
    q, k, v, g, b, cu, h0 = (t.to(dev) for t in (case.q, case.k, case.v, case.g, case.beta,
                                                  case.cu_seqlens, case.h0))
    T, n = q.shape[0], cu.numel() - 1
    ws = torch.empty(gdn.workspace_size(T, n, 2, 8, 128), dtype=torch.uint8, device=dev)
    gdn.chunk_intra(q, k, g, b, cu, 8, ws, split_f32=True)
    o2, h2 = gdn.chunk_scan(q, k, v, g, b, cu, ws, initial_state=h0,
                            final_state=torch.empty_like(h0), out_dtype=torch.float32,
                            split_f32=True)
    torch.cuda.synchronize()
    assert torch.equal(o2.cpu(), o) and torch.equal(h2.cpu(), ht)


def test_split_f32_rejects_bf16_inputs():
    case = si.make_core_case([10], 1, 1, 32, 32, dtype="bf16", seed=933)
    with pytest.raises(gdn.GdnError):
        _run(case, split=True)


@pytest.mark.parametrize("layout", ["few", "many"])
def test_split_f32_scale_and_bf16_state(layout):
    """Output scale 0.37 (folded into P by the intra kernel and into the Q H term by the scan) and
    bf16 initial / final states, against the oracle on the same bf16 initial state."""
    c = CASES[(layout, 128)]
    case = si.make_core_case(c["lengths"], c["hqk"], c["hv"], 128, 128, dtype="f32",
                             gate="model", h0_std=0.02, seed=934)
    case = dataclasses.replace(case, h0=case.h0.to(torch.bfloat16).float())  # bf16 values
    dev = "cuda"
    d = {k: getattr(case, k).to(dev) for k in ("q", "k", "v", "g", "beta", "cu_seqlens")}
    h0 = case.h0.to(torch.bfloat16).to(dev)
    o, ht = gdn.chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                              initial_state=h0, scale=0.37, out_dtype=torch.float32,
                              split_f32=True)
    torch.cuda.synchronize()
    assert ht.dtype == torch.bfloat16
    ref_o, ref_h = oracle_case(case)
    assert_rms_close(o.cpu(), 0.37 * ref_o, TOL["bf16"], "split o, scale 0.37")
    # the final state is stored as bf16: one bf16 rounding of the reference allowed
    assert_rms_close_rounded_out(ht.cpu(), ref_h, TOL["bf16"], "split bf16 final state")
