"""Parity at the full workload sizes, in the launch configuration the benchmark times
(bf16 inputs; the library picks the same grid for the same shape)."""

import pytest
import torch

import gated_deltanet_linear_amd as gdn
import synthetic_inputs as si
from gdn_testutil import TOL, assert_rms_close, oracle_case, to_dev

pytestmark = pytest.mark.gpu


def test_prefill_35b_a3b_workload_full():
    """Workload 2 (1 x 4096 tokens, 16/32 heads, d = 128): every output against the oracle."""
    case = si.workload_case(2)
    d = to_dev(case)
    o, ht = gdn.chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                              out_dtype=torch.float32)
    o16, _ = gdn.chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(o16, o.to(torch.bfloat16))
    o_ref, h_ref = oracle_case(case)
    assert_rms_close(o, o_ref, TOL["bf16"], "workload 2 o")
    assert_rms_close(ht, h_ref, TOL["bf16"], "workload 2 final state")


def test_slow_decay_at_prefill_workload_shape():
    case = si.slow_decay_case([4096], 16, 32, 128, 128, dtype="bf16", seed=1002)
    d = to_dev(case)
    o, ht = gdn.chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                              initial_state=d["h0"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle_case(case)
    assert_rms_close(o, o_ref, TOL["bf16"], "slow decay 1x4096 o")
    assert_rms_close(ht, h_ref, TOL["bf16"], "slow decay 1x4096 final state")


def test_long_context_workload_all_chains():
    """Workload 3 (4 x 32768 tokens, initial states, the benchmark's headline): every output and
    every final state of all 128 (sequence, V head) chains against the float64 oracle."""
    case = si.workload_case(3)
    d = to_dev(case)
    o, ht = gdn.chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                              initial_state=d["h0"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    o, ht = o.cpu(), ht.cpu()
    o_ref, h_ref = oracle_case(case)
    assert_rms_close(o, o_ref, TOL["bf16"], "workload 3 o (all chains)")
    del o, o_ref
    assert_rms_close(ht, h_ref, TOL["bf16"], "workload 3 final states (all chains)")


def test_long_context_slow_decay_all_chains():
    """Slow decay at the long-context shape (the state crosses 512 chunks): all 128 chains."""
    case = si.slow_decay_case([32768] * 4, 16, 32, 128, 128, dtype="bf16", seed=1003)
    d = to_dev(case)
    o, ht = gdn.chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                              initial_state=d["h0"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    o, ht = o.cpu(), ht.cpu()
    o_ref, h_ref = oracle_case(case)
    assert_rms_close(o, o_ref, TOL["bf16"], "slow decay 4x32768 o (all chains)")
    del o, o_ref
    assert_rms_close(ht, h_ref, TOL["bf16"], "slow decay 4x32768 final states (all chains)")
