"""Parity at the full workload sizes, in the launch configuration the benchmark times
(bf16 inputs; the library picks the same grid for the same shape)."""

import numpy as np
import pytest
import torch

import gated_deltanet_linear_amd as gdn
import synthetic_inputs as si
from gdn_testutil import TOL, assert_rms_close, f64, oracle_case, oracle_chains, to_dev

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


def test_long_context_workload_sampled():
    """Workload 3 (4 x 32768 tokens, initial states): sampled (sequence, V head) chains."""
    case = si.workload_case(3)
    d = to_dev(case)
    o, ht = gdn.chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                              initial_state=d["h0"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    chains = [(0, 0), (1, 17), (2, 31), (3, 8), (3, 30)]
    refs = oracle_chains(case, chains)
    cu = case.cu_seqlens.numpy()
    got_o = np.concatenate([f64(o[cu[n]:cu[n + 1], h]) for n, h in chains])
    ref_o = np.concatenate([refs[c][0] for c in chains])
    assert_rms_close(got_o, ref_o, TOL["bf16"], "workload 3 o (sampled chains)")
    assert_rms_close(np.stack([f64(ht[n, h]) for n, h in chains]),
                     np.stack([refs[c][1] for c in chains]), TOL["bf16"],
                     "workload 3 final states (sampled chains)")


def test_long_context_slow_decay_sampled():
    """Slow decay at the long-context shape: the state crosses 512 chunks."""
    case = si.slow_decay_case([32768] * 4, 16, 32, 128, 128, dtype="bf16", seed=1003)
    d = to_dev(case)
    o, ht = gdn.chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                              initial_state=d["h0"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    chains = [(0, 5), (2, 12), (3, 31)]
    refs = oracle_chains(case, chains)
    cu = case.cu_seqlens.numpy()
    got_o = np.concatenate([f64(o[cu[n]:cu[n + 1], h]) for n, h in chains])
    ref_o = np.concatenate([refs[c][0] for c in chains])
    assert_rms_close(got_o, ref_o, TOL["bf16"], "slow decay 4x32768 o (sampled)")
    assert_rms_close(np.stack([f64(ht[n, h]) for n, h in chains]),
                     np.stack([refs[c][1] for c in chains]), TOL["bf16"],
                     "slow decay 4x32768 final states (sampled)")
