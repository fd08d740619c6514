"""GPU parity of the many-chain scan layout on its edge cases.

The chunked prefill picks its scan layout from the shape alone: bf16 q/k/v with more than 512
(chain, 16-column tile) pairs, a chain being a (sequence, V head), run the many-chain kernel
(chain, output and producer waves per workgroup). Here 80 packed sequences whose lengths repeat
0, 1, 5, 63, 64, 65, 130 and 300 tokens (empty sequences, single tokens, chunk boundaries and
ragged tails), 2 QK heads serving 8 V heads (G = 4), give 640 chains: 1280 pairs at d = 32, 2560
at d = 64, 5120 at d = 128, all on that kernel. Each variant compares every output and final
state with the float64 oracle at the bf16-input bar, max|err| <= 2e-2 x RMS."""

import numpy as np
import pytest
import torch

import gated_deltanet_linear_amd as gdn
import synthetic_inputs as si
from gdn_testutil import (TOL, assert_rms_close, assert_rms_close_rounded_out, oracle_case,
                          to_dev)

pytestmark = pytest.mark.gpu

LENGTHS = [0, 1, 5, 63, 64, 65, 130, 300] * 10


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("variant", ["fp32_states", "no_initial_state_bf16_out", "bf16_states",
                                     "no_final_state"])
def test_many_chain_edge_cases(d, variant):
    case = si.make_core_case(LENGTHS, 2, 8, d, d, dtype="bf16", gate="model",
                             h0_std=0.0 if variant == "no_initial_state_bf16_out" else 0.02,
                             seed=700 + d)
    if variant == "bf16_states":  # the stored initial state is bf16; the oracle starts from it
        case = si.CoreCase(q=case.q, k=case.k, v=case.v, g=case.g, beta=case.beta,
                           cu_seqlens=case.cu_seqlens, h0=case.h0.to(torch.bfloat16).float(),
                           meta=case.meta)
    print(f"[many-chain] d={d} {variant}", flush=True)
    dv = to_dev(case)
    h0 = dv["h0"]
    if variant == "no_initial_state_bf16_out":
        h0 = None
    elif variant == "bf16_states":
        h0 = h0.to(torch.bfloat16)
    out_dtype = torch.bfloat16 if variant == "no_initial_state_bf16_out" else torch.float32
    o, ht = gdn.chunk_forward(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], dv["cu_seqlens"],
                              initial_state=h0, output_final_state=variant != "no_final_state",
                              out_dtype=out_dtype)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle_case(case)
    tol = TOL["bf16"]
    if out_dtype == torch.bfloat16:
        assert_rms_close_rounded_out(o, o_ref, tol, f"d={d} {variant} o")
    else:
        assert_rms_close(o, o_ref, tol, f"d={d} {variant} o")
    if variant == "no_final_state":
        assert ht is None
    elif variant == "bf16_states":
        assert ht.dtype == torch.bfloat16
        assert_rms_close_rounded_out(ht, h_ref, tol, f"d={d} {variant} final state")
    else:
        assert_rms_close(ht, h_ref, tol, f"d={d} {variant} final state")
    # empty sequences pass their initial state through unchanged
    cu = case.cu_seqlens.numpy()
    for n in np.flatnonzero(np.diff(cu) == 0)[:3]:
        if ht is not None:
            want = torch.zeros_like(ht[n]) if h0 is None else h0[n]
            assert torch.equal(ht[n], want), (d, variant, n)
