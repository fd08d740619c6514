"""GPU test of gdn_chunk_forward_noalloc (the chunked prefill with its workspace in the library's
own device array): through the C ABI, two calls in a row, the second with a smaller input, each
against gdn_chunk_forward on the same inputs. Both run the same kernels on the same inputs, so
the outputs and final states must be bit-identical; the first is also checked against the oracle
at the bf16 bar."""

import pytest
import torch

import gated_deltanet_linear_amd as gdn
import synthetic_inputs as si
from gdn_testutil import TOL, assert_rms_close, oracle_case, to_dev

pytestmark = pytest.mark.gpu


def _both(case, out_dtype, split_f32=False):
    d = to_dev(case)
    print(f"[noalloc] lengths={case.meta['lengths'][:4]} heads={case.meta['hv']} "
          f"d={case.meta['dk']} out={out_dtype} split_f32={split_f32}", flush=True)
    o_a, h_a = gdn.chunk_forward_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                         d["cu_seqlens"], initial_state=d["h0"],
                                         out_dtype=out_dtype, split_f32=split_f32)
    torch.cuda.synchronize()
    o_b, h_b = gdn.chunk_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"],
                                 initial_state=d["h0"], out_dtype=out_dtype, split_f32=split_f32)
    torch.cuda.synchronize()
    return (o_a.cpu(), h_a.cpu()), (o_b.cpu(), h_b.cpu())


def test_noalloc_matches_chunk_forward_twice_then_smaller():
    big = si.make_core_case([4096], 16, 32, 128, 128, dtype="bf16", gate="model", h0_std=0.02,
                            seed=1201)  # 65 x 32 records: 52 MB of the 64 MiB array
    small = si.make_core_case([300, 64, 5], 2, 4, 64, 64, dtype="bf16", gate="model",
                              h0_std=0.02, seed=1202)
    (o1, h1), (r1, s1) = _both(big, torch.float32)
    assert torch.equal(o1, r1) and torch.equal(h1, s1)
    (o2, h2), (r2, s2) = _both(small, torch.float32)
    assert torch.equal(o2, r2) and torch.equal(h2, s2)
    (o3, h3), (r3, s3) = _both(small, torch.bfloat16)
    assert torch.equal(o3, r3) and torch.equal(h3, s3)
    o_ref, h_ref = oracle_case(small)
    assert_rms_close(o2, o_ref, TOL["bf16"], "noalloc o")
    assert_rms_close(h2, h_ref, TOL["bf16"], "noalloc final state")


def test_noalloc_split_f32_matches_chunk_forward():
    """fp32 q/k/v on the split-bf16 path (GDN_DTYPE_F32_SPLIT) through the library's array, two
    calls in a row, the second smaller."""
    big = si.make_core_case([(71 * i) % 700 for i in range(9)], 2, 8, 128, 128, dtype="f32",
                            gate="model", h0_std=0.02, seed=1204)  # many-chain layout
    small = si.make_core_case([130, 7], 1, 2, 32, 32, dtype="f32", gate="model", h0_std=0.02,
                              seed=1205)
    for case in (big, small):
        (o1, h1), (r1, s1) = _both(case, torch.float32, split_f32=True)
        assert torch.equal(o1, r1) and torch.equal(h1, s1)
    o_ref, h_ref = oracle_case(small)
    assert_rms_close(o1, o_ref, TOL["bf16"], "noalloc split o")
    assert_rms_close(h1, h_ref, TOL["bf16"], "noalloc split final state")


def test_noalloc_refuses_a_shape_beyond_its_array():
    case = si.make_core_case([8192], 16, 32, 128, 128, dtype="bf16", gate="model", seed=1203)
    d = to_dev(case)
    with pytest.raises(gdn.GdnError, match="SCRATCH_LIMIT"):
        gdn.chunk_forward_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"])
