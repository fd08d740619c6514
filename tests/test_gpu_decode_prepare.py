"""GPU parity of gdn_recurrent_step (decode) and gdn_prepare (front end) against the oracle."""

import numpy as np
import pytest
import torch

import gated_deltanet_linear_amd as gdn
import oracle
import synthetic_inputs as si
from gdn_testutil import TOL, rel_err, assert_rms_close, f64, oracle_case, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,dtype", [(32, "f32"), (64, "bf16"), (128, "bf16"), (128, "f32")])
def test_recurrent_step_small(d, dtype):
    case = si.make_core_case([1] * 12, 2, 6, d, d, dtype=dtype, gate="model", h0_std=0.5,
                             seed=d + len(dtype))
    print(f"[decode] d={d} {dtype}", flush=True)
    dd = to_dev(case)
    state = dd["h0"].clone()
    o = gdn.recurrent_step(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], state,
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_case(case)
    assert_rms_close(o, o_ref, TOL[dtype], "decode o")
    assert_rms_close(state, s_ref, TOL[dtype], "decode state")


def test_recurrent_step_decode_workload_full():
    """Workload 4 at full size: 256 sequences x 1 token, 16/32 heads, d = 128, 537 MB state."""
    case = si.workload_case(4)
    dd = to_dev(case)
    state = dd["h0"].clone()
    o16 = gdn.recurrent_step(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], state)
    state32 = dd["h0"].clone()
    o32 = gdn.recurrent_step(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], state32,
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(torch.bfloat16))  # bf16 output = RNE of the fp32 output
    assert torch.equal(state, state32)
    o_ref, s_ref = oracle_case(case)
    assert_rms_close(o32, o_ref, TOL["bf16"], "decode workload o")
    assert_rms_close(state32, s_ref, TOL["bf16"], "decode workload state")


def test_decode_steps_equal_chunked_prefill():
    """T decode steps on the GPU ~ one chunked prefill of the same T tokens (both vs oracle)."""
    case = si.slow_decay_case([70], 1, 2, 128, 128, dtype="bf16", seed=4)
    dd = to_dev(case)
    state = dd["h0"].clone()
    outs = []
    for t in range(70):
        sl = slice(t, t + 1)
        outs.append(gdn.recurrent_step(dd["q"][sl], dd["k"][sl], dd["v"][sl], dd["g"][sl],
                                       dd["beta"][sl], state, out_dtype=torch.float32))
    oc, hc = gdn.chunk_forward(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], dd["cu_seqlens"],
                               initial_state=dd["h0"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle_case(case)
    assert_rms_close(torch.cat(outs), o_ref, TOL["bf16"], "decode x70 o")
    assert_rms_close(state, h_ref, TOL["bf16"], "decode x70 state")
    assert_rms_close(oc, f64(torch.cat(outs)), 2 * TOL["bf16"], "chunk vs decode o")


def _prep_case(lengths, d=32, hqk=2, hv=4, seed=0, dtype="bf16", bias=False):
    fc = si.make_front_case(lengths, hqk, hv, d, d, dtype=dtype, seed=seed)
    if bias:
        rng = np.random.default_rng(seed + 1)
        fc.meta["bias"] = si._round(rng.standard_normal(fc.conv_weight.shape[0]) * 0.1,
                                    fc.conv_weight.dtype)
    return fc


def _prep_gpu(fc, qkv_dtype=None, bias=None):
    dev = "cuda"
    return gdn.prepare(fc.mixed_qkv.to(dev), fc.conv_weight.to(dev), fc.a.to(dev), fc.b.to(dev),
                       fc.A_log.to(dev), fc.dt_bias.to(dev), fc.cu_seqlens.to(dev),
                       fc.meta["hqk"], fc.meta["dk"], fc.meta["hv"], fc.meta["dv"],
                       conv_bias=None if bias is None else bias.to(dev), qkv_dtype=qkv_dtype)


def _prep_oracle(fc, bias=None):
    return oracle.prepare(f64(fc.mixed_qkv), f64(fc.conv_weight), f64(fc.a), f64(fc.b),
                          f64(fc.A_log), f64(fc.dt_bias), fc.cu_seqlens.numpy(), fc.meta["hqk"],
                          fc.meta["dk"], fc.meta["hv"], fc.meta["dv"], conv_bias=f64(bias))


def _check_prepare(got, ref, out_dtype):
    # q, k, v: one rounding to the output dtype after fp32 math; g, beta in fp32.
    rt = 2.0 ** -8 if out_dtype == torch.bfloat16 else 1e-5
    names = ("q", "k", "v", "g", "beta")
    for gt, rf, nm in zip(got, ref, names):
        gt = f64(gt)
        bound = (rt if nm in "qkv" else 1e-5) * np.abs(rf) + 1e-6
        bad = np.abs(gt - rf) > bound
        assert not bad.any(), f"prepare {nm}: {bad.sum()} elements off, worst " \
            f"{np.max(np.abs(gt - rf) - bound):.3e}"


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("qkv", [torch.bfloat16, torch.float32])
def test_prepare_small(d, qkv):
    fc = _prep_case([5, 0, 1, 300, 3, 260], d=d, seed=d)
    print(f"[prepare] d={d} qkv={qkv}", flush=True)
    got = _prep_gpu(fc, qkv_dtype=qkv)
    torch.cuda.synchronize()
    _check_prepare(got, _prep_oracle(fc), qkv)


def test_prepare_with_bias_fp32_inputs():
    fc = _prep_case([40, 17], d=64, dtype="f32", seed=3, bias=True)
    got = _prep_gpu(fc, qkv_dtype=torch.float32, bias=fc.meta["bias"])
    torch.cuda.synchronize()
    _check_prepare(got, _prep_oracle(fc, bias=fc.meta["bias"]), torch.float32)


def test_front_end_workload_stagewise_and_end_to_end():
    """Workload 5 (8 packed sequences, 16/64 heads, d = 128).

    Stage by stage: the front end against the oracle's front end, and the core on the front
    end's bf16 outputs against the oracle core on the same values (all 512 chains).

    End to end: gdn_prepare with fp32 q / k / v, then gdn_chunk_intra and gdn_chunk_scan with a
    bf16 output, on the fp32-MFMA path and on the split-bf16 path (split_f32, the benchmark's call
    sequence), against the float64 front end + float64 core (all chains): the fp32 output twin
    meets the bf16 bar and the bf16 output is its round-to-nearest-even cast. The path with bf16
    q / k / v between the two stages is measured and printed but not held to the bar: that
    rounding alone moves the float64 result by ~13% x RMS on this workload."""
    fc = si.workload_case(5)
    print(f"[front] lengths={fc.meta['lengths']}", flush=True)
    dev = "cuda"
    q, k, v, g, beta = _prep_gpu(fc, qkv_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = _prep_oracle(fc)
    _check_prepare((q, k, v, g, beta), ref, torch.bfloat16)

    h0 = fc.h0.to(dev)
    cu = fc.cu_seqlens.to(dev)
    o, ht = gdn.chunk_forward(q, k, v, g, beta, cu, initial_state=h0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    core = si.CoreCase(q=q.cpu(), k=k.cpu(), v=v.cpu(), g=g.cpu(), beta=beta.cpu(),
                       cu_seqlens=fc.cu_seqlens, h0=fc.h0, meta=fc.meta)
    o, ht = o.cpu(), ht.cpu()
    core_o, core_h = oracle_case(core)
    assert_rms_close(o, core_o, TOL["bf16"], "front workload core o (all chains)")
    assert_rms_close(ht, core_h, TOL["bf16"], "front workload core final state (all chains)")
    del core_o, core_h

    # float64 front end + float64 core on all chains
    rq, rk, rv, rg, rb = ref
    e2e_ref, e2e_href = oracle.recurrent(rq, rk, rv, rg, rb, fc.cu_seqlens.numpy(),
                                         initial_state=f64(fc.h0))

    # the old bf16-intermediate path, for the record
    print(f"  bf16 q/k/v between the stages: end-to-end o {rel_err(f64(o), e2e_ref):.3e} x RMS, "
          f"final state {rel_err(f64(ht), e2e_href):.3e} x RMS (not held to the bar)", flush=True)
    del o, ht

    # fp32 q/k/v, intra, scan, on the fp32-MFMA path and on the split-bf16 one (the benchmark's
    # sequence); bf16 output and its fp32 twin
    q32, k32, v32, g32, b32 = _prep_gpu(fc, qkv_dtype=torch.float32)
    T, n_seqs = q32.shape[0], len(fc.meta["lengths"])
    ws = torch.empty(gdn.workspace_size(T, n_seqs, 16, 64, 128), dtype=torch.uint8, device=dev)
    for split in (False, True):
        path = "split-bf16" if split else "fp32"
        outs = {}
        for od in (torch.float32, torch.bfloat16):
            gdn.chunk_intra(q32, k32, g32, b32, cu, 64, ws, split_f32=split)
            o_e, h_e = gdn.chunk_scan(q32, k32, v32, g32, b32, cu, ws, initial_state=h0,
                                      final_state=torch.empty_like(h0), out_dtype=od,
                                      split_f32=split)
            torch.cuda.synchronize()
            outs[od] = (o_e.cpu(), h_e.cpu())
        eo, eh = outs[torch.float32]
        assert_rms_close(eo, e2e_ref, TOL["bf16"],
                         f"front workload end-to-end o, {path} (all chains)")
        assert_rms_close(eh, e2e_href, TOL["bf16"],
                         f"front workload end-to-end final state, {path} (all chains)")
        assert torch.equal(outs[torch.bfloat16][0], outs[torch.float32][0].to(torch.bfloat16))
        assert torch.equal(outs[torch.bfloat16][1], outs[torch.float32][1])
