"""GPU parity of the chunked backward (gdn_chunk_backward) against the float64 oracle's reverse
mode (itself pinned by finite differences of the forward oracle).

Every gradient is held to the fp32 bar (max|err| <= 1e-4 * RMS of the reference gradient), for
bf16 inputs too, although there most products run on bf16 MFMA with the computed operands carried
as hi + lo bf16 pairs; gradients written in bf16 (dq, dk, dv for bf16 inputs) are allowed their
own rounding (one bf16 ulp of the reference) on top.
"""

import numpy as np
import pytest
import torch

import gated_deltanet_linear_amd as gdn
import oracle
import synthetic_inputs as si
from gdn_testutil import TOL, assert_rms_close, assert_rms_close_rounded_out, f64

pytestmark = pytest.mark.gpu


def _run(case, dout, dht, h0, scale):
    dev = "cuda"
    args = [getattr(case, a).to(dev) for a in ("q", "k", "v", "g", "beta", "cu_seqlens")]
    return gdn.chunk_backward(*args, dout.to(dev), initial_state=None if h0 is None else h0.to(dev),
                              dht=None if dht is None else dht.to(dev), scale=scale)


def _check(case, dout, dht, h0, scale, what):
    got = _run(case, dout, dht, h0, scale)
    torch.cuda.synchronize()
    ref = oracle.recurrent_backward(f64(case.q), f64(case.k), f64(case.v), f64(case.g),
                                    f64(case.beta), case.cu_seqlens.numpy(), f64(dout),
                                    initial_state=None if h0 is None else f64(h0),
                                    dht=None if dht is None else f64(dht), scale=scale)
    bf = case.q.dtype == torch.bfloat16
    for name, gv, rv in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), got, ref):
        check = assert_rms_close_rounded_out if (bf and name in ("dq", "dk", "dv")) else \
            assert_rms_close
        check(gv, rv, TOL["f32"], f"{what} {name}")


@pytest.mark.parametrize("d,dtype", [(32, "f32"), (32, "bf16"), (64, "bf16"), (64, "f32"),
                                     (128, "bf16"), (128, "f32")])
@pytest.mark.parametrize("lengths", [[1], [63], [64, 65], [130, 7]])
def test_backward_small(d, dtype, lengths):
    rng = np.random.default_rng(d * 1000 + sum(lengths))
    hqk, hv = 1, 2
    case = si.make_core_case(lengths, hqk, hv, d, d, dtype=dtype, gate="model",
                             seed=d + sum(lengths))
    n, T = len(lengths), sum(lengths)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    dout = torch.from_numpy(rng.standard_normal((T, hv, d))).to(dt)
    dht = torch.from_numpy(rng.standard_normal((n, hv, d, d)) * 0.1).float()
    h0 = torch.from_numpy(rng.standard_normal((n, hv, d, d)) * 0.05).float()
    print(f"[backward] d={d} {dtype} lengths={lengths}", flush=True)
    _check(case, dout, dht, h0, 0.8, f"d={d} {dtype} {lengths}")


def test_backward_gqa_varlen_no_state_terms():
    rng = np.random.default_rng(3)
    lengths = [70, 0, 129, 1]
    hqk, hv, d = 2, 8, 64
    case = si.make_core_case(lengths, hqk, hv, d, d, dtype="bf16", gate="model", seed=5)
    T = sum(lengths)
    dout = torch.from_numpy(rng.standard_normal((T, hv, d))).to(torch.bfloat16)
    print("[backward] GQA varlen, no initial state, no final-state term", flush=True)
    _check(case, dout, None, None, 1.0, "gqa varlen")


def test_backward_slow_decay_long():
    # slow decay: the state carries over all chunks of a 1000-token sequence
    rng = np.random.default_rng(9)
    case = si.slow_decay_case([1000], 1, 1, 64, 64, dtype="bf16", seed=9)
    dout = torch.from_numpy(rng.standard_normal((1000, 1, 64))).to(torch.bfloat16)
    dht = torch.from_numpy(rng.standard_normal((1, 1, 64, 64)) * 0.1).float()
    print("[backward] slow decay, 1000 tokens", flush=True)
    _check(case, dout, dht, case.h0, 1.0, "slow decay 1000")


def test_backward_bf16_states():
    rng = np.random.default_rng(21)
    lengths = [100, 30]
    hqk, hv, d = 1, 2, 64
    case = si.make_core_case(lengths, hqk, hv, d, d, dtype="bf16", gate="model", seed=21)
    n, T = len(lengths), sum(lengths)
    dout = torch.from_numpy(rng.standard_normal((T, hv, d))).to(torch.bfloat16)
    dht = torch.from_numpy(rng.standard_normal((n, hv, d, d)) * 0.1).to(torch.bfloat16)
    h0 = torch.from_numpy(rng.standard_normal((n, hv, d, d)) * 0.05).to(torch.bfloat16)
    got = _run(case, dout, dht, h0, 1.0)
    torch.cuda.synchronize()
    assert got[5].dtype == torch.bfloat16
    ref = oracle.recurrent_backward(f64(case.q), f64(case.k), f64(case.v), f64(case.g),
                                    f64(case.beta), case.cu_seqlens.numpy(), f64(dout),
                                    initial_state=f64(h0), dht=f64(dht))
    for name, gv, rv in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), got, ref):
        check = assert_rms_close if name in ("dg", "dbeta") else assert_rms_close_rounded_out
        check(gv, rv, TOL["f32"], f"bf16 states {name}")


def test_backward_full_size_sampled_heads():
    """The 1 x 4096 prefill shape (16 QK / 32 V heads, d = 128, bf16): every gradient of two
    sampled QK heads (and their four V heads) against the oracle run on those heads alone."""
    case = si.workload_case(2)
    rng = np.random.default_rng(22)
    T, hqk, d = case.q.shape
    hv = case.v.shape[1]
    dout = torch.from_numpy(rng.standard_normal((T, hv, d))).to(torch.bfloat16)
    print("[backward] 1x4096, 16/32 heads", flush=True)
    got = _run(case, dout, None, None, 1.0)
    torch.cuda.synchronize()
    qk_heads = [0, 11]
    v_heads = [h for m in qk_heads for h in (2 * m, 2 * m + 1)]
    ref = oracle.recurrent_backward(f64(case.q[:, qk_heads]), f64(case.k[:, qk_heads]),
                                    f64(case.v[:, v_heads]), f64(case.g[:, v_heads]),
                                    f64(case.beta[:, v_heads]), case.cu_seqlens.numpy(),
                                    f64(dout[:, v_heads]))
    sel = dict(dq=qk_heads, dk=qk_heads, dv=v_heads, dg=v_heads, dbeta=v_heads)
    for name, gv, rv in zip(("dq", "dk", "dv", "dg", "dbeta"), got, ref):
        gs = gv[:, sel[name]].cpu()
        check = assert_rms_close_rounded_out if name in ("dq", "dk", "dv") else assert_rms_close
        check(gs, rv, TOL["f32"], f"1x4096 {name}")
    # no initial state given: dh0 is still the gradient of the (zero) initial state
    assert_rms_close(got[5][:, v_heads].cpu(), ref[5], TOL["f32"], "1x4096 dh0")


def test_backward_all_sequences_empty():
    # no tokens: every gradient is empty and dh0 is the final-state gradient passed through
    hqk, hv, d = 1, 2, 32
    case = si.make_core_case([0, 0], hqk, hv, d, d, dtype="f32", seed=1)
    dout = torch.zeros((0, hv, d))
    dht = torch.from_numpy(np.random.default_rng(2).standard_normal((2, hv, d, d))).float()
    got = _run(case, dout, dht, None, 1.0)
    torch.cuda.synchronize()
    assert all(t.shape[0] == 0 for t in got[:5])
    assert torch.equal(got[5].cpu(), dht)
