"""GPU parity of the output gate (gdn_gated_rmsnorm) and the decode-side front end
(gdn_decode_prepare) against the float64 oracle, and of a whole decode step from projected
inputs (decode_prepare + recurrent_step) against the oracle run over the whole sequence.

Tolerances as everywhere: max|err| <= 1e-4 * RMS(reference) for fp32 inputs, 2e-2 * RMS for
bf16 inputs; where the output itself is bf16, its own rounding (one bf16 ulp of the reference)
is allowed on top. Copies (the conv window) must be bit-exact.
"""

import numpy as np
import pytest
import torch

import gated_deltanet_linear_amd as gdn
import oracle
from gdn_testutil import TOL, assert_rms_close, assert_rms_close_rounded_out, f64

pytestmark = pytest.mark.gpu

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _rand(rng, shape, dtype, scale=1.0):
    return torch.from_numpy(rng.standard_normal(shape) * scale).to(dtype)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("odt,zdt", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16"),
                                     ("bf16", "f32")])
def test_gated_rmsnorm_small(d, odt, zdt):
    rng = np.random.default_rng(1000 + d)
    T, hv = 77, 3  # 231 rows: not a multiple of the rows a workgroup covers
    o = _rand(rng, (T, hv, d), _DT[odt], 0.7)
    z = _rand(rng, (T, hv, d), _DT[zdt], 1.5)
    tol = TOL["f32"] if odt == "f32" and zdt == "f32" else TOL["bf16"]
    for weight, off in ((None, 0.0), (rng.standard_normal(d) * 0.1, 1.0),
                        (rng.uniform(0.5, 1.5, d), 0.0)):
        w = None if weight is None else torch.tensor(weight, dtype=torch.float32)
        print(f"[gate] d={d} o={odt} z={zdt} weight={'none' if w is None else 'yes'} off={off}",
              flush=True)
        out = gdn.gated_rmsnorm(o.cuda(), z.cuda(), None if w is None else w.cuda(), off, 1e-6)
        torch.cuda.synchronize()
        ref = oracle.gated_rmsnorm(f64(o), f64(z), weight, off, 1e-6)
        check = assert_rms_close_rounded_out if odt == "bf16" else assert_rms_close
        check(out, ref, tol, f"gate d={d}")


def test_gated_rmsnorm_in_place_and_full_size_sampled():
    rng = np.random.default_rng(7)
    T, hv, d = 4096, 32, 128  # the 1x4096 prefill shape
    o = _rand(rng, (T, hv, d), torch.bfloat16)
    z = _rand(rng, (T, hv, d), torch.bfloat16)
    od = o.cuda()
    ref_full = gdn.gated_rmsnorm(od, z.cuda(), None, 0.0, 1e-6)
    out = gdn.gated_rmsnorm(od, z.cuda(), None, 0.0, 1e-6, out=od)  # in place
    torch.cuda.synchronize()
    assert out.data_ptr() == od.data_ptr() and torch.equal(out, ref_full)
    rows = rng.choice(T * hv, size=512, replace=False)
    got = out.view(-1, d)[torch.from_numpy(rows).cuda()].cpu()
    ref = oracle.gated_rmsnorm(f64(o.view(-1, d)[rows]), f64(z.view(-1, d)[rows]))
    assert_rms_close_rounded_out(got, ref, TOL["bf16"], "gate 1x4096 sampled rows")


def _front(rng, N, hqk, hv, d, dtype, bias=True):
    conv_dim = 2 * hqk * d + hv * d
    x = _rand(rng, (N, conv_dim), dtype)
    win = _rand(rng, (N, conv_dim, 3), dtype)
    w = _rand(rng, (conv_dim, 4), dtype, 0.5)
    bc = _rand(rng, (conv_dim,), dtype, 0.1) if bias else None
    a = _rand(rng, (N, hv), dtype)
    b = _rand(rng, (N, hv), dtype)
    A_log = torch.tensor(rng.uniform(-1.0, 1.0, hv), dtype=torch.float32)
    dt_bias = torch.tensor(rng.standard_normal(hv) * 0.2, dtype=torch.float32)
    return x, win, w, bc, a, b, A_log, dt_bias


@pytest.mark.parametrize("d,dt", [(32, "f32"), (64, "bf16"), (128, "bf16"), (128, "f32")])
def test_decode_prepare_against_oracle(d, dt):
    rng = np.random.default_rng(300 + d)
    N, hqk, hv = 37, 2, 6
    x, win, w, bc, a, b, A_log, dt_bias = _front(rng, N, hqk, hv, d, _DT[dt], bias=(d != 64))
    print(f"[decode_prepare] d={d} {dt} N={N}", flush=True)
    wd = win.cuda()
    q, k, v, g, beta = gdn.decode_prepare(x.cuda(), wd, w.cuda(), a.cuda(), b.cuda(),
                                          A_log.cuda(), dt_bias.cuda(), hqk, d, hv, d,
                                          conv_bias=None if bc is None else bc.cuda())
    torch.cuda.synchronize()
    rq, rk, rv, rg, rb, rwin = oracle.decode_prepare(
        f64(x), f64(win), f64(w), f64(a), f64(b), f64(A_log), f64(dt_bias), hqk, d, hv, d,
        conv_bias=f64(bc))
    tol = TOL[dt]
    check = assert_rms_close_rounded_out if dt == "bf16" else assert_rms_close
    for got, ref, name in ((q, rq, "q"), (k, rk, "k"), (v, rv, "v")):
        check(got, ref, tol, f"decode_prepare {name}")
    for got, ref, name in ((g, rg, "g"), (beta, rb, "beta")):  # fp32 outputs
        assert_rms_close(got, ref, tol, f"decode_prepare {name}")
    # the window is a shift of stored values: exact
    assert np.array_equal(f64(wd), rwin)


def test_decode_steps_from_projected_inputs_match_whole_sequence():
    """Prefill the first L0 tokens (front end + chunked core), then decode the remaining tokens
    one at a time with decode_prepare + recurrent_step: the decode outputs must match the oracle
    run over the whole sequence (front end + token recurrence). The front end writes fp32
    q/k/v here, so that every value the oracle does not see is an fp32 intermediate: the fp32
    tolerance applies."""
    rng = np.random.default_rng(11)
    hqk, hv, d, dtype = 2, 4, 128, torch.bfloat16
    L0, steps = 133, 3
    L = L0 + steps
    conv_dim = 2 * hqk * d + hv * d
    x = _rand(rng, (L, conv_dim), dtype)
    w = _rand(rng, (conv_dim, 4), dtype, 0.5)
    a = _rand(rng, (L, hv), dtype)
    b = _rand(rng, (L, hv), dtype)
    A_log = torch.tensor(rng.uniform(-1.0, 1.0, hv), dtype=torch.float32)
    dt_bias = torch.tensor(rng.standard_normal(hv) * 0.2, dtype=torch.float32)
    cu = torch.tensor([0, L0], dtype=torch.int32)
    # prefill
    q, k, v, g, beta = gdn.prepare(x[:L0].cuda(), w.cuda(), a[:L0].cuda(), b[:L0].cuda(),
                                   A_log.cuda(), dt_bias.cuda(), cu.cuda(), hqk, d, hv, d,
                                   qkv_dtype=torch.float32)
    _, state = gdn.chunk_forward(q, k, v, g, beta, cu.cuda(), out_dtype=torch.float32)
    window = x[L0 - 3:L0].T.contiguous().unsqueeze(0).cuda()  # [1, conv_dim, 3], oldest first
    outs = []
    for t in range(L0, L):
        qs, ks, vs, gs, bs = gdn.decode_prepare(x[t:t + 1].cuda(), window, w.cuda(),
                                                a[t:t + 1].cuda(), b[t:t + 1].cuda(),
                                                A_log.cuda(), dt_bias.cuda(), hqk, d, hv, d,
                                                qkv_dtype=torch.float32)
        outs.append(gdn.recurrent_step(qs, ks, vs, gs, bs, state, out_dtype=torch.float32))
    torch.cuda.synchronize()
    got = torch.cat(outs).cpu()
    rq, rk, rv, rg, rb = oracle.prepare(f64(x), f64(w), f64(a), f64(b), f64(A_log),
                                        f64(dt_bias), [0, L], hqk, d, hv, d)
    ro, rh = oracle.recurrent(rq, rk, rv, rg, rb, [0, L])
    assert_rms_close(got, ro[L0:], TOL["f32"], "decode outputs from projected inputs")
    assert_rms_close(state.cpu(), rh, TOL["f32"], "state after decode")
