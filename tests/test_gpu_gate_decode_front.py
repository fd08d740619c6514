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


def _decode_oracle(x, win, w, bc, a, b, A_log, dt_bias, h0, hqk, hv, d, scale=1.0):
    """Float64 decode step from projected inputs: the oracle's front end, then one token of the
    oracle's recurrence per sequence from the given state."""
    N = x.shape[0]
    rq, rk, rv, rg, rb, rwin = oracle.decode_prepare(
        f64(x), f64(win), f64(w), f64(a), f64(b), f64(A_log), f64(dt_bias), hqk, d, hv, d,
        conv_bias=f64(bc))
    ro, rh = oracle.recurrent(rq, rk, rv, rg, rb, np.arange(N + 1), initial_state=f64(h0),
                              scale=scale)
    return ro, rh, rwin


@pytest.mark.parametrize("d,dt,G", [(32, "f32", 1), (64, "bf16", 2), (128, "bf16", 2),
                                    (128, "f32", 4), (64, "bf16", 3)])
def test_decode_step_fused_against_oracle(d, dt, G):
    rng = np.random.default_rng(500 + d + G)
    N, hqk = 19, 2
    hv = hqk * G
    x, win, w, bc, a, b, A_log, dt_bias = _front(rng, N, hqk, hv, d, _DT[dt], bias=(G != 3))
    h0 = torch.from_numpy(rng.standard_normal((N, hv, d, d)) * 0.05).float()
    for odt in ("f32", dt):
        print(f"[decode_step] d={d} {dt} G={G} out={odt}", flush=True)
        wd, hd = win.cuda(), h0.cuda()
        o = gdn.decode_step(x.cuda(), wd, w.cuda(), a.cuda(), b.cuda(), A_log.cuda(),
                            dt_bias.cuda(), hd, hqk, d, hv,
                            conv_bias=None if bc is None else bc.cuda(), scale=0.7,
                            out_dtype=_DT[odt])
        torch.cuda.synchronize()
        ro, rh, rwin = _decode_oracle(x, win, w, bc, a, b, A_log, dt_bias, h0, hqk, hv, d,
                                      scale=0.7)
        # every value the oracle does not see is an fp32 intermediate: the fp32 bar
        check = assert_rms_close_rounded_out if odt == "bf16" else assert_rms_close
        check(o, ro, TOL["f32"], "fused decode o")
        assert_rms_close(hd.cpu(), rh, TOL["f32"], "fused decode state")
        assert np.array_equal(f64(wd), rwin)


def test_decode_step_fused_matches_two_call_path():
    rng = np.random.default_rng(77)
    N, hqk, hv, d = 33, 4, 8, 128
    x, win, w, bc, a, b, A_log, dt_bias = _front(rng, N, hqk, hv, d, torch.bfloat16)
    h0 = torch.from_numpy(rng.standard_normal((N, hv, d, d)) * 0.02).float().cuda()
    w1, w2 = win.cuda(), win.cuda()
    s1, s2 = h0.clone(), h0.clone()
    o1 = gdn.decode_step(x.cuda(), w1, w.cuda(), a.cuda(), b.cuda(), A_log.cuda(),
                         dt_bias.cuda(), s1, hqk, d, hv, conv_bias=bc.cuda(),
                         out_dtype=torch.float32)
    q, k, v, g, beta = gdn.decode_prepare(x.cuda(), w2, w.cuda(), a.cuda(), b.cuda(),
                                          A_log.cuda(), dt_bias.cuda(), hqk, d, hv, d,
                                          conv_bias=bc.cuda(), qkv_dtype=torch.float32)
    o2 = gdn.recurrent_step(q, k, v, g, beta, s2, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(w1, w2)
    assert_rms_close(o1.cpu(), f64(o2), 1e-5, "fused vs two-call o")
    assert_rms_close(s1.cpu(), f64(s2), 1e-5, "fused vs two-call state")


def test_decode_step_fused_after_prefill_matches_whole_sequence():
    """Prefill 70 tokens, then 5 fused decode steps: the decode outputs and the final state must
    match the oracle over the whole 75-token sequence (front end + recurrence)."""
    rng = np.random.default_rng(12)
    hqk, hv, d, dtype = 2, 4, 64, torch.bfloat16
    L0, steps = 70, 5
    L = L0 + steps
    conv_dim = (2 * hqk + hv) * d
    x = _rand(rng, (L, conv_dim), dtype)
    w = _rand(rng, (conv_dim, 4), dtype, 0.5)
    a = _rand(rng, (L, hv), dtype)
    b = _rand(rng, (L, hv), dtype)
    A_log = torch.tensor(rng.uniform(-1.0, 1.0, hv), dtype=torch.float32)
    dt_bias = torch.tensor(rng.standard_normal(hv) * 0.2, dtype=torch.float32)
    cu = torch.tensor([0, L0], dtype=torch.int32)
    q, k, v, g, beta = gdn.prepare(x[:L0].cuda(), w.cuda(), a[:L0].cuda(), b[:L0].cuda(),
                                   A_log.cuda(), dt_bias.cuda(), cu.cuda(), hqk, d, hv, d,
                                   qkv_dtype=torch.float32)
    _, state = gdn.chunk_forward(q, k, v, g, beta, cu.cuda(), out_dtype=torch.float32)
    window = x[L0 - 3:L0].T.contiguous().unsqueeze(0).cuda()
    outs = [gdn.decode_step(x[t:t + 1].cuda(), window, w.cuda(), a[t:t + 1].cuda(),
                            b[t:t + 1].cuda(), A_log.cuda(), dt_bias.cuda(), state, hqk, d, hv,
                            out_dtype=torch.float32)
            for t in range(L0, L)]
    torch.cuda.synchronize()
    got = torch.cat(outs).cpu()
    rq, rk, rv, rg, rb = oracle.prepare(f64(x), f64(w), f64(a), f64(b), f64(A_log),
                                        f64(dt_bias), [0, L], hqk, d, hv, d)
    ro, rh = oracle.recurrent(rq, rk, rv, rg, rb, [0, L])
    assert_rms_close(got, ro[L0:], TOL["f32"], "fused decode outputs after prefill")
    assert_rms_close(state.cpu(), rh, TOL["f32"], "state after fused decode")
    assert np.array_equal(f64(window[0]), f64(x[L - 3:L]).T)


def test_decode_step_fused_full_size_sampled():
    """256 sequences of the 35B-A3B shape (16 QK / 32 V heads, d = 128, 537 MB state): outputs,
    states and windows of 6 sampled sequences against the oracle."""
    import synthetic_inputs as si

    dc = si.make_decode_front_case(256, 16, 32, 128, 128, seed=1007)
    dev = "cuda"
    x, win, w, a, b = (t.to(dev) for t in (dc.mixed_qkv, dc.window, dc.conv_weight, dc.a, dc.b))
    A_log, dt_bias, state = dc.A_log.to(dev), dc.dt_bias.to(dev), dc.h0.to(dev)
    o = gdn.decode_step(x, win, w, a, b, A_log, dt_bias, state, 16, 128, 32)
    torch.cuda.synchronize()
    rows = [0, 1, 77, 128, 200, 255]
    sel = torch.tensor(rows)
    ro, rh, rwin = _decode_oracle(dc.mixed_qkv[sel], dc.window[sel], dc.conv_weight, None,
                                  dc.a[sel], dc.b[sel], dc.A_log, dc.dt_bias, dc.h0[sel], 16, 32,
                                  128)
    assert_rms_close_rounded_out(o[sel.cuda()].cpu(), ro, TOL["f32"], "fused decode 256x1 o")
    assert_rms_close(state[sel.cuda()].cpu(), rh, TOL["f32"], "fused decode 256x1 state")
    assert np.array_equal(f64(win[sel.cuda()].cpu()), rwin)


# ---- output gate fused into the decode step ---------------------------------------------------

def _gate_inputs(rng, N, hv, d, zdt, form):
    z = _rand(rng, (N, hv, d), _DT[zdt], 1.5)
    if form == "none":
        return z, None, 0.0
    if form == "plus1":
        return z, torch.tensor(rng.standard_normal(d) * 0.1, dtype=torch.float32), 1.0
    return z, torch.tensor(rng.uniform(0.5, 1.5, d), dtype=torch.float32), 0.0


@pytest.mark.parametrize("d,dt,G,sdt", [(32, "f32", 1, "f32"), (64, "bf16", 2, "f32"),
                                        (128, "bf16", 2, "f32"), (128, "f32", 3, "bf16"),
                                        (128, "bf16", 4, "bf16")])
def test_recurrent_step_gated_against_oracle(d, dt, G, sdt):
    """The fused step + output gate against the float64 oracle's recurrence followed by its
    output gate. Every value the oracle does not see is an fp32 intermediate: the fp32 bar (a
    bf16 state is stored as the RNE cast of the fp32 state: its own rounding is allowed)."""
    rng = np.random.default_rng(900 + d + G)
    N, hqk = 13, 2
    hv = hqk * G
    q = torch.nn.functional.normalize(torch.from_numpy(rng.standard_normal((N, hqk, d))), dim=-1)
    k = torch.nn.functional.normalize(torch.from_numpy(rng.standard_normal((N, hqk, d))), dim=-1)
    q, k = q.to(_DT[dt]), k.to(_DT[dt])
    v = _rand(rng, (N, hv, d), _DT[dt])
    g = torch.from_numpy(-rng.uniform(0.0, 2.0, (N, hv))).float()
    beta = torch.from_numpy(rng.uniform(0.0, 1.0, (N, hv))).float()
    h0 = _rand(rng, (N, hv, d, d), _DT[sdt], 0.05)
    for zdt, form, odt in (("f32", "none", "f32"), ("bf16", "plus1", "f32"),
                           (dt, "plain", "bf16")):
        z, w, off = _gate_inputs(rng, N, hv, d, zdt, form)
        print(f"[step_gated] d={d} qkv={dt} G={G} state={sdt} z={zdt} weight={form} "
              f"out={odt}", flush=True)
        hd = h0.cuda()
        out = gdn.recurrent_step_gated(q.cuda(), k.cuda(), v.cuda(), g.cuda(), beta.cuda(), hd,
                                       z.cuda(), None if w is None else w.cuda(), off, 1e-6,
                                       scale=0.8, out_dtype=_DT[odt])
        torch.cuda.synchronize()
        ro, rh = oracle.recurrent(f64(q), f64(k), f64(v), f64(g), f64(beta), np.arange(N + 1),
                                  initial_state=f64(h0), scale=0.8)
        ref = oracle.gated_rmsnorm(ro, f64(z), f64(w), off, 1e-6)
        check = assert_rms_close_rounded_out if odt == "bf16" else assert_rms_close
        check(out, ref, TOL["f32"], "gated step out")
        scheck = assert_rms_close_rounded_out if sdt == "bf16" else assert_rms_close
        scheck(hd.cpu(), rh, TOL["f32"], "gated step state")


def test_recurrent_step_gated_matches_step_then_gate():
    """Fused gate = recurrent_step (fp32 o) followed by gdn_gated_rmsnorm, to fp32 rounding;
    the state update is the plain step's, bit for bit."""
    rng = np.random.default_rng(91)
    N, hqk, hv, d = 40, 4, 8, 128
    q = torch.nn.functional.normalize(torch.randn(N, hqk, d, dtype=torch.float64), dim=-1)
    k = torch.nn.functional.normalize(torch.randn(N, hqk, d, dtype=torch.float64), dim=-1)
    q, k = q.bfloat16().cuda(), k.bfloat16().cuda()
    v = _rand(rng, (N, hv, d), torch.bfloat16).cuda()
    g = torch.from_numpy(-rng.uniform(0.0, 2.0, (N, hv))).float().cuda()
    beta = torch.from_numpy(rng.uniform(0.0, 1.0, (N, hv))).float().cuda()
    h0 = _rand(rng, (N, hv, d, d), torch.float32, 0.02).cuda()
    z, w, off = _gate_inputs(rng, N, hv, d, "bf16", "plus1")
    z, w = z.cuda(), w.cuda()
    s1, s2 = h0.clone(), h0.clone()
    out1 = gdn.recurrent_step_gated(q, k, v, g, beta, s1, z, w, off, 1e-6,
                                    out_dtype=torch.float32)
    o2 = gdn.recurrent_step(q, k, v, g, beta, s2, out_dtype=torch.float32)
    out2 = gdn.gated_rmsnorm(o2, z, w, off, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    assert_rms_close(out1.cpu(), f64(out2), 1e-5, "fused vs two-call gated out")


@pytest.mark.parametrize("d,dt,G,sdt", [(32, "f32", 1, "f32"), (128, "bf16", 2, "f32"),
                                        (64, "bf16", 3, "bf16"), (128, "f32", 4, "f32")])
def test_decode_step_gated_against_oracle(d, dt, G, sdt):
    """Projected inputs to the gated mixer output in one kernel, against the oracle's front
    end, one recurrence step and its output gate (fp32 bar)."""
    rng = np.random.default_rng(950 + d + G)
    N, hqk = 17, 2
    hv = hqk * G
    x, win, wc, bc, a, b, A_log, dt_bias = _front(rng, N, hqk, hv, d, _DT[dt], bias=(G != 3))
    h0 = _rand(rng, (N, hv, d, d), _DT[sdt], 0.05)
    z, w, off = _gate_inputs(rng, N, hv, d, dt, "plus1" if G % 2 == 0 else "none")
    for odt in ("f32", dt):
        print(f"[decode_step_gated] d={d} {dt} G={G} state={sdt} out={odt}", flush=True)
        wd, hd = win.cuda(), h0.cuda()
        out = gdn.decode_step_gated(x.cuda(), wd, wc.cuda(), a.cuda(), b.cuda(), A_log.cuda(),
                                    dt_bias.cuda(), hd, z.cuda(), hqk, d, hv,
                                    weight=None if w is None else w.cuda(), weight_offset=off,
                                    conv_bias=None if bc is None else bc.cuda(), scale=0.7,
                                    out_dtype=_DT[odt])
        torch.cuda.synchronize()
        ro, rh, rwin = _decode_oracle(x, win, wc, bc, a, b, A_log, dt_bias, h0, hqk, hv, d,
                                      scale=0.7)
        ref = oracle.gated_rmsnorm(ro, f64(z), f64(w), off, 1e-6)
        check = assert_rms_close_rounded_out if odt == "bf16" else assert_rms_close
        check(out, ref, TOL["f32"], "gated decode out")
        scheck = assert_rms_close_rounded_out if sdt == "bf16" else assert_rms_close
        scheck(hd.cpu(), rh, TOL["f32"], "gated decode state")
        assert np.array_equal(f64(wd), rwin)


def test_decode_step_gated_full_size_sampled():
    """The benchmark's shape (256 sequences, 16 QK / 32 V heads, d = 128, bf16, fp32 state):
    the fused gated step equals the fused step followed by the gate kernel to fp32 rounding on
    every row, and the oracle on 6 sampled sequences."""
    rng = np.random.default_rng(1234)
    N, hqk, hv, d = 256, 16, 32, 128
    x, win, wc, bc, a, b, A_log, dt_bias = _front(rng, N, hqk, hv, d, torch.bfloat16, bias=False)
    h0 = _rand(rng, (N, hv, d, d), torch.float32, 0.02)
    z, w, off = _gate_inputs(rng, N, hv, d, "bf16", "plus1")
    dev = [t.cuda() for t in (x, win, wc, a, b, A_log, dt_bias, h0, z, w)]
    xd, w1, wcd, ad, bd, Ad, dtd, s1, zd, wd = dev
    w2, s2 = w1.clone(), s1.clone()
    out1 = gdn.decode_step_gated(xd, w1, wcd, ad, bd, Ad, dtd, s1, zd, hqk, d, hv, weight=wd,
                                 weight_offset=off, out_dtype=torch.float32)
    o2 = gdn.decode_step(xd, w2, wcd, ad, bd, Ad, dtd, s2, hqk, d, hv, out_dtype=torch.float32)
    out2 = gdn.gated_rmsnorm(o2, zd, wd, off, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(w1, w2)
    assert_rms_close(out1.cpu(), f64(out2), 1e-5, "fused gated vs step + gate (all rows)")
    seqs = rng.choice(N, size=6, replace=False)
    ro, rh, _ = _decode_oracle(x[seqs], win[seqs], wc, None, a[seqs], b[seqs], A_log, dt_bias,
                               h0[seqs], hqk, hv, d)
    ref = oracle.gated_rmsnorm(ro, f64(z[seqs]), f64(w), off, 1e-6)
    assert_rms_close(out1.cpu()[torch.from_numpy(seqs)], ref, TOL["f32"],
                     "gated decode out, sampled sequences")
