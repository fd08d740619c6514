"""GPU parity of the bf16 recurrent state against the float64 oracle.

A bf16 state is read exactly, carried in fp32 inside a call and stored as the round-to-nearest-
even cast of the fp32 state. Bars:
* one step (decode) or one prefill call from a bf16 state: every value the oracle does not see is
  an fp32 intermediate except the stored state itself, so outputs meet the fp32 bar (1e-4 * RMS,
  fp32 outputs; bf16 inputs of the chunked path: the bf16 bar) and the stored state meets the
  same bar on top of its own rounding (one bf16 ulp of the reference);
* many steps: the rounding of the stored state accumulates. The bar of each checked step is an
  error model of the storage format (float64 arithmetic, state stored through RNE bf16 after each
  step, same inputs) times 1.25 plus the fp32 bar; the same run with an fp32 state meets the fp32
  bar.
"""

import numpy as np
import pytest
import torch

import gated_deltanet_linear_amd as gdn
import oracle
import synthetic_inputs as si
from gdn_testutil import (TOL, assert_rms_close, assert_rms_close_rounded_out,
                          decode_state_storage_model, f64, rel_err)

pytestmark = pytest.mark.gpu


def _bf16_state(rng, shape, std):
    return torch.from_numpy(rng.standard_normal(shape) * std).to(torch.bfloat16)


@pytest.mark.parametrize("d,dt", [(32, torch.float32), (64, torch.bfloat16),
                                  (128, torch.bfloat16), (128, torch.float32)])
def test_recurrent_step_bf16_state_one_step(d, dt):
    rng = np.random.default_rng(900 + d)
    N, hqk, hv = 21, 2, 4
    case = si.make_core_case([1] * N, hqk, hv, d, d, dtype="f32" if dt == torch.float32 else "bf16",
                             seed=900 + d)
    h0 = _bf16_state(rng, (N, hv, d, d), 0.05)
    st = h0.cuda()
    print(f"[bf16 state step] d={d} {dt}", flush=True)
    o = gdn.recurrent_step(case.q.cuda(), case.k.cuda(), case.v.cuda(), case.g.cuda(),
                           case.beta.cuda(), st, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rh = oracle.recurrent(f64(case.q), f64(case.k), f64(case.v), f64(case.g), f64(case.beta),
                              np.arange(N + 1), initial_state=f64(h0))
    assert st.dtype == torch.bfloat16
    assert_rms_close(o, ro, TOL["f32"], "o from a bf16 state")
    assert_rms_close_rounded_out(st.cpu(), rh, TOL["f32"], "stored bf16 state")


@pytest.mark.parametrize("G", [1, 2])
def test_decode_step_fused_bf16_state(G):
    rng = np.random.default_rng(950 + G)
    N, hqk, d = 17, 2, 128
    hv = hqk * G
    conv_dim = (2 * hqk + hv) * d
    x = torch.from_numpy(rng.standard_normal((N, conv_dim))).to(torch.bfloat16)
    win = torch.from_numpy(rng.standard_normal((N, conv_dim, 3))).to(torch.bfloat16)
    w = torch.from_numpy(rng.standard_normal((conv_dim, 4)) * 0.5).to(torch.bfloat16)
    a = torch.from_numpy(rng.standard_normal((N, hv))).to(torch.bfloat16)
    b = torch.from_numpy(rng.standard_normal((N, hv))).to(torch.bfloat16)
    A_log = torch.tensor(rng.uniform(0.0, 2.7, hv), dtype=torch.float32)
    dt_bias = torch.tensor(rng.standard_normal(hv) * 0.1, dtype=torch.float32)
    h0 = _bf16_state(rng, (N, hv, d, d), 0.02)
    st, wd = h0.cuda(), win.cuda()
    o = gdn.decode_step(x.cuda(), wd, w.cuda(), a.cuda(), b.cuda(), A_log.cuda(), dt_bias.cuda(),
                        st, hqk, d, hv, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rq, rk, rv, rg, rb, rwin = oracle.decode_prepare(
        f64(x), f64(win), f64(w), f64(a), f64(b), f64(A_log), f64(dt_bias), hqk, d, hv, d)
    ro, rh = oracle.recurrent(rq, rk, rv, rg, rb, np.arange(N + 1), initial_state=f64(h0))
    assert_rms_close(o, ro, TOL["f32"], "fused o from a bf16 state")
    assert_rms_close_rounded_out(st.cpu(), rh, TOL["f32"], "fused stored bf16 state")
    assert np.array_equal(f64(wd), rwin)


def _multi_step_errors(case, h0, steps_checked):
    """Run len(T) decode steps (one token per sequence per step) with a bf16 state and with an
    fp32 state; return the errors against the float64 oracle at the checked step counts."""
    N = case.h0.shape[0] if case.h0 is not None else h0.shape[0]
    T = case.q.shape[0] // N  # tokens per sequence, laid out token-major: row = t * N + n
    st16, st32 = h0.to(torch.bfloat16).cuda(), h0.float().cuda()
    q, k, v, g, beta = (getattr(case, a).cuda() for a in ("q", "k", "v", "g", "beta"))
    outs16, outs32 = [], []
    for t in range(T):
        sl = slice(t * N, (t + 1) * N)
        outs16.append(gdn.recurrent_step(q[sl], k[sl], v[sl], g[sl], beta[sl], st16,
                                         out_dtype=torch.float32))
        outs32.append(gdn.recurrent_step(q[sl], k[sl], v[sl], g[sl], beta[sl], st32,
                                         out_dtype=torch.float32))
    torch.cuda.synchronize()
    o16 = torch.stack(outs16, 1).cpu()  # [N, T, hv, d]
    o32 = torch.stack(outs32, 1).cpu()
    # oracle per sequence: its tokens are rows n, N + n, 2N + n, ...
    perm = np.arange(T * N).reshape(T, N).T.reshape(-1)
    cu = np.arange(0, T * N + 1, T)
    ro, rh = oracle.recurrent(f64(case.q)[perm], f64(case.k)[perm], f64(case.v)[perm],
                              f64(case.g)[perm], f64(case.beta)[perm], cu,
                              initial_state=f64(h0.to(torch.bfloat16)))
    ro = ro.reshape(N, T, *ro.shape[1:])
    res = {}
    for s in steps_checked:
        res[s] = (rel_err(o16[:, s - 1], ro[:, s - 1]), rel_err(o32[:, s - 1], ro[:, s - 1]))
    res["state"] = (rel_err(st16.cpu(), rh), rel_err(st32.cpu(), rh))
    # the stored bf16 state beyond its own rounding (one bf16 ulp of the reference)
    rms = float(np.sqrt(np.mean(rh * rh)))
    res["state_beyond_ulp"] = float(np.max(np.abs(f64(st16.cpu()) - rh) - 2.0 ** -8 * np.abs(rh))) / rms
    return res


@pytest.mark.parametrize("gate", ["model", "slow"])
def test_bf16_state_many_decode_steps(gate):
    """256 decode steps of 16 sequences x 4 heads (d = 128) from and to a bf16 state. The bar at
    every checked step is the storage-error model of the bf16 state (float64 arithmetic with the
    state stored through round-to-nearest-even bf16 after every step, on the same inputs) times
    1.25, plus the fp32 bar for the kernel's own arithmetic; a truncating cast exceeds it (shown
    on the CPU in test_bf16_state_model). The same run with an fp32 state meets the fp32 bar."""
    N, hqk, hv, d, T = 16, 2, 4, 128, 256
    lengths = [N] * T  # T groups of N tokens; token t of sequence n is row t * N + n
    if gate == "model":
        case = si.make_core_case(lengths, hqk, hv, d, d, dtype="bf16", gate="model", seed=31)
    else:
        case = si.make_core_case(lengths, hqk, hv, d, d, dtype="bf16", gate="uniform",
                                 g_low=-0.01, seed=32)
    rng = np.random.default_rng(33)
    h0 = _bf16_state(rng, (N, hv, d, d), 0.02)
    steps = [1, 16, 64, 256]
    res = _multi_step_errors(case, h0, steps)
    # the storage-error model on the same inputs (CPU)
    perm = np.arange(T * N).reshape(T, N).T.reshape(-1)
    ro, rh = oracle.recurrent(f64(case.q)[perm], f64(case.k)[perm], f64(case.v)[perm],
                              f64(case.g)[perm], f64(case.beta)[perm], np.arange(0, T * N + 1, T),
                              initial_state=f64(h0))
    ro = ro.reshape(N, T, *ro.shape[1:])
    mo, mh = decode_state_storage_model(case, h0, N, T, "rne")
    rms = float(np.sqrt(np.mean(rh * rh)))
    model = {s: rel_err(mo[:, s - 1], ro[:, s - 1]) for s in steps}
    model["state"] = float(np.max(np.abs(mh - rh) - 2.0 ** -8 * np.abs(rh))) / rms
    bar = {key: 1.25 * e + TOL["f32"] for key, e in model.items()}
    for s in steps:
        print(f"  {gate} gates, step {s}: o max|err| bf16 state {res[s][0]:.3e} x RMS "
              f"(model {model[s]:.3e}, bar {bar[s]:.3e}), fp32 state {res[s][1]:.3e}", flush=True)
    print(f"  {gate} gates, final state beyond one ulp: bf16 {res['state_beyond_ulp']:.3e} "
          f"(model {model['state']:.3e}, bar {bar['state']:.3e}), fp32 {res['state'][1]:.3e}",
          flush=True)
    for s in steps:
        assert res[s][0] <= bar[s], f"{gate} step {s}: {res[s][0]:.3e} > {bar[s]:.3e}"
        assert res[s][1] <= TOL["f32"]
    assert res["state_beyond_ulp"] <= bar["state"]
    assert res["state"][1] <= TOL["f32"]


def test_prefill_bf16_state_then_decode():
    """Chunked prefill from a bf16 initial state writing a bf16 final state, then 4 decode steps on
    it: outputs and the final state against the oracle over the whole sequences."""
    rng = np.random.default_rng(41)
    lengths = [130, 64, 7]
    hqk, hv, d = 2, 4, 64
    pre = si.make_core_case(lengths, hqk, hv, d, d, dtype="bf16", gate="model", seed=41)
    n = len(lengths)
    h0 = _bf16_state(rng, (n, hv, d, d), 0.02)
    st = h0.cuda()
    o, ht = gdn.chunk_forward(pre.q.cuda(), pre.k.cuda(), pre.v.cuda(), pre.g.cuda(),
                              pre.beta.cuda(), pre.cu_seqlens.cuda(), initial_state=st,
                              final_state=st, out_dtype=torch.float32)
    assert ht.data_ptr() == st.data_ptr() and ht.dtype == torch.bfloat16
    dec = si.make_core_case([1] * (4 * n), hqk, hv, d, d, dtype="bf16", gate="model", seed=42)
    outs = []
    for t in range(4):
        sl = slice(t * n, (t + 1) * n)
        outs.append(gdn.recurrent_step(dec.q[sl].cuda(), dec.k[sl].cuda(), dec.v[sl].cuda(),
                                       dec.g[sl].cuda(), dec.beta[sl].cuda(), st,
                                       out_dtype=torch.float32))
    torch.cuda.synchronize()
    # oracle over each whole sequence: its prefill tokens, then its 4 decode tokens
    rows, cu = [], [0]
    for i, L in enumerate(lengths):
        rows.append(("pre", pre.cu_seqlens[i].item(), L))
        cu.append(cu[-1] + L + 4)
    cat = {a: [] for a in ("q", "k", "v", "g", "beta")}
    for i, (_, s0, L) in enumerate(rows):
        for a in cat:
            cat[a].append(f64(getattr(pre, a))[s0:s0 + L])
            cat[a].append(f64(getattr(dec, a))[[t * n + i for t in range(4)]])
    full = {a: np.concatenate(cat[a]) for a in cat}
    ro, rh = oracle.recurrent(full["q"], full["k"], full["v"], full["g"], full["beta"], cu,
                              initial_state=f64(h0))
    got_pre = o.cpu()
    ref_pre = np.concatenate([ro[cu[i]:cu[i] + L] for i, L in enumerate(lengths)])
    assert_rms_close(got_pre, ref_pre, TOL["bf16"], "prefill o from a bf16 state")
    got_dec = torch.stack(outs, 1).cpu()  # [n, 4, hv, d]
    ref_dec = np.stack([ro[cu[i] + L:cu[i] + L + 4] for i, L in enumerate(lengths)])
    assert_rms_close(got_dec, ref_dec, TOL["bf16"], "decode o after a bf16-state prefill")
    assert_rms_close_rounded_out(st.cpu(), rh, TOL["bf16"], "bf16 state after prefill + decode")
