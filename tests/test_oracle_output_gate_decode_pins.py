"""Pins of the oracle's output gate (RMSNorm(o) * SiLU(z)) and decode-side front end (one token
per sequence with a cached conv window) to facts other than their own formulas.

Gated norm ([xiwon notes] "Qwen3_5MoeGatedDeltaNet" output stage; [MoE report] §3.3 stage 4 and
§7.5): scale invariance of RMSNorm, the zero gate, unit RMS of the normed vector, the closed
form on a constant vector, and the equivalence of the weight forms; SiLU(z) = z * sigmoid(z)
is taken from scipy's expit, not from the oracle.

Decode front end ([xiwon notes] "Cache"; [MoE report] §3.3 stage 2): stepping a sequence token
by token from an empty window must reproduce the (separately pinned) whole-sequence front end
at every row, and leave the last three inputs in the window.
"""

import numpy as np
import pytest
from scipy.special import expit

import oracle


def _silu(z):
    return z * expit(z)


@pytest.fixture(scope="module")
def rng():
    return np.random.default_rng(20261203)


def test_gated_norm_is_scale_invariant(rng):
    o = rng.standard_normal((5, 16))
    z = rng.standard_normal((5, 16))
    ref = oracle.gated_rmsnorm(o, z, eps=0.0)
    for lam in (0.1, 7.0):
        np.testing.assert_allclose(oracle.gated_rmsnorm(lam * o, z, eps=0.0), ref, rtol=1e-13)


def test_gated_norm_zero_gate_gives_zero(rng):
    o = rng.standard_normal((3, 8))
    assert np.all(oracle.gated_rmsnorm(o, np.zeros_like(o)) == 0.0)


def test_gated_norm_unit_rms(rng):
    # eps = 0, no weight, one gate value per row: out / SiLU(Z) has mean square exactly 1
    o = rng.standard_normal((6, 32)) * rng.uniform(0.1, 10.0, size=(6, 1))
    Z = rng.uniform(-3.0, 3.0, size=(6, 1)) + 0.5
    out = oracle.gated_rmsnorm(o, np.broadcast_to(Z, o.shape), eps=0.0)
    ms = np.mean((out / _silu(Z)) ** 2, axis=1)
    np.testing.assert_allclose(ms, 1.0, rtol=1e-13)
    # and the direction of o is kept
    assert np.all(np.sign(out / _silu(Z)) == np.sign(o))


def test_gated_norm_constant_vector_closed_form():
    dv, eps = 8, 1e-3
    w = np.linspace(-0.5, 0.5, dv)
    for c in (-2.0, 0.3):
        for Z in (-1.5, 0.0, 2.0):
            o = np.full((1, dv), c)
            z = np.full((1, dv), Z)
            out = oracle.gated_rmsnorm(o, z, weight=w, weight_offset=1.0, eps=eps)
            expect = c / np.sqrt(c * c + eps) * (1.0 + w) * _silu(Z)
            np.testing.assert_allclose(out[0], expect, rtol=1e-13, atol=1e-15)


def test_gated_norm_weight_forms(rng):
    o = rng.standard_normal((4, 16))
    z = rng.standard_normal((4, 16))
    none = oracle.gated_rmsnorm(o, z)
    np.testing.assert_allclose(oracle.gated_rmsnorm(o, z, weight=np.zeros(16), weight_offset=1.0),
                               none, rtol=1e-14)
    np.testing.assert_allclose(oracle.gated_rmsnorm(o, z, weight=np.ones(16)), none, rtol=1e-14)
    np.testing.assert_allclose(oracle.gated_rmsnorm(o, z, weight=np.full(16, 2.0)), 2 * none,
                               rtol=1e-14)


def _front_case(rng, L, hqk=2, hv=4, d=8, bias=True):
    conv_dim = 2 * hqk * d + hv * d
    x = rng.standard_normal((L, conv_dim))
    w = rng.standard_normal((conv_dim, 4)) * 0.5
    b_conv = rng.standard_normal(conv_dim) * 0.1 if bias else None
    a = rng.standard_normal((L, hv))
    b = rng.standard_normal((L, hv))
    A_log = rng.uniform(-1.0, 1.0, hv)
    dt_bias = rng.standard_normal(hv) * 0.2
    return x, w, b_conv, a, b, A_log, dt_bias, hqk, hv, d


@pytest.mark.parametrize("L", [1, 2, 3, 7])
def test_decode_steps_reproduce_whole_sequence_front_end(rng, L):
    x, w, bc, a, b, A_log, dt_bias, hqk, hv, d = _front_case(rng, L)
    q, k, v, g, beta = oracle.prepare(x, w, a, b, A_log, dt_bias, [0, L], hqk, d, hv, d,
                                      conv_bias=bc)
    win = np.zeros((1, x.shape[1], 3))
    for t in range(L):
        qs, ks, vs, gs, bs, win = oracle.decode_prepare(
            x[t:t + 1], win, w, a[t:t + 1], b[t:t + 1], A_log, dt_bias, hqk, d, hv, d,
            conv_bias=bc)
        np.testing.assert_allclose(qs[0], q[t], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(ks[0], k[t], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(vs[0], v[t], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(gs[0], g[t], rtol=1e-12)
        np.testing.assert_allclose(bs[0], beta[t], rtol=1e-12)
    # the window holds the last three inputs, oldest first, zeros before the sequence start
    hist = np.zeros((3, x.shape[1]))
    last = x[max(0, L - 3):L]
    hist[3 - last.shape[0]:] = last
    np.testing.assert_array_equal(win[0], hist.T)


def test_decode_prepare_batch_of_sequences(rng):
    # three sequences at different positions: each row matches its own whole-sequence front end
    Ls = [5, 1, 9]
    cases = [_front_case(rng, L, bias=False) for L in Ls]
    _, w, _, _, _, A_log, dt_bias, hqk, hv, d = cases[0]
    xs, wins, a_last, b_last, expect = [], [], [], [], []
    for (x, _, _, a, b, _, _, _, _, _), L in zip(cases, Ls):
        q, k, v, g, beta = oracle.prepare(x, w, a, b, A_log, dt_bias, [0, L], hqk, d, hv, d)
        hist = np.zeros((3, x.shape[1]))
        prev = x[max(0, L - 4):L - 1]
        hist[3 - prev.shape[0]:] = prev
        xs.append(x[L - 1])
        wins.append(hist.T)
        a_last.append(a[L - 1])
        b_last.append(b[L - 1])
        expect.append((q[L - 1], k[L - 1], v[L - 1], g[L - 1], beta[L - 1]))
    got = oracle.decode_prepare(np.stack(xs), np.stack(wins), w, np.stack(a_last),
                                np.stack(b_last), A_log, dt_bias, hqk, d, hv, d)
    for n in range(len(Ls)):
        for gi, ei in zip(got[:5], expect[n]):
            np.testing.assert_allclose(gi[n], ei, rtol=1e-12, atol=1e-14)
