"""Pins of the oracle's front end (conv + SiLU, split, L2 norm, gates) against library
routines: numpy.convolve for the causal conv, scipy.special.expit for SiLU and the
sigmoid, numpy.linalg.norm for the normalisation and numpy.logaddexp for softplus."""

import numpy as np
from scipy.special import expit

import oracle


def _case(rng, lengths, hqk=2, hv=4, dk=8, dv=6, bias=True):
    T = sum(lengths)
    conv_dim = 2 * hqk * dk + hv * dv
    x = rng.standard_normal((T, conv_dim))
    w = rng.standard_normal((conv_dim, 4)) * 0.5
    b_conv = rng.standard_normal(conv_dim) * 0.1 if bias else None
    a = rng.standard_normal((T, hv))
    b = rng.standard_normal((T, hv)) * 3
    A_log = rng.uniform(0, 2.7, hv)
    dt_bias = rng.normal(0, 0.1, hv)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    return dict(x=x, w=w, bias=b_conv, a=a, b=b, A_log=A_log, dt_bias=dt_bias, cu=cu,
                hqk=hqk, hv=hv, dk=dk, dv=dv)


def _run(c, eps=1e-6):
    return oracle.prepare(c["x"], c["w"], c["a"], c["b"], c["A_log"], c["dt_bias"], c["cu"],
                          c["hqk"], c["dk"], c["hv"], c["dv"], conv_bias=c["bias"], l2_eps=eps)


def test_conv_silu_split_norm_against_numpy_convolve():
    rng = np.random.default_rng(1)
    c = _case(rng, [7, 1, 12])
    q, k, v, g, beta = _run(c)
    hqk, hv, dk, dv = c["hqk"], c["hv"], c["dk"], c["dv"]
    conv_dim = c["x"].shape[1]
    for n in range(3):
        s, e = c["cu"][n], c["cu"][n + 1]
        L = e - s
        y = np.zeros((L, conv_dim))
        for ch in range(conv_dim):
            # true convolution with the reversed taps = cross-correlation, zero history
            y[:, ch] = np.convolve(c["x"][s:e, ch], c["w"][ch, ::-1])[:L] + c["bias"][ch]
        y = y * expit(y)
        yq = y[:, :hqk * dk].reshape(L, hqk, dk)
        yk = y[:, hqk * dk:2 * hqk * dk].reshape(L, hqk, dk)
        yv = y[:, 2 * hqk * dk:].reshape(L, hv, dv)
        nq = np.sqrt(np.linalg.norm(yq, axis=-1, keepdims=True) ** 2 + 1e-6)
        nk = np.sqrt(np.linalg.norm(yk, axis=-1, keepdims=True) ** 2 + 1e-6)
        np.testing.assert_allclose(q[s:e], yq / nq, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(k[s:e], yk / nk, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(v[s:e], yv, rtol=1e-12, atol=1e-14)
    # unit norms up to eps: |q|^2 = s / (s + eps) <= 1
    nrm = np.linalg.norm(q, axis=-1)
    assert np.all(nrm <= 1.0) and np.allclose(nrm, 1.0, atol=1e-4)


def test_gates_against_library_sigmoid_softplus():
    rng = np.random.default_rng(2)
    c = _case(rng, [9, 4])
    _, _, _, g, beta = _run(c)
    np.testing.assert_allclose(beta, expit(c["b"]), rtol=1e-14)
    sp = np.logaddexp(0.0, c["a"] + c["dt_bias"][None, :])
    np.testing.assert_allclose(g, -np.exp(c["A_log"])[None, :] * sp, rtol=1e-13)
    assert np.all(g <= 0) and np.all((beta > 0) & (beta < 1))


def test_extreme_gate_inputs_stay_finite():
    rng = np.random.default_rng(3)
    c = _case(rng, [6])
    c["a"][:3] = [[-800.0] * 4, [800.0] * 4, [0.0] * 4]
    c["b"][:3] = [[-800.0] * 4, [800.0] * 4, [0.0] * 4]
    _, _, _, g, beta = _run(c)
    assert np.all(np.isfinite(g)) and np.all(np.isfinite(beta))
    assert np.all(g[0] == -0.0) or np.all(np.abs(g[0]) < 1e-300)
    np.testing.assert_allclose(g[1], -np.exp(c["A_log"]) * (800.0 + c["dt_bias"]), rtol=1e-14)
    assert np.all(beta[0] < 1e-300) and np.all(beta[1] == 1.0)


def test_no_leak_across_packed_sequences():
    rng = np.random.default_rng(4)
    lengths = [3, 5, 2]
    c = _case(rng, lengths, bias=False)
    full = _run(c)
    for n in range(3):
        s, e = c["cu"][n], c["cu"][n + 1]
        sub = dict(c, x=c["x"][s:e], a=c["a"][s:e], b=c["b"][s:e], cu=np.array([0, e - s]))
        part = _run(sub)
        for f, p in zip(full, part):
            assert np.array_equal(f[s:e], p)


def test_current_token_uses_last_tap():
    """A single token sees only tap 3 (the current position)."""
    rng = np.random.default_rng(5)
    c = _case(rng, [1], bias=False)
    q, k, v, _, _ = _run(c)
    y = c["x"][0] * c["w"][:, 3]
    y = y * expit(y)
    dq = c["hqk"] * c["dk"]
    np.testing.assert_allclose(v.reshape(-1), y[2 * dq:], rtol=1e-13)
