"""Pins of the oracle's reverse mode (gdn_oracle_recurrent_backward) to facts other than its own
formulas: central finite differences of the (separately pinned) forward oracle, and special cases
where a gradient is exactly zero or has a closed form.

Loss: L = sum(o * dout) + sum(ht * dht). The directional derivative of L along a random direction,
by central differences in float64 (step 1e-6, truncation error ~1e-12 relative), must equal the
inner product of the oracle's gradient with that direction.
"""

import numpy as np
import pytest

import oracle


def _case(rng, lengths, hqk, hv, dk, dv, beta_zero=False):
    T = sum(lengths)
    q = rng.standard_normal((T, hqk, dk))
    k = rng.standard_normal((T, hqk, dk)) * 0.5
    v = rng.standard_normal((T, hv, dv))
    g = -rng.uniform(0.01, 0.8, (T, hv))
    beta = np.zeros((T, hv)) if beta_zero else rng.uniform(0.1, 0.9, (T, hv))
    n = len(lengths)
    h0 = rng.standard_normal((n, hv, dk, dv)) * 0.3
    cu = np.concatenate([[0], np.cumsum(lengths)])
    dout = rng.standard_normal((T, hv, dv))
    dht = rng.standard_normal((n, hv, dk, dv))
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=h0), cu, dout, dht


def _loss(x, cu, dout, dht, scale):
    o, ht = oracle.recurrent(x["q"], x["k"], x["v"], x["g"], x["beta"], cu,
                             initial_state=x["h0"], scale=scale)
    return float(np.sum(o * dout) + np.sum(ht * dht))


@pytest.mark.parametrize("lengths,hqk,hv,dk,dv", [([4, 3], 1, 2, 3, 2), ([5, 0, 6], 2, 4, 4, 3),
                                                 ([9], 1, 1, 5, 5)])
def test_backward_matches_finite_differences(lengths, hqk, hv, dk, dv):
    rng = np.random.default_rng(sum(lengths) * 7 + dk)
    x, cu, dout, dht = _case(rng, lengths, hqk, hv, dk, dv)
    scale = 0.8
    dq, dk_, dv_, dg, dbeta, dh0 = oracle.recurrent_backward(
        x["q"], x["k"], x["v"], x["g"], x["beta"], cu, dout, initial_state=x["h0"], dht=dht,
        scale=scale)
    grads = dict(q=dq, k=dk_, v=dv_, g=dg, beta=dbeta, h0=dh0)
    eps = 1e-6
    for name in ("q", "k", "v", "g", "beta", "h0"):
        d = rng.standard_normal(x[name].shape)
        xp = dict(x)
        xm = dict(x)
        xp[name] = x[name] + eps * d
        xm[name] = x[name] - eps * d
        fd = (_loss(xp, cu, dout, dht, scale) - _loss(xm, cu, dout, dht, scale)) / (2 * eps)
        an = float(np.sum(grads[name] * d))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), (name, fd, an)


def test_backward_single_entries_by_finite_differences():
    # entry by entry for the gate inputs (a wrong index shows up here even if a random direction
    # averages it out)
    rng = np.random.default_rng(5)
    x, cu, dout, dht = _case(rng, [6], 1, 2, 3, 3)
    _, _, _, dg, dbeta, _ = oracle.recurrent_backward(
        x["q"], x["k"], x["v"], x["g"], x["beta"], cu, dout, initial_state=x["h0"], dht=dht)
    eps = 1e-6
    for name, grad in (("g", dg), ("beta", dbeta)):
        for idx in np.ndindex(x[name].shape):
            xp, xm = dict(x), dict(x)
            xp[name] = x[name].copy()
            xm[name] = x[name].copy()
            xp[name][idx] += eps
            xm[name][idx] -= eps
            fd = (_loss(xp, cu, dout, dht, 1.0) - _loss(xm, cu, dout, dht, 1.0)) / (2 * eps)
            assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def test_backward_with_zero_beta_has_no_key_or_value_gradient():
    # beta = 0: nothing is written, so o and the final state do not depend on k or v at all
    rng = np.random.default_rng(6)
    x, cu, dout, dht = _case(rng, [5, 4], 1, 2, 4, 3, beta_zero=True)
    dq, dk_, dv_, dg, dbeta, dh0 = oracle.recurrent_backward(
        x["q"], x["k"], x["v"], x["g"], x["beta"], cu, dout, initial_state=x["h0"], dht=dht)
    assert np.all(dk_ == 0.0) and np.all(dv_ == 0.0)
    assert np.any(dbeta != 0.0)
    # and the state is pure decay: dh0 = sum_t scale * prod(alpha) q_t dout_t^T + prod(alpha) dht
    n0 = 5
    alpha = np.exp(x["g"][:n0, 0])
    ref = np.prod(alpha) * dht[0, 0]
    for t in range(n0):
        ref = ref + np.prod(alpha[:t + 1]) * np.outer(x["q"][t, 0], dout[t, 0])
    np.testing.assert_allclose(dh0[0, 0], ref, rtol=1e-12, atol=1e-14)


def test_backward_without_final_state_term():
    rng = np.random.default_rng(8)
    x, cu, dout, _ = _case(rng, [7], 1, 1, 3, 2)
    zeros = np.zeros_like(x["h0"])
    a = oracle.recurrent_backward(x["q"], x["k"], x["v"], x["g"], x["beta"], cu, dout,
                                  initial_state=x["h0"], dht=None)
    b = oracle.recurrent_backward(x["q"], x["k"], x["v"], x["g"], x["beta"], cu, dout,
                                  initial_state=x["h0"], dht=zeros)
    for ga, gb in zip(a, b):
        np.testing.assert_array_equal(ga, gb)
