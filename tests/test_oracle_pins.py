"""Pins of the float64 oracle's core recurrence against values it does not compute.

Each test compares ``oracle.recurrent`` (token-by-token, in C) with a different
route to the same numbers: a dense closed form solved by LAPACK, the chunked
WY/UT form of the MoE report's §3.7 at several chunk sizes, the matrix form
of the gated delta rule S_t = a S (I - b k k^T) + b v k^T, closed forms of special cases,
and exact rational arithmetic. A dropped decay, a wrong sign, a transposed state
or a wrong GQA index fails at least one of them.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle


def _rand_chain(rng, T, dk, dv, g_low=-0.5, unit=True):
    q = rng.standard_normal((T, 1, dk))
    k = rng.standard_normal((T, 1, dk))
    if unit:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, 1, dv))
    g = rng.uniform(g_low, 0.0, size=(T, 1))
    beta = rng.uniform(0.0, 1.0, size=(T, 1))
    h0 = rng.standard_normal((1, 1, dk, dv)) * 0.5
    return q, k, v, g, beta, h0


def _rel(a, b):
    return np.max(np.abs(a - b)) / np.sqrt(np.mean(b * b))


def test_dense_closed_form_lapack():
    """Whole sequence as one block: (I + A) U = diag(b) V - diag(b g) K H0, solved by LAPACK."""
    rng = np.random.default_rng(11)
    T, dk, dv, scale = 200, 16, 12, 0.7
    q, k, v, g, beta, h0 = _rand_chain(rng, T, dk, dv)
    o, ht = oracle.recurrent(q, k, v, g, beta, [0, T], initial_state=h0, scale=scale)
    Q, K, V, H0 = q[:, 0], k[:, 0], v[:, 0], h0[0, 0]
    gg, bb = g[:, 0], beta[:, 0]
    csum = np.cumsum(gg)
    gam = np.exp(csum)
    diff = csum[:, None] - csum[None, :]
    lower_incl = np.tril(np.ones((T, T), dtype=bool))
    Gam = np.where(lower_incl, np.exp(np.where(lower_incl, diff, 0.0)), 0.0)
    A = np.tril(bb[:, None] * Gam * (K @ K.T), -1)
    rhs = bb[:, None] * V - (bb * gam)[:, None] * (K @ H0)
    U = np.linalg.solve(np.eye(T) + A, rhs)
    O = scale * (gam[:, None] * (Q @ H0) + ((Q @ K.T) * Gam) @ U)
    HT = gam[-1] * H0 + (Gam[-1][:, None] * K).T @ U
    assert _rel(o[:, 0], O) < 1e-10
    assert _rel(ht[0, 0], HT) < 1e-10


def _chunked_wy(q, k, v, g, beta, h0, C, scale):
    """Chunked WY/UT form (MoE report §3.7 steps 2-7), padded with identity steps."""
    T, dk = q.shape
    dv = v.shape[1]
    pad = (C - T % C) % C
    padz = lambda x: np.concatenate([x, np.zeros((pad,) + x.shape[1:])], axis=0)  # noqa: E731
    q, k, v, g, beta = (padz(x) for x in (q, k, v, g, beta))
    H = h0.copy()
    out = np.zeros((T + pad, dv))
    tril_incl = np.tril(np.ones((C, C), dtype=bool))
    for c0 in range(0, T + pad, C):
        sl = slice(c0, c0 + C)
        Q, K, V, gg, bb = q[sl], k[sl], v[sl], g[sl], beta[sl]
        b = np.cumsum(gg)
        diff = np.where(tril_incl, b[:, None] - b[None, :], -np.inf)  # mask before exp
        Gam = np.exp(diff)
        A = np.tril(bb[:, None] * Gam * (K @ K.T), -1)
        # unit-lower-triangular inverse by forward substitution, row by row
        Tm = np.eye(C)
        for i in range(1, C):
            Tm[i, :i] = -A[i, :i] @ Tm[:i, :i]
        W = Tm @ ((bb * np.exp(b))[:, None] * K)
        U = Tm @ (bb[:, None] * V)
        Vn = U - W @ H
        out[sl] = scale * (np.exp(b)[:, None] * (Q @ H) + ((Q @ K.T) * Gam) @ Vn)
        H = np.exp(b[-1]) * H + (np.exp(b[-1] - b)[:, None] * K).T @ Vn
    return out[:T], H


@pytest.mark.parametrize("C", [1, 5, 16, 64])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 130])
def test_chunked_wy_form_equals_recurrence(C, T):
    rng = np.random.default_rng(100 + 7 * C + T)
    q, k, v, g, beta, h0 = _rand_chain(rng, T, 8, 6, g_low=-0.3)
    o, ht = oracle.recurrent(q, k, v, g, beta, [0, T], initial_state=h0, scale=1.3)
    O, H = _chunked_wy(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], h0[0, 0], C, 1.3)
    assert _rel(o[:, 0], O) < 1e-10
    assert _rel(ht[0, 0], H) < 1e-10


def test_delta_rule_matrix_form():
    """S_t = a_t S_{t-1} (I - b_t k k^T) + b_t v k^T,  o_t = S_t q_t  with S = H^T."""
    rng = np.random.default_rng(5)
    T, dk, dv = 50, 7, 9
    q, k, v, g, beta, h0 = _rand_chain(rng, T, dk, dv)
    o, ht = oracle.recurrent(q, k, v, g, beta, [0, T], initial_state=h0)
    S = h0[0, 0].T.copy()
    for t in range(T):
        kt, vt = k[t, 0], v[t, 0]
        S = np.exp(g[t, 0]) * S @ (np.eye(dk) - beta[t, 0] * np.outer(kt, kt)) \
            + beta[t, 0] * np.outer(vt, kt)
        assert np.allclose(o[t, 0], S @ q[t, 0], rtol=0, atol=1e-12)
    assert np.allclose(ht[0, 0], S.T, rtol=0, atol=1e-12)


def test_beta_zero_only_decays():
    """beta = 0: H_t = (prod of alphas) H0 and o_t = (prod alphas) H0^T q_t."""
    rng = np.random.default_rng(3)
    T, dk, dv = 40, 10, 6
    q, k, v, g, beta, h0 = _rand_chain(rng, T, dk, dv)
    beta[:] = 0.0
    o, ht = oracle.recurrent(q, k, v, g, beta, [0, T], initial_state=h0)
    decay = np.exp(np.cumsum(g[:, 0]))
    expect = decay[:, None] * (q[:, 0] @ h0[0, 0])
    assert _rel(o[:, 0], expect) < 1e-12
    assert _rel(ht[0, 0], decay[-1] * h0[0, 0]) < 1e-12


def test_exact_retrieval_orthonormal_keys():
    """alpha = 1, beta = 1, orthonormal keys, H0 = 0: H_n^T k_i = v_i for every stored key,
    and reading with q_t = k_t right after the write returns v_t."""
    rng = np.random.default_rng(9)
    dk, dv, n = 16, 5, 12
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:, :n].T.copy()                       # n orthonormal rows
    v = rng.standard_normal((n, 1, dv))
    k = keys[:, None, :]
    g = np.zeros((n, 1))
    beta = np.ones((n, 1))
    o, ht = oracle.recurrent(k, k, v, g, beta, [0, n])
    H = ht[0, 0]
    assert np.max(np.abs(keys @ H - v[:, 0])) < 1e-12
    assert np.max(np.abs(o[:, 0] - v[:, 0])) < 1e-12


def test_identity_steps_pass_state_through():
    """g = 0, beta = 0 leave the state bit-exact and o_t = H0^T q_t."""
    rng = np.random.default_rng(4)
    T, dk, dv = 33, 8, 8
    q, k, v, g, beta, h0 = _rand_chain(rng, T, dk, dv)
    g[:] = 0.0
    beta[:] = 0.0
    o, ht = oracle.recurrent(q, k, v, g, beta, [0, T], initial_state=h0)
    assert np.array_equal(ht, h0)
    assert _rel(o[:, 0], q[:, 0] @ h0[0, 0]) < 1e-14


def test_scalar_case_exact_rationals():
    """d_k = d_v = 1: s_t = a s (1 - b k^2) + b v k, o_t = s_t q_t; checked against exact
    rational arithmetic for three steps (alphas chosen as exp of a logarithm)."""
    alphas = [Fraction(1, 2), Fraction(3, 4), Fraction(7, 8)]
    betas = [Fraction(1, 4), Fraction(1, 2), Fraction(3, 4)]
    ks = [Fraction(1), Fraction(-1), Fraction(1)]
    vs = [Fraction(3, 2), Fraction(-5, 4), Fraction(2)]
    qs = [Fraction(-1), Fraction(1), Fraction(1)]
    s = Fraction(1, 3)
    exact_o = []
    for a, b, kk, vv, qq in zip(alphas, betas, ks, vs, qs):
        s = a * s * (1 - b * kk * kk) + b * vv * kk
        exact_o.append(s * qq)
    q = np.array([[[float(x)]] for x in qs])
    k = np.array([[[float(x)]] for x in ks])
    v = np.array([[[float(x)]] for x in vs])
    g = np.log(np.array([[float(a)] for a in alphas]))
    beta = np.array([[float(b)] for b in betas])
    o, ht = oracle.recurrent(q, k, v, g, beta, [0, 3], initial_state=np.array([[[[1 / 3]]]]))
    for t in range(3):
        assert abs(o[t, 0, 0] - float(exact_o[t])) < 1e-14
    assert abs(ht[0, 0, 0, 0] - float(s)) < 1e-14


def test_gqa_is_repeat_interleave():
    """V head h reads QK head h // G: same as repeat_interleave of q, k on the head axis."""
    rng = np.random.default_rng(21)
    T, hqk, G, dk, dv = 20, 2, 3, 6, 4
    hv = hqk * G
    q = rng.standard_normal((T, hqk, dk))
    k = rng.standard_normal((T, hqk, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, hv, dv))
    g = rng.uniform(-0.3, 0, (T, hv))
    beta = rng.uniform(0, 1, (T, hv))
    h0 = rng.standard_normal((1, hv, dk, dv))
    o1, h1 = oracle.recurrent(q, k, v, g, beta, [0, T], initial_state=h0)
    o2, h2 = oracle.recurrent(np.repeat(q, G, axis=1), np.repeat(k, G, axis=1), v, g, beta,
                              [0, T], initial_state=h0)
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)
    # and not the tiled (h % Hqk) mapping
    o3, _ = oracle.recurrent(np.tile(q, (1, G, 1)), np.tile(k, (1, G, 1)), v, g, beta, [0, T],
                             initial_state=h0)
    assert not np.allclose(o1, o3)


def test_varlen_packing_equals_separate_runs():
    rng = np.random.default_rng(8)
    lengths = [5, 0, 17, 1, 64]
    T = sum(lengths)
    hqk, hv, dk, dv = 1, 2, 6, 5
    q = rng.standard_normal((T, hqk, dk))
    k = rng.standard_normal((T, hqk, dk))
    v = rng.standard_normal((T, hv, dv))
    g = rng.uniform(-0.3, 0, (T, hv))
    beta = rng.uniform(0, 1, (T, hv))
    h0 = rng.standard_normal((len(lengths), hv, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lengths)])
    o, ht = oracle.recurrent(q, k, v, g, beta, cu, initial_state=h0)
    for n in range(len(lengths)):
        s, e = cu[n], cu[n + 1]
        on, hn = oracle.recurrent(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e], [0, e - s],
                                  initial_state=h0[n:n + 1])
        assert np.array_equal(o[s:e], on)
        assert np.array_equal(ht[n], hn[0])
    assert np.array_equal(ht[1], h0[1])   # empty sequence returns its initial state


def test_state_handoff_and_scale_linearity():
    rng = np.random.default_rng(12)
    T, T1 = 70, 29
    q, k, v, g, beta, h0 = _rand_chain(rng, T, 8, 8)
    o, ht = oracle.recurrent(q, k, v, g, beta, [0, T], initial_state=h0)
    oa, ha = oracle.recurrent(q[:T1], k[:T1], v[:T1], g[:T1], beta[:T1], [0, T1],
                              initial_state=h0)
    ob, hb = oracle.recurrent(q[T1:], k[T1:], v[T1:], g[T1:], beta[T1:], [0, T - T1],
                              initial_state=ha)
    assert np.array_equal(np.concatenate([oa, ob]), o)
    assert np.array_equal(hb, ht)
    o2, _ = oracle.recurrent(q, k, v, g, beta, [0, T], initial_state=h0, scale=0.25)
    assert np.array_equal(o2, 0.25 * o)


def test_bad_arguments_rejected():
    q = np.zeros((4, 2, 3))
    v = np.zeros((4, 3, 3))
    g = np.zeros((4, 3))
    with pytest.raises(ValueError):  # 3 V heads do not split over 2 QK heads
        oracle.recurrent(q, q, v, g, g, [0, 4])
