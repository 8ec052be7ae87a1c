"""Pins of the Gated DeltaNet-2 oracle (CPU).

The recurrence ("Gated DeltaNet-2" summary, section 1):
    S_t = (I - k_t (b_t o k_t)^T) D_t S_{t-1} + k_t (w_t o v_t)^T,   o_t = S_t^T q_t
with an erase gate b_t per key channel and a write gate w_t per value channel.
Each pin below fixes the oracle against something other than its own code: a
hand-worked case, dense transition-matrix products, the KDA reduction the page
states (b = w = beta), the read-back property of a full erase, and the closed
form of the no-erase case.
"""
import os

import numpy as np
import pytest

import oracle
from test_oracle import GOLDEN, RTOL, _read_fixture


def _rand_gdn2(rng, T, dk, dv, ckda=True):
    q = rng.standard_normal((1, T, 1, dk))
    k = rng.standard_normal((1, T, 1, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, T, 1, dv))
    if ckda:
        a = np.tanh(2 * rng.standard_normal((1, T, 1, dk)))
        m = rng.random(a.shape) < 0.15
        a[m] = rng.choice([-1.0, 0.0, 1.0], size=int(m.sum()))
    else:
        a = np.exp(-0.1 * np.logaddexp(0, rng.standard_normal((1, T, 1, dk))))
    e = 1.0 / (1.0 + np.exp(-rng.standard_normal((1, T, 1, dk))))
    w = 1.0 / (1.0 + np.exp(-rng.standard_normal((1, T, 1, dv))))
    return q, k, v, a, e, w


def _dense_run(q, k, v, a, e, w, S0):
    """Brute force with dense d_k x d_k transition matrices
    A_t = (I - k_t (b_t o k_t)^T) Diag(alpha_t) and writes k_t (w_t o v_t)^T."""
    T, dk = k.shape
    S = S0.copy()
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        A = (np.eye(dk) - np.outer(k[t], e[t] * k[t])) @ np.diag(a[t])
        S = A @ S + np.outer(k[t], w[t] * v[t])
        o[t] = S.T @ q[t]
    return o, S


def test_gdn2_hand_derived_two_tokens():
    fx = _read_fixture("gdn2_hand_two_steps.txt")
    dk, dv = int(fx["dk"][0]), int(fx["dv"][0])
    toks = fx["tokens"]
    st = lambda key: np.stack([t[key] for t in toks])[None, :, None, :]
    q, k, v, a, e, w = (st(x) for x in ("q", "k", "v", "alpha", "erase", "write"))
    S0 = fx["S0"].reshape(1, dk, dv)
    o, S = oracle.fwd_gdn2(q, k, v, a, e, w, S0=S0)
    for t in range(len(toks)):
        np.testing.assert_allclose(o[0, t], toks[t]["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(S[0].ravel(), toks[-1]["S"], rtol=0, atol=1e-14)
    state = S0.astype(np.float64).copy()
    for t in range(len(toks)):
        od = oracle.decode_gdn2(q[:, t], k[:, t], v[:, t], a[:, t], e[:, t], w[:, t], state)
        np.testing.assert_allclose(od[0], toks[t]["o"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(state[0].ravel(), toks[t]["S"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("dk,dv,T", [(2, 3, 17), (3, 2, 32), (4, 4, 25), (3, 5, 9)])
def test_gdn2_explicit_transition_products(dk, dv, T):
    rng = np.random.default_rng(300 + dk * 10 + dv)
    q, k, v, a, e, w = _rand_gdn2(rng, T, dk, dv)
    S0 = rng.standard_normal((dk, dv))
    o, S = oracle.fwd_gdn2(q, k, v, a, e, w, S0=S0[None])
    o_ref, S_ref = _dense_run(*(x[0, :, 0] for x in (q, k, v, a, e, w)), S0)
    np.testing.assert_allclose(o[0], o_ref, rtol=0, atol=RTOL * max(1.0, np.abs(o_ref).max()))
    np.testing.assert_allclose(S[0], S_ref, rtol=0, atol=RTOL * max(1.0, np.abs(S_ref).max()))


def test_gdn2_with_tied_gates_is_kda():
    """b_t = w_t = beta_t (every channel) recovers KDA, the reduction the page states."""
    rng = np.random.default_rng(7)
    B, T, H, dk, dv = 2, 40, 3, 6, 5
    q, k, v, a, _, _ = _rand_gdn2(rng, T * B * H, dk, dv)
    resh = lambda x: x.reshape(B, T, H, -1)
    q, k, v, a = (resh(x) for x in (q, k, v, a))
    beta = 2.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    e = np.repeat(beta[..., None], dk, axis=-1)
    w = np.repeat(beta[..., None], dv, axis=-1)
    S0 = rng.standard_normal((B * H, dk, dv))
    o1, S1 = oracle.fwd_gdn2(q, k, v, a, e, w, S0=S0)
    o2, S2 = oracle.fwd(q, k, v, a, beta, S0=S0)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12 * max(1.0, np.abs(o2).max()))
    np.testing.assert_allclose(S1, S2, rtol=0, atol=1e-12 * max(1.0, np.abs(S2).max()))


def test_gdn2_full_erase_reads_back_the_write():
    """b = 1, alpha = 1, unit k: the step erases everything stored along k and writes
    w o v there, so S_t^T k_t = w_t o v_t exactly (for any earlier state)."""
    rng = np.random.default_rng(11)
    T, dk, dv = 30, 5, 4
    q, k, v, _, _, w = _rand_gdn2(rng, T, dk, dv)
    a = np.ones((1, T, 1, dk))
    e = np.ones((1, T, 1, dk))
    state = rng.standard_normal((1, dk, dv))
    for t in range(T):
        oracle.decode_gdn2(q[:, t], k[:, t], v[:, t], a[:, t], e[:, t], w[:, t], state)
        np.testing.assert_allclose(state[0].T @ k[0, t, 0], w[0, t, 0] * v[0, t, 0], rtol=0, atol=1e-13)


def test_gdn2_without_erase_is_a_decayed_sum_of_writes():
    """b = 0: S_T = Diag(prod alpha) S0 + sum_t Diag(prod_{m>t} alpha_m) k_t (w_t o v_t)^T."""
    rng = np.random.default_rng(12)
    T, dk, dv = 25, 4, 3
    q, k, v, a, _, w = _rand_gdn2(rng, T, dk, dv, ckda=True)
    e = np.zeros((1, T, 1, dk))
    S0 = rng.standard_normal((dk, dv))
    _, S = oracle.fwd_gdn2(q, k, v, a, e, w, S0=S0[None])
    aa, kk, vv, ww = a[0, :, 0], k[0, :, 0], v[0, :, 0], w[0, :, 0]
    ref = np.prod(aa, axis=0)[:, None] * S0
    for t in range(T):
        tail = np.prod(aa[t + 1:], axis=0) if t + 1 < T else np.ones(dk)
        ref += tail[:, None] * np.outer(kk[t], ww[t] * vv[t])
    np.testing.assert_allclose(S[0], ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max()))
