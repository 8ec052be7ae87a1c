"""Pins of the SFDA (phase-control) oracle (CPU).

The recurrence ("Resumen Tecnico: Atencion Delta de Fourier Semidirecta (SFDA)",
section "Arquitectura Central"):
    S_t = (I - beta_t k_t k_t^T) Lambda_t S_{t-1} + beta_t k_t v_t^T,   o_t = S_t^T q_t
with Lambda_t = diag(alpha_t o e^{i theta_t}) in complex coordinates, built in real
coordinates from 2 x 2 rotation-decay blocks: key channels (2p, 2p+1) are the real and
imaginary parts of coordinate p, and the gate lambda_p = alpha_p e^{i theta_p} arrives as
(Re, Im) in channels (2p, 2p+1) of the gate tensor.

Each pin fixes the oracle against something other than its own code: a hand-worked
case, dense real transition matrices, the KDA reduction the page states for zero phases,
numpy's complex products for pure rotation-decay, and an exact phase-only cyclic counter
(the page's "Expresividad de Estado Finito": phase-only SFDA realises cyclic counters).
"""
import numpy as np
import pytest

import oracle
from test_oracle import RTOL, _read_fixture


def _rand_sfda(rng, T, dk, dv, B=1, H=1, special=0.15):
    """fp64 inputs: unit keys, complex gates |lambda| <= 1 with exact zeros and quarter
    turns mixed in, beta in [0, 2]."""
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    mag = rng.uniform(0.0, 1.0, (B, T, H, dk // 2))
    th = rng.uniform(-np.pi, np.pi, mag.shape)
    lam = mag * np.exp(1j * th)
    m = rng.random(mag.shape) < special
    lam[m] = rng.choice(np.array([0, 1, -1, 1j, -1j]), size=int(m.sum()))
    gates = np.empty((B, T, H, dk))
    gates[..., 0::2], gates[..., 1::2] = lam.real, lam.imag
    beta = rng.uniform(0.0, 2.0, (B, T, H))
    return q, k, v, gates, beta


def _dense_lambda(g):
    """Dense real d_k x d_k block-diagonal matrix of the gates g[2p] + i g[2p+1]."""
    dk = g.shape[0]
    L = np.zeros((dk, dk))
    for p in range(dk // 2):
        re, im = g[2 * p], g[2 * p + 1]
        L[2 * p:2 * p + 2, 2 * p:2 * p + 2] = [[re, -im], [im, re]]
    return L


def _dense_run(q, k, v, g, beta, S0):
    """Brute force with dense transition matrices (I - beta k k^T) Lambda_t."""
    T, dk = k.shape
    S = S0.copy()
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        A = (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) @ _dense_lambda(g[t])
        S = A @ S + beta[t] * np.outer(k[t], v[t])
        o[t] = S.T @ q[t]
    return o, S


def test_sfda_hand_derived_two_tokens():
    fx = _read_fixture("sfda_hand_two_steps.txt")
    dk, dv = int(fx["dk"][0]), int(fx["dv"][0])
    toks = fx["tokens"]
    st = lambda key: np.stack([t[key] for t in toks])[None, :, None, :]
    q, k, v, lam = (st(x) for x in ("q", "k", "v", "lambda"))
    beta = np.array([t["beta"][0] for t in toks])[None, :, None]
    S0 = fx["S0"].reshape(1, dk, dv)
    o, S = oracle.fwd_sfda(q, k, v, lam, beta, S0=S0)
    for t in range(len(toks)):
        np.testing.assert_allclose(o[0, t], toks[t]["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(S[0].ravel(), toks[-1]["S"], rtol=0, atol=1e-14)
    state = S0.astype(np.float64).copy()
    for t in range(len(toks)):
        od = oracle.decode_sfda(q[:, t], k[:, t], v[:, t], lam[:, t], beta[:, t], state)
        np.testing.assert_allclose(od[0], toks[t]["o"], rtol=0, atol=1e-14)
        np.testing.assert_allclose(state[0].ravel(), toks[t]["S"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("dk,dv,T", [(2, 3, 17), (4, 2, 32), (6, 4, 25)])
def test_sfda_explicit_transition_products(dk, dv, T):
    rng = np.random.default_rng(500 + dk * 10 + dv)
    q, k, v, g, beta = _rand_sfda(rng, T, dk, dv)
    S0 = rng.standard_normal((dk, dv))
    o, S = oracle.fwd_sfda(q, k, v, g, beta, S0=S0[None])
    o_ref, S_ref = _dense_run(*(x[0, :, 0] for x in (q, k, v, g)), beta[0, :, 0], S0)
    np.testing.assert_allclose(o[0], o_ref, rtol=0, atol=RTOL * max(1.0, np.abs(o_ref).max()))
    np.testing.assert_allclose(S[0], S_ref, rtol=0, atol=RTOL * max(1.0, np.abs(S_ref).max()))


def test_sfda_with_zero_phases_is_kda_with_paired_decay():
    """Im lambda = 0 everywhere: Lambda = Diag(alpha) with both channels of a pair decayed
    by Re lambda -- the KDA recurrence, as the page's "Principales Contribuciones" item 1
    states for zero phases."""
    rng = np.random.default_rng(11)
    B, T, H, dk, dv = 2, 40, 3, 8, 5
    q, k, v, g, beta = _rand_sfda(rng, T, dk, dv, B=B, H=H)
    g[..., 1::2] = 0.0
    a = np.repeat(g[..., 0::2], 2, axis=-1)
    S0 = rng.standard_normal((B * H, dk, dv))
    o1, S1 = oracle.fwd_sfda(q, k, v, g, beta, S0=S0)
    o2, S2 = oracle.fwd(q, k, v, a, beta, S0=S0)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S1, S2, rtol=0, atol=1e-13)
    st1, st2 = S0.copy(), S0.copy()
    for t in range(3):
        d1 = oracle.decode_sfda(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], st1)
        d2 = oracle.decode(q[:, t], k[:, t], v[:, t], a[:, t], beta[:, t], st2)
        np.testing.assert_allclose(d1, d2, rtol=0, atol=1e-13)
        np.testing.assert_allclose(st1, st2, rtol=0, atol=1e-13)


def test_sfda_pure_rotation_decay_closed_form():
    """beta = 0: no erase, no write; coordinate p of every state column is multiplied by
    the running complex product of its gates (numpy complex128), and the readout is the
    real inner product of q with the rotated state."""
    rng = np.random.default_rng(12)
    T, dk, dv = 30, 6, 3
    q, k, v, g, _ = _rand_sfda(rng, T, dk, dv)
    beta = np.zeros((1, T, 1))
    S0 = rng.standard_normal((dk, dv))
    o, S = oracle.fwd_sfda(q, k, v, g, beta, S0=S0[None])
    lam = g[0, :, 0, 0::2] + 1j * g[0, :, 0, 1::2]        # [T, dk/2]
    z0 = S0[0::2] + 1j * S0[1::2]                          # [dk/2, dv]
    run = np.cumprod(lam, axis=0)                          # prod_{s <= t} lambda_s
    for t in range(T):
        zt = run[t][:, None] * z0
        St = np.empty((dk, dv))
        St[0::2], St[1::2] = zt.real, zt.imag
        np.testing.assert_allclose(o[0, t], St.T @ q[0, t, 0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(S[0, 0::2] + 1j * S[0, 1::2], run[-1][:, None] * z0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("n", [3, 5, 8])
def test_sfda_phase_only_cyclic_counter(n):
    """|lambda| = 1 with phase 2 pi / n and beta = 0: the state turns a full circle in n
    steps (a mod-n counter); with n even, half a circle negates it."""
    rng = np.random.default_rng(13 + n)
    dk, dv, T = 4, 3, 3 * n
    lam = np.exp(2j * np.pi / n)
    g = np.zeros((1, T, 1, dk))
    g[..., 0::2], g[..., 1::2] = lam.real, lam.imag
    q = rng.standard_normal((1, T, 1, dk))
    k = rng.standard_normal((1, T, 1, dk))
    v = rng.standard_normal((1, T, 1, dv))
    S0 = rng.standard_normal((1, dk, dv))
    beta = np.zeros((1, T, 1))
    for steps in (n, 2 * n, 3 * n):
        _, S = oracle.fwd_sfda(q[:, :steps], k[:, :steps], v[:, :steps], g[:, :steps], beta[:, :steps], S0=S0)
        np.testing.assert_allclose(S, S0, rtol=0, atol=1e-12)
    if n % 2 == 0:
        _, S = oracle.fwd_sfda(q[:, :n // 2], k[:, :n // 2], v[:, :n // 2], g[:, :n // 2], beta[:, :n // 2], S0=S0)
        np.testing.assert_allclose(S, -S0, rtol=0, atol=1e-12)
    # a quarter turn maps coordinate z to i z: row 2p <- -row 2p+1, row 2p+1 <- row 2p
    gq = np.zeros((1, 1, 1, dk))
    gq[..., 1::2] = 1.0
    _, S = oracle.fwd_sfda(q[:, :1], k[:, :1], v[:, :1], gq, beta[:, :1], S0=S0)
    np.testing.assert_array_equal(S[0, 0::2], -S0[0, 1::2])
    np.testing.assert_array_equal(S[0, 1::2], S0[0, 0::2])


def test_sfda_norm_never_grows_without_writes():
    """|lambda| <= 1, beta in [0, 2], unit keys, v = 0: every transition is a contraction
    (the 2 x 2 blocks scale by |lambda|, I - beta k k^T has eigenvalues 1 and 1 - beta)."""
    rng = np.random.default_rng(14)
    T, dk, dv = 50, 8, 4
    q, k, _, g, beta = _rand_sfda(rng, T, dk, dv)
    v = np.zeros((1, T, 1, dv))
    S = rng.standard_normal((1, dk, dv))
    prev = np.linalg.norm(S)
    for t in range(T):
        oracle.decode_sfda(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], S)
        cur = np.linalg.norm(S)
        assert cur <= prev * (1 + 1e-14)
        prev = cur


def test_sfda_split_and_heads():
    """fwd over T1 + T2 equals fwd over T2 from the state after T1, and a selection of
    heads equals the same heads run alone."""
    rng = np.random.default_rng(15)
    B, T, H, dk, dv = 2, 33, 3, 4, 3
    q, k, v, g, beta = _rand_sfda(rng, T, dk, dv, B=B, H=H)
    S0 = rng.standard_normal((B * H, dk, dv))
    o, S = oracle.fwd_sfda(q, k, v, g, beta, S0=S0)
    t1 = 14
    o1, S1 = oracle.fwd_sfda(q[:, :t1], k[:, :t1], v[:, :t1], g[:, :t1], beta[:, :t1], S0=S0)
    o2, S2 = oracle.fwd_sfda(q[:, t1:], k[:, t1:], v[:, t1:], g[:, t1:], beta[:, t1:], S0=S1)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(S2, S, rtol=0, atol=1e-13)
    sel = [4, 1]
    os_, Ss = oracle.fwd_sfda(q, k, v, g, beta, S0=S0[sel], heads=sel)
    np.testing.assert_array_equal(os_, o[sel])
    np.testing.assert_array_equal(Ss, S[sel])
