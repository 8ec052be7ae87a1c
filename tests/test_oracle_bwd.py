"""Pins of the oracle's backward (CPU).

The gradients are those of L = sum_t <dO_t, o_t> + <dS_T, S_T> through the forward
recurrence.  The pins use the forward oracle (itself pinned in test_oracle.py), never the
backward's own code:

* L is affine in each single entry of q, v, alpha, beta and S0 (each enters every
  state and output at most linearly), so the secant L(x + s e) - L(x) equals s times
  the gradient exactly, for any step s -- including at an exact zero gate, where a
  division-based log-derivative would be undefined;
* k enters quadratically, so its gradient is pinned by central finite differences;
* a one-token scalar case is checked against derivatives worked by hand.
"""
import numpy as np
import pytest

import oracle


def _inputs(rng, B, T, H, dk, dv, zeros=0.1):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    a = np.tanh(2 * rng.standard_normal((B, T, H, dk)))
    m = rng.random(a.shape) < zeros
    a[m] = rng.choice([-1.0, 0.0, 1.0], size=int(m.sum()))
    b = rng.uniform(0.0, 2.0, (B, T, H))
    S0 = rng.standard_normal((B * H, dk, dv))
    dO = rng.standard_normal((B * H, T, dv))
    dST = rng.standard_normal((B * H, dk, dv))
    return dict(q=q, k=k, v=v, alpha=a, beta=b, S0=S0), dO, dST


def _loss(x, dO, dST):
    o, S = oracle.fwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0=x["S0"])
    return float((o * dO).sum() + (S * dST).sum())


def _grads(x, dO, dST):
    return oracle.bwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dO, S0=x["S0"], dST=dST)


def _entry_grad(g, name, idx, H):
    """Gradient entry for input `name` at input index idx (inputs are [B, T, H, d])."""
    if name == "S0":
        return g["dS0"][idx]
    key = {"q": "dq", "k": "dk", "v": "dv", "alpha": "dalpha", "beta": "dbeta"}[name]
    b, t, h = idx[:3]
    return g[key][(b * H + h, t) + tuple(idx[3:])]


@pytest.mark.parametrize("T", [5, 150])
def test_bwd_exact_secants(T):
    """Affine inputs: a secant of any step equals the gradient (zero gates included)."""
    rng = np.random.default_rng(100 + T)
    B, H, dk, dv = 2, 2, 4, 3
    x, dO, dST = _inputs(rng, B, T, H, dk, dv)
    x["alpha"][0, 1, 0, 2] = 0.0   # exact zero gates, two in one channel
    x["alpha"][0, 3, 0, 2] = 0.0
    g = _grads(x, dO, dST)
    L0 = _loss(x, dO, dST)
    checked_zero = 0
    for name in ("q", "v", "alpha", "beta", "S0"):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in x[name].shape)
            if name == "alpha" and checked_zero < 2:  # make sure exact zero gates are covered
                z = np.argwhere(x["alpha"] == 0.0)
                if len(z):
                    idx = tuple(int(c) for c in z[int(rng.integers(0, len(z)))])
                    checked_zero += 1
            step = 0.75
            y = {kk: vv.copy() for kk, vv in x.items()}
            y[name][idx] += step
            sec = (_loss(y, dO, dST) - L0) / step
            ref = _entry_grad(g, name, idx, H)
            assert abs(sec - ref) <= 1e-9 * max(1.0, abs(ref)), (name, idx, sec, ref)
    assert checked_zero > 0


def test_bwd_key_central_differences():
    rng = np.random.default_rng(7)
    B, T, H, dk, dv = 1, 70, 2, 4, 3
    x, dO, dST = _inputs(rng, B, T, H, dk, dv)
    g = _grads(x, dO, dST)
    h = 1e-5
    for _ in range(12):
        idx = tuple(int(rng.integers(0, n)) for n in x["k"].shape)
        yp = {kk: vv.copy() for kk, vv in x.items()}
        ym = {kk: vv.copy() for kk, vv in x.items()}
        yp["k"][idx] += h
        ym["k"][idx] -= h
        fd = (_loss(yp, dO, dST) - _loss(ym, dO, dST)) / (2 * h)
        ref = _entry_grad(g, "k", idx, H)
        assert abs(fd - ref) <= 1e-6 * max(1.0, abs(ref)), (idx, fd, ref)


def test_bwd_scalar_token_by_hand():
    """d_k = d_v = 1, one token, L = o = q ((1 - beta k^2) alpha S0 + beta k v):
       dq = S1, dv = q beta k, dbeta = q (k v - k^2 alpha S0), dk = q beta (v - 2 k alpha S0),
       dalpha = q (1 - beta k^2) S0, dS0 = q (1 - beta k^2) alpha."""
    q, k, v, a, b, s0 = 1.5, 0.5, 2.0, 0.8, 1.2, -0.4
    f = lambda z: np.array(z, dtype=np.float64).reshape(1, 1, 1, 1)
    g = oracle.bwd(f(q), f(k), f(v), f(a), np.array([[[b]]]), np.ones((1, 1, 1)), S0=np.array([[[s0]]]))
    S1 = (1 - b * k * k) * a * s0 + b * k * v
    want = {"dq": S1, "dv": q * b * k, "dbeta": q * (k * v - k * k * a * s0), "dk": q * b * (v - 2 * k * a * s0),
            "dalpha": q * (1 - b * k * k) * s0, "dS0": q * (1 - b * k * k) * a}
    for key, val in want.items():
        np.testing.assert_allclose(g[key].ravel()[0], val, rtol=0, atol=1e-15)


def test_bwd_head_selection_and_no_final_gradient():
    rng = np.random.default_rng(9)
    B, T, H, dk, dv = 2, 20, 3, 3, 2
    x, dO, _ = _inputs(rng, B, T, H, dk, dv)
    g = oracle.bwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dO, S0=x["S0"])
    sel = [5, 0, 3]
    gs = oracle.bwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dO[sel], S0=x["S0"][sel], heads=sel)
    for key in g:
        np.testing.assert_array_equal(gs[key], g[key][sel])
    # dST = None is the zero upstream gradient
    g0 = oracle.bwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dO, S0=x["S0"], dST=np.zeros((B * H, dk, dv)))
    for key in g:
        np.testing.assert_array_equal(g0[key], g[key])


# ---- Gated DeltaNet-2: erase gate b per key channel (read side), write gate w per value
# channel (write side): S_t = (I - k (b o k)^T) Diag(alpha) S + k (w o v)^T.

def _gdn2_inputs(rng, B, T, H, dk, dv):
    x, dO, dST = _inputs(rng, B, T, H, dk, dv)
    x.pop("beta")
    x["erase"] = rng.uniform(0.0, 1.0, (B, T, H, dk))
    x["write"] = rng.uniform(0.0, 1.0, (B, T, H, dv))
    return x, dO, dST


def _gdn2_loss(x, dO, dST):
    o, S = oracle.fwd_gdn2(x["q"], x["k"], x["v"], x["alpha"], x["erase"], x["write"], S0=x["S0"])
    return float((o * dO).sum() + (S * dST).sum())


def _gdn2_grads(x, dO, dST):
    return oracle.bwd_gdn2(x["q"], x["k"], x["v"], x["alpha"], x["erase"], x["write"], dO, S0=x["S0"], dST=dST)


def _gdn2_entry(g, name, idx, H):
    if name == "S0":
        return g["dS0"][idx]
    key = {"q": "dq", "k": "dk", "v": "dv", "alpha": "dalpha", "erase": "derase", "write": "dwrite"}[name]
    b, t, h = idx[:3]
    return g[key][(b * H + h, t) + tuple(idx[3:])]


@pytest.mark.parametrize("T", [5, 150])
def test_gdn2_bwd_exact_secants(T):
    """L is affine in each single entry of q, v, alpha, the erase gate, the write gate and
    S0: a secant of any step is the gradient (zero gates included)."""
    rng = np.random.default_rng(200 + T)
    B, H, dk, dv = 2, 2, 4, 3
    x, dO, dST = _gdn2_inputs(rng, B, T, H, dk, dv)
    x["alpha"][0, 1, 0, 2] = 0.0
    x["erase"][1, 2, 1, 0] = 0.0
    g = _gdn2_grads(x, dO, dST)
    L0 = _gdn2_loss(x, dO, dST)
    for name in ("q", "v", "alpha", "erase", "write", "S0"):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in x[name].shape)
            y = {kk: vv.copy() for kk, vv in x.items()}
            y[name][idx] += 0.75
            sec = (_gdn2_loss(y, dO, dST) - L0) / 0.75
            ref = _gdn2_entry(g, name, idx, H)
            assert abs(sec - ref) <= 1e-9 * max(1.0, abs(ref)), (name, idx, sec, ref)


def test_gdn2_bwd_key_central_differences():
    rng = np.random.default_rng(17)
    B, T, H, dk, dv = 1, 70, 2, 4, 3
    x, dO, dST = _gdn2_inputs(rng, B, T, H, dk, dv)
    g = _gdn2_grads(x, dO, dST)
    h = 1e-5
    for _ in range(12):
        idx = tuple(int(rng.integers(0, n)) for n in x["k"].shape)
        yp = {kk: vv.copy() for kk, vv in x.items()}
        ym = {kk: vv.copy() for kk, vv in x.items()}
        yp["k"][idx] += h
        ym["k"][idx] -= h
        fd = (_gdn2_loss(yp, dO, dST) - _gdn2_loss(ym, dO, dST)) / (2 * h)
        ref = _gdn2_entry(g, "k", idx, H)
        assert abs(fd - ref) <= 1e-6 * max(1.0, abs(ref)), (idx, fd, ref)


def test_gdn2_bwd_reduces_to_kda():
    """Both gates tied to beta (the KDA case of the GDN-2 page's section 1): every gradient
    equals the KDA backward's, and dbeta = sum_c derase_c + sum_j dwrite_j."""
    rng = np.random.default_rng(23)
    B, T, H, dk, dv = 2, 90, 2, 4, 3
    x, dO, dST = _inputs(rng, B, T, H, dk, dv)
    b = x["beta"]
    ga = oracle.bwd(x["q"], x["k"], x["v"], x["alpha"], b, dO, S0=x["S0"], dST=dST)
    gb = oracle.bwd_gdn2(x["q"], x["k"], x["v"], x["alpha"], np.repeat(b[..., None], dk, -1),
                         np.repeat(b[..., None], dv, -1), dO, S0=x["S0"], dST=dST)
    for key in ("dq", "dk", "dv", "dalpha", "dS0"):
        np.testing.assert_allclose(gb[key], ga[key], rtol=0, atol=1e-12 * max(1.0, np.abs(ga[key]).max()))
    np.testing.assert_allclose(gb["derase"].sum(-1) + gb["dwrite"].sum(-1), ga["dbeta"], rtol=0, atol=1e-12)


def test_gdn2_bwd_scalar_token_by_hand():
    """d_k = d_v = 1, one token: o = q (a s0 + k (w v - b k a s0)):
       dq = S1, dv = q k w, dwrite = q k v, derase = -q k^2 a s0, dk = q (w v - 2 b k a s0),
       dalpha = q s0 (1 - b k^2), dS0 = q a (1 - b k^2)."""
    q, k, v, a, b, w, s0 = 1.5, 0.5, 2.0, 0.8, 0.6, 0.9, -0.4
    f = lambda z: np.array(z, dtype=np.float64).reshape(1, 1, 1, 1)
    g = oracle.bwd_gdn2(f(q), f(k), f(v), f(a), f(b), f(w), np.ones((1, 1, 1)), S0=np.array([[[s0]]]))
    S1 = a * s0 + k * (w * v - b * k * a * s0)
    want = {"dq": S1, "dv": q * k * w, "dwrite": q * k * v, "derase": -q * k * k * a * s0,
            "dk": q * (w * v - 2 * b * k * a * s0), "dalpha": q * s0 * (1 - b * k * k),
            "dS0": q * a * (1 - b * k * k)}
    for key, val in want.items():
        np.testing.assert_allclose(g[key].ravel()[0], val, rtol=0, atol=1e-15)


# ---- SFDA: complex rotation-decay gates on key-channel pairs (SFDA page, "Arquitectura
# Central"): lam holds (Re, Im) of each pair's gate in channels (2p, 2p+1); rows 2p, 2p+1
# of the state, read as z = S_2p + i S_2p+1, become lam_p z before the delta-rule step.

def _sfda_inputs(rng, B, T, H, dk, dv):
    x, dO, dST = _inputs(rng, B, T, H, dk, dv)
    mag = rng.uniform(0.0, 1.0, (B, T, H, dk // 2))
    th = rng.uniform(-np.pi, np.pi, (B, T, H, dk // 2))
    lam = np.empty((B, T, H, dk))
    lam[..., 0::2], lam[..., 1::2] = mag * np.cos(th), mag * np.sin(th)
    lam[0, 1, 0, 0:2] = 0.0                 # an exact zero gate
    lam[0, 2, 0, 2:4] = (0.0, 1.0)          # a quarter turn
    lam[0, 3, 0, 0:2] = (-1.0, 0.0)         # a half turn
    x["alpha"] = lam
    return x, dO, dST


def _sfda_loss(x, dO, dST):
    o, S = oracle.fwd_sfda(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S0=x["S0"])
    return float((o * dO).sum() + (S * dST).sum())


def _sfda_grads(x, dO, dST):
    return oracle.bwd_sfda(x["q"], x["k"], x["v"], x["alpha"], x["beta"], dO, S0=x["S0"], dST=dST)


@pytest.mark.parametrize("T", [5, 150])
def test_sfda_bwd_exact_secants(T):
    """L is affine in each single entry of q, v, beta, S0 and in the real or imaginary part
    of each single gate (Lambda_t enters S_t linearly): secants are the gradient exactly,
    at the zero gate and the quarter and half turns too."""
    rng = np.random.default_rng(300 + T)
    B, H, dk, dv = 2, 2, 4, 3
    x, dO, dST = _sfda_inputs(rng, B, T, H, dk, dv)
    g = _sfda_grads(x, dO, dST)
    L0 = _sfda_loss(x, dO, dST)
    forced = [(0, 1, 0, 0), (0, 1, 0, 1), (0, 2, 0, 3), (0, 3, 0, 0)]
    for name in ("q", "v", "alpha", "beta", "S0"):
        picks = [tuple(int(rng.integers(0, n)) for n in x[name].shape) for _ in range(6)]
        if name == "alpha":
            picks += forced
        for idx in picks:
            y = {kk: vv.copy() for kk, vv in x.items()}
            y[name][idx] += 0.75
            sec = (_sfda_loss(y, dO, dST) - L0) / 0.75
            ref = _entry_grad(g, name, idx, H)
            assert abs(sec - ref) <= 1e-9 * max(1.0, abs(ref)), (name, idx, sec, ref)


def test_sfda_bwd_key_central_differences():
    rng = np.random.default_rng(31)
    B, T, H, dk, dv = 1, 70, 2, 4, 3
    x, dO, dST = _sfda_inputs(rng, B, T, H, dk, dv)
    g = _sfda_grads(x, dO, dST)
    h = 1e-5
    for _ in range(12):
        idx = tuple(int(rng.integers(0, n)) for n in x["k"].shape)
        yp = {kk: vv.copy() for kk, vv in x.items()}
        ym = {kk: vv.copy() for kk, vv in x.items()}
        yp["k"][idx] += h
        ym["k"][idx] -= h
        fd = (_sfda_loss(yp, dO, dST) - _sfda_loss(ym, dO, dST)) / (2 * h)
        ref = _entry_grad(g, "k", idx, H)
        assert abs(fd - ref) <= 1e-6 * max(1.0, abs(ref)), (idx, fd, ref)


def test_sfda_bwd_zero_phase_reduces_to_kda():
    """Every phase zero (the page's "Principales Contribuciones" item 1: KDA recovered, both
    channels of a pair decayed by Re lam): dq, dk, dv, dbeta, dS0 are the KDA backward's with
    alpha_2p = alpha_2p+1 = Re lam_p, and dRe lam_p = dalpha_2p + dalpha_2p+1."""
    rng = np.random.default_rng(37)
    B, T, H, dk, dv = 2, 90, 2, 4, 3
    x, dO, dST = _inputs(rng, B, T, H, dk, dv)
    re = np.tanh(2 * rng.standard_normal((B, T, H, dk // 2)))
    re[0, 4, 1, 1] = 0.0
    lam = np.zeros((B, T, H, dk))
    lam[..., 0::2] = re
    ga = oracle.bwd(x["q"], x["k"], x["v"], np.repeat(re, 2, axis=-1), x["beta"], dO, S0=x["S0"], dST=dST)
    gb = oracle.bwd_sfda(x["q"], x["k"], x["v"], lam, x["beta"], dO, S0=x["S0"], dST=dST)
    for key in ("dq", "dk", "dv", "dbeta", "dS0"):
        np.testing.assert_allclose(gb[key], ga[key], rtol=0, atol=1e-12 * max(1.0, np.abs(ga[key]).max()))
    np.testing.assert_allclose(gb["dalpha"][..., 0::2], ga["dalpha"][..., 0::2] + ga["dalpha"][..., 1::2],
                               rtol=0, atol=1e-12 * max(1.0, np.abs(ga["dalpha"]).max()))


def test_sfda_bwd_pure_rotation_closed_form():
    """beta = 0: each column of each coordinate is a complex number z_t = lam_t z_{t-1},
    o_t = sum_p Re(conj(q_t,p) z_t,p) and <dS_T, S_T> = sum_p Re(conj(dS_T,p) z_T,p).  With
    c_t = dO_t conj(q_t) (plus conj(dS_T) at the last token) and P_tm the product of the
    gates 1..t except m, dL/dRe lam_m - i dL/dIm lam_m = sum_{t >= m} c_t P_tm z_0, dz_0 likewise
    with every gate, and dq_t = z_t dO_t -- numpy complex products, no division (a zero gate
    included)."""
    rng = np.random.default_rng(41)
    B, T, H, dk, dv = 1, 12, 1, 4, 3
    x, dO, dST = _sfda_inputs(rng, B, T, H, dk, dv)
    x["beta"][:] = 0.0
    g = _sfda_grads(x, dO, dST)
    lam = x["alpha"][0, :, 0, 0::2] + 1j * x["alpha"][0, :, 0, 1::2]          # [T, P]
    qc = x["q"][0, :, 0, 0::2] + 1j * x["q"][0, :, 0, 1::2]                   # [T, P]
    z0 = x["S0"][0, 0::2] + 1j * x["S0"][0, 1::2]                             # [P, dv]
    dsc = dST[0, 0::2] + 1j * dST[0, 1::2]                                    # [P, dv]
    c = dO[0][:, None, :] * np.conj(qc)[:, :, None]                           # [T, P, dv]
    c[-1] += np.conj(dsc)
    prod_to = lambda t, skip=None: np.prod([np.ones(dk // 2)] + [lam[s] for s in range(t + 1) if s != skip], axis=0)
    for m in range(T):
        Gm = sum(c[t] * prod_to(t, skip=m)[:, None] * z0 for t in range(m, T)).sum(axis=-1)   # [P]
        np.testing.assert_allclose(g["dalpha"][0, m, 0::2], Gm.real, rtol=0, atol=1e-12)
        np.testing.assert_allclose(g["dalpha"][0, m, 1::2], -Gm.imag, rtol=0, atol=1e-12)
    Gz = sum(c[t] * prod_to(t)[:, None] for t in range(T))                  # [P, dv]
    np.testing.assert_allclose(g["dS0"][0, 0::2], Gz.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dS0"][0, 1::2], -Gz.imag, rtol=0, atol=1e-12)
    for t in range(T):
        zt = prod_to(t)[:, None] * z0                                         # [P, dv]
        dq = (zt * dO[0, t][None, :]).sum(axis=-1)
        np.testing.assert_allclose(g["dq"][0, t, 0::2], dq.real, rtol=0, atol=1e-12)
        np.testing.assert_allclose(g["dq"][0, t, 1::2], dq.imag, rtol=0, atol=1e-12)
