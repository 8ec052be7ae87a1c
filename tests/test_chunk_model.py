"""The chunk-WY algebra (as the kernel computes it) against the fp64 oracle (CPU only).

The SFDA page reports its chunk-WY recursion and affine block transfer agreeing
with brute force to residuals between 1e-10 and 1e-15 ("Resultados",
numerical verification); the fp64 model here is held to 1e-10.
"""
import numpy as np
import pytest

import chunk_model as cm
import oracle
from test_oracle import _rand_case


def _run(T, dk, dv, seed, ckda=True, zero_frac=0.15):
    rng = np.random.default_rng(seed)
    q, k, v, a, b = _rand_case(rng, 1, T, 1, dk, dv, ckda=ckda)
    S0 = rng.standard_normal((dk, dv))
    o, S = oracle.fwd(q, k, v, a, b, S0=S0[None])
    dbg = []
    om, Sm = cm.chunk_forward(q[0, :, 0], k[0, :, 0], v[0, :, 0], a[0, :, 0], b[0, :, 0], S0, debug=dbg)
    return o[0], S[0], om, Sm, dbg, b[0, :, 0]


@pytest.mark.parametrize("T,dk,dv,seed", [(64, 8, 8, 1), (150, 8, 6, 2), (257, 16, 4, 3),
                                          (1, 4, 4, 4), (63, 5, 7, 5), (200, 32, 32, 6)])
def test_chunk_model_matches_oracle(T, dk, dv, seed):
    o, S, om, Sm, _, _ = _run(T, dk, dv, seed)
    scale = max(1.0, np.abs(o).max())
    assert np.abs(om - o).max() <= 1e-10 * scale
    assert np.abs(Sm - S).max() <= 1e-10 * max(1.0, np.abs(S).max())


def test_chunk_model_kda_gates():
    o, S, om, Sm, _, _ = _run(300, 16, 16, 7, ckda=False)
    assert np.abs(om - o).max() <= 1e-10 * max(1.0, np.abs(o).max())


def test_all_zero_and_sign_gates():
    """Gates only in {-1, 0, 1}: every decay factor is exactly a signed 0/1 pattern."""
    rng = np.random.default_rng(8)
    T, dk, dv = 192, 8, 8
    q, k, v, _, b = _rand_case(rng, 1, T, 1, dk, dv)
    a = rng.choice([-1.0, 0.0, 1.0], size=(1, T, 1, dk))
    S0 = rng.standard_normal((dk, dv))
    o, S = oracle.fwd(q, k, v, a, b, S0=S0[None])
    om, Sm = cm.chunk_forward(q[0, :, 0], k[0, :, 0], v[0, :, 0], a[0, :, 0], b[0, :, 0], S0)
    assert np.abs(om - o[0]).max() <= 1e-10 * max(1.0, np.abs(o).max())
    assert np.abs(Sm - S[0]).max() <= 1e-10


def test_inverse_entries_bounded_by_beta():
    """|((I+T)^-1)_ij| <= max beta for i != j: the entry is -beta_i k_i^T D_i A_{i-1}..A_{j+1} k_j,
    a product of non-expansive factors (unit k, |alpha| <= 1, beta in [0, 2])."""
    _, _, _, _, dbg, b = _run(256, 16, 8, 9)
    for d in dbg:
        M = d["M"].copy()
        np.fill_diagonal(M, 0.0)
        assert np.abs(M).max() <= b.max() + 1e-12
        np.testing.assert_allclose(M + np.eye(M.shape[0]), np.linalg.inv(np.eye(M.shape[0]) + d["T"]),
                                   atol=1e-12)


def test_bf16_emulation_within_tolerance():
    """bf16 operands with fp32 accumulation stay well inside the 2e-2 parity gate."""
    from gated_delta_rule_78_amd.inputs import make, bf16_to_f32
    inp = make(1, 640, 1, 128, 128, "bf16", "ckda", False, seed=21)
    o, S = oracle.fwd(inp.q, inp.k, inp.v, inp.alpha, inp.beta, S0=inp.S0.reshape(1, 128, 128))
    f = lambda x: bf16_to_f32(x[0, :, 0])
    om, Sm = cm.chunk_forward(f(inp.q), f(inp.k), f(inp.v), f(inp.alpha), bf16_to_f32(inp.beta[0, :, 0]),
                              inp.S0[0, 0], emulate="bf16")
    assert np.abs(om - o[0]).max() / np.abs(o[0]).max() < 1e-2
    assert np.abs(Sm - S[0]).max() / np.abs(S[0]).max() < 1e-2


@pytest.mark.parametrize("T,dk,dv,zero_frac,check", [(150, 6, 5, 0.1, True), (64, 4, 3, 0.3, True),
                                                     (200, 8, 4, 0.0, False)])
def test_chunk_backward_matches_oracle(T, dk, dv, zero_frac, check):
    """The chunkwise backward (adjoint state pass, dv contractions, WY and inverse
    adjoints, decayed-product gradients, reverse-summed gate gradient with the
    exclusive-product form at zero gates) equals the oracle's reverse-mode gradients."""
    import oracle
    rng = np.random.default_rng(T + dk)
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    a = np.tanh(2 * rng.standard_normal((T, dk)))
    m = rng.random(a.shape) < zero_frac
    a[m] = rng.choice([-1.0, 0.0, 1.0], size=int(m.sum()))
    b = rng.uniform(0.0, 2.0, T)
    S0 = rng.standard_normal((dk, dv))
    dO = rng.standard_normal((T, dv))
    dST = rng.standard_normal((dk, dv))
    g = cm.chunk_backward(q, k, v, a, b, dO, S0, dST, C=64, check_zero_formula=check)
    r = oracle.bwd(q[None, :, None], k[None, :, None], v[None, :, None], a[None, :, None], b[None, :, None],
                   dO[None], S0=S0[None], dST=dST[None])
    for key in ("dq", "dk", "dv", "dalpha", "dbeta", "dS0"):
        y = r[key][0]
        assert np.abs(g[key] - y).max() <= 1e-10 * max(1.0, np.abs(y).max()), key


@pytest.mark.parametrize("T,dk,dv,zero_frac", [(150, 6, 5, 0.1), (64, 4, 3, 0.3), (200, 8, 4, 0.0), (37, 3, 2, 0.5)])
def test_blocked_gate_gradient_matches_oracle(T, dk, dv, zero_frac):
    """The GPU gradient kernel's decomposition (block-anchored products, rows below a
    block folded into its last row, in-block recursion over the gates) gives the
    oracle's gradients, exact zero gates included."""
    import oracle
    rng = np.random.default_rng(3 * T + dk)
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    a = np.tanh(2 * rng.standard_normal((T, dk)))
    m = rng.random(a.shape) < zero_frac
    a[m] = rng.choice([-1.0, 0.0, 1.0], size=int(m.sum()))
    a[5, 0] = a[17, 0] = 0.0   # zeros in both of two adjacent blocks of one channel
    b = rng.uniform(0.0, 2.0, T)
    S0 = rng.standard_normal((dk, dv))
    dO = rng.standard_normal((T, dv))
    dST = rng.standard_normal((dk, dv))
    g = cm.chunk_backward(q, k, v, a, b, dO, S0, dST, C=64, blocked=True)
    r = oracle.bwd(q[None, :, None], k[None, :, None], v[None, :, None], a[None, :, None], b[None, :, None],
                   dO[None], S0=S0[None], dST=dST[None])
    for key in ("dq", "dk", "dv", "dalpha", "dbeta", "dS0"):
        y = r[key][0]
        assert np.abs(g[key] - y).max() <= 1e-10 * max(1.0, np.abs(y).max()), key


@pytest.mark.parametrize("T,dk,dv,blocked", [(150, 6, 5, False), (150, 6, 5, True), (70, 4, 3, True)])
def test_gdn2_chunk_backward_matches_oracle(T, dk, dv, blocked):
    """The Gated DeltaNet-2 chunk backward (erase vector on T's row side and in W, write
    gate on V), directly and in the GPU kernel's blocked decomposition (zero gates
    included), equals the oracle's GDN-2 backward."""
    import oracle
    rng = np.random.default_rng(5 * T + dk)
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    a = np.tanh(2 * rng.standard_normal((T, dk)))
    if blocked:
        m = rng.random(a.shape) < 0.1
        a[m] = rng.choice([-1.0, 0.0, 1.0], size=int(m.sum()))
    else:
        a = 0.5 + 0.5 * np.abs(a)          # the direct form divides by the gates
    b = rng.uniform(0.0, 1.0, (T, dk))
    w = rng.uniform(0.0, 1.0, (T, dv))
    S0 = rng.standard_normal((dk, dv))
    dO = rng.standard_normal((T, dv))
    dST = rng.standard_normal((dk, dv))
    g = cm.chunk_backward_gdn2(q, k, v, a, b, w, dO, S0, dST, C=64, blocked=blocked)
    r = oracle.bwd_gdn2(q[None, :, None], k[None, :, None], v[None, :, None], a[None, :, None], b[None, :, None],
                        w[None, :, None], dO[None], S0=S0[None], dST=dST[None])
    for key in ("dq", "dk", "dv", "dalpha", "derase", "dwrite", "dS0"):
        y = r[key][0]
        assert np.abs(g[key] - y).max() <= 1e-10 * max(1.0, np.abs(y).max()), key


@pytest.mark.parametrize("T,dk,dv,blocked", [(100, 8, 4, False), (130, 8, 4, True), (64, 4, 3, True)])
def test_sfda_chunk_backward_matches_oracle(T, dk, dv, blocked):
    """The SFDA chunk backward in complex pair arithmetic, directly and in the GPU kernel's
    blocked decomposition (conj(r) on the key side, conjugated pair weights), equals the
    oracle's SFDA backward; gates include an exact zero and quarter and half turns."""
    import oracle
    rng = np.random.default_rng(11 * T + dk)
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    mag, th = rng.uniform(0.0, 1.0, (T, dk // 2)), rng.uniform(-np.pi, np.pi, (T, dk // 2))
    lam = np.empty((T, dk))
    lam[:, 0::2], lam[:, 1::2] = mag * np.cos(th), mag * np.sin(th)
    lam[3, 0:2], lam[20, 2:4], lam[40, 0:2] = (0.0, 0.0), (0.0, 1.0), (-1.0, 0.0)
    b = rng.uniform(0.0, 2.0, T)
    S0 = rng.standard_normal((dk, dv))
    dO = rng.standard_normal((T, dv))
    dST = rng.standard_normal((dk, dv))
    g = cm.chunk_backward_sfda(q, k, v, lam, b, dO, S0, dST, C=64, blocked=blocked)
    r = oracle.bwd_sfda(q[None, :, None], k[None, :, None], v[None, :, None], lam[None, :, None], b[None, :, None],
                        dO[None], S0=S0[None], dST=dST[None])
    for key in ("dq", "dk", "dv", "dalpha", "dbeta", "dS0"):
        y = r[key][0]
        assert np.abs(g[key] - y).max() <= 1e-10 * max(1.0, np.abs(y).max()), key
