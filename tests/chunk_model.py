"""numpy model of the chunkwise WY algebra the HIP kernel computes (test infrastructure).

This is a specification of the GPU arithmetic, written for checking, not GPU
code: it is compared with the fp64 oracle (the token recurrence) in
``test_chunk_model.py`` and, with ``emulate="bf16"``, gives the error budget of
bf16 matrix-core operands with fp32 accumulation.

Per chunk of C positions (start state S, d_k x d_v), with r_ij = prod_{m=j+1..i} alpha_m:

* T_ij = beta_i sum_c k_ic k_jc r_ijc (j < i),   A_ij = sum_c q_ic k_jc r_ijc (j <= i)
* (I + T) Delta = diag(beta) V - diag(beta) (K o gamma) S      (gamma_i = r_{i,-1})
  so Delta = U - W S with M = (I + T)^-1, U = M diag(beta) V, W = M diag(beta) (K o gamma)
* O = (Q o gamma) S + A Delta,   S_next = diag(gamma_last) S + (K o rho)^T Delta  (rho_j = r_{C-1,j})

This is the chunk-WY product form of the SFDA page ("El Teorema de Chunk-WY
Constructivo", with the block write summary of "Principales Contribuciones"
item 3) and the decay-absorbed triangular solve of the Gated DeltaNet-2 page
(section 3).  Decay ratios are never divided: every r_ij is a product of
alpha's over a range, taken from running products that are local to 16-row
sub-blocks:

* off-diagonal 16x16 tiles (I > J): r_ij = F_i * Pi_IJ * Bk_j with F the
  prefix product from the start of block I, Bk the suffix product to the end
  of block J and Pi_IJ the product of the whole blocks in between;
* inside a diagonal tile the pair (i, j) is split at the highest bit in which
  the local indices differ (level lam = 8, 4, 2, 1): r_ij = F^lam_i * B^lam_j
  with prefix / suffix products inside aligned lam-segments.

Every factor has magnitude <= 1 and is exactly zero across a zero gate.
"""
from __future__ import annotations

import numpy as np

SUB = 16


def _bf16(x):
    x = np.asarray(x, np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


class _Arith:
    def __init__(self, emulate):
        self.emulate = emulate
        self.f = np.float64 if emulate is None else np.float32

    def op(self, x):
        """Round a matrix-core operand."""
        if self.emulate == "bf16":
            return _bf16(x).astype(np.float32)
        return np.asarray(x, self.f)

    def mm(self, a, b):
        return (self.op(a) @ self.op(b)).astype(self.f)

    def mm_exact(self, a, b):
        """Products kept at working precision (the small fp32 triangular inverse)."""
        return (np.asarray(a, self.f) @ np.asarray(b, self.f)).astype(self.f)


def block_factors(a):
    """Sub-block-local product factors for one chunk of gates a [C, dk].

    Returns dict with F16, B16 [C, dk], g [nb, dk], and per level lam:
    Flam (valid on rows whose local bit lam is set) and Blam (valid where clear).
    """
    C, dk = a.shape
    nb = C // SUB
    F = np.ones_like(a)
    Bk = np.ones_like(a)
    g = np.ones((nb, dk), a.dtype)
    lev = {}
    for I in range(nb):
        blk = a[I * SUB:(I + 1) * SUB]
        run = np.ones(dk, a.dtype)
        for m in range(SUB):
            run = run * blk[m]
            F[I * SUB + m] = run
        g[I] = run
        run = np.ones(dk, a.dtype)
        for m in range(SUB - 1, -1, -1):
            Bk[I * SUB + m] = run
            run = run * blk[m]
    for lam in (8, 4, 2, 1):
        Fl = np.zeros_like(a)
        Bl = np.zeros_like(a)
        for p in range(C):
            m = p % SUB
            base = p - m
            if m & lam:
                s = base + (m & ~(lam - 1))
                Fl[p] = np.prod(a[s:p + 1], axis=0)
            else:
                e = base + (m | (lam - 1))
                Bl[p] = np.prod(a[p + 1:e + 1], axis=0) if e > p else np.ones(dk, a.dtype)
        lev[lam] = (Fl, Bl)
    return dict(F16=F, B16=Bk, g=g, lev=lev)


def intra_matrices(q, k, a, beta, ar: _Arith):
    """T (strictly lower, beta-scaled rows) and A (lower incl. diagonal), [C, C]."""
    C = q.shape[0]
    nb = C // SUB
    fx = block_factors(a)
    F, Bk, g = fx["F16"], fx["B16"], fx["g"]
    T = np.zeros((C, C), ar.f)
    A = np.zeros((C, C), ar.f)
    Y = k * Bk
    for I in range(nb):
        ri = slice(I * SUB, (I + 1) * SUB)
        for J in range(I):
            rj = slice(J * SUB, (J + 1) * SUB)
            Pi = np.prod(g[J + 1:I], axis=0) if I > J + 1 else np.ones(q.shape[1], q.dtype)
            YJ = Y[rj] * Pi
            A[ri, rj] = ar.mm(q[ri] * F[ri], YJ.T)
            T[ri, rj] = ar.mm(k[ri] * F[ri], YJ.T)
        # diagonal tile: one pass per level, selected by the pair's highest differing bit
        Dq = {}
        Dk = {}
        for lam, (Fl, Bl) in fx["lev"].items():
            Yl = (k[ri] * Bl[ri]).T
            Dq[lam] = ar.mm(q[ri] * Fl[ri], Yl)
            Dk[lam] = ar.mm(k[ri] * Fl[ri], Yl)
        D0 = ar.mm(q[ri], k[ri].T)
        for i in range(SUB):
            A[I * SUB + i, I * SUB + i] = D0[i, i]
            for j in range(i):
                lam = 1 << ((i ^ j).bit_length() - 1)
                A[I * SUB + i, I * SUB + j] = Dq[lam][i, j]
                T[I * SUB + i, I * SUB + j] = Dk[lam][i, j]
    T = (T * np.asarray(beta, ar.f)[:, None]).astype(ar.f)
    return T, A, fx


def unit_lower_inverse(T, ar: _Arith):
    """(I + T)^-1 for strictly lower T: forward substitution on 16x16 diagonal
    blocks, then M_IJ = -N_II sum_{K=J..I-1} T_IK M_KJ block by block."""
    C = T.shape[0]
    nb = C // SUB
    M = np.zeros((C, C), ar.f)
    for I in range(nb):
        r = slice(I * SUB, (I + 1) * SUB)
        Tb = T[r, r]
        N = np.zeros((SUB, SUB), ar.f)
        for i in range(SUB):
            row = np.zeros(SUB, ar.f)
            row[i] = 1
            row = row - Tb[i, :i] @ N[:i]
            N[i] = row
        M[r, r] = N
    for I in range(1, nb):
        ri = slice(I * SUB, (I + 1) * SUB)
        for J in range(I):
            Z = np.zeros((SUB, SUB), ar.f)
            for K in range(J, I):
                rk = slice(K * SUB, (K + 1) * SUB)
                Z = Z + ar.mm_exact(T[ri, rk], M[rk, J * SUB:(J + 1) * SUB])
            M[ri, J * SUB:(J + 1) * SUB] = -ar.mm_exact(M[ri, ri], Z)
    return M


def chunk_forward(q, k, v, a, beta, S0=None, C=64, emulate=None, debug=None):
    """Whole-sequence forward for one head via the chunk algebra.

    q, k, a: [T, dk]; v: [T, dv]; beta: [T]; S0: [dk, dv] or None.
    emulate: None (fp64 throughout) or "bf16" (bf16 matrix-core operands,
    fp32 accumulation and fp32 state, bf16 output).
    debug: optional list; per chunk a dict of intermediates is appended.
    Returns (o [T, dv], S_T [dk, dv]).
    """
    ar = _Arith(emulate)
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv), ar.f) if S0 is None else np.asarray(S0, ar.f).copy()
    o = np.zeros((T, dv), ar.f)
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        # ragged tail: identity transitions (alpha 1, beta 0, k 0) that write nothing
        qc = np.zeros((C, dk), ar.f); qc[:n] = q[c0:c0 + n]
        kc = np.zeros((C, dk), ar.f); kc[:n] = k[c0:c0 + n]
        ac = np.ones((C, dk), ar.f); ac[:n] = a[c0:c0 + n]
        vc = np.zeros((C, dv), ar.f); vc[:n] = v[c0:c0 + n]
        bc = np.zeros(C, ar.f); bc[:n] = beta[c0:c0 + n]
        Tm, Am, fx = intra_matrices(qc, kc, ac, bc, ar)
        nb = C // SUB
        g = fx["g"]
        G = np.ones((nb, dk), ar.f)
        R = np.ones((nb, dk), ar.f)
        for I in range(1, nb):
            G[I] = G[I - 1] * g[I - 1]
        for I in range(nb - 2, -1, -1):
            R[I] = R[I + 1] * g[I + 1]
        gam = fx["F16"] * np.repeat(G, SUB, axis=0)
        rho = fx["B16"] * np.repeat(R, SUB, axis=0)
        gC = G[-1] * g[-1]
        M = unit_lower_inverse(Tm, ar)
        Mt = (M * bc[None, :]).astype(ar.f)
        W = ar.mm(Mt, kc * gam)
        U = ar.mm(Mt, vc)
        Dl = (U - ar.mm(W, S)).astype(ar.f)
        O = (ar.mm(qc * gam, S) + ar.mm(Am, Dl)).astype(ar.f)
        S = (gC[:, None] * S + ar.mm((kc * rho).T, Dl)).astype(ar.f)
        o[c0:c0 + n] = O[:n]
        if debug is not None:
            debug.append(dict(T=Tm, A=Am, M=M, W=W, U=U, Delta=Dl, O=O, S=S.copy(),
                              gamma=gam, rho=rho))
    if emulate == "bf16":
        o = _bf16(o)
    return o, S
