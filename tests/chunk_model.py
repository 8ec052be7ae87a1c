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


# ---------------------------------------------------------------------------
# Backward of the chunk algebra (fp64 specification, test infrastructure).
#
# Gradients of L = sum <dO, O> + <dS_T, S_T>.  Per chunk, in reverse order, with the
# chunk's start state S and the gradient dS' of its end state:
#   dDelta = K^ dS' + A^T dO                 (K^ = K o rho, A lower incl. diagonal)
#   dS     = diag(gamma_L) dS' + Q~^T dO - W^T dDelta        (carried to the previous chunk)
#   dQ~ = dO S^T,  dA = (dO Delta^T) o lower,  dK^ = Delta dS'^T,  dgamma_L = rowsum(dS' o S)
#   dW = -dDelta S^T,  dV = M~^T dDelta,  dM~ = (dDelta V^T + dW K~^T) o lower,  dK~ = M~^T dW
#   dbeta_j = sum_i dM~_ij M_ij,  dM = dM~ diag(beta),  dT = -(M^T dM M^T) o strict lower
#   dbeta_i += sum_j dT_ij D_ij,  dD = diag(beta) dT          (T = diag(beta) D)
# and through the decayed products A_ij = sum_c q_ic k_jc r_ijc, D_ij = sum_c k_ic k_jc r_ijc:
#   Zq_i = sum_{j<=i} dA_ij k_j o r_ij,   Zr_i = sum_{j<i} dD_ij k_j o r_ij,
#   Zc_j = sum_{i>=j} dA_ij q_i o r_ij + sum_{i>j} dD_ij k_i o r_ij,
#   dq = dQ~ o gamma + Zq,   dk = dK~ o gamma + dK^ o rho + Zr + Zc.
# Gate gradient, per channel: with
#   dG_i = dQ~_i Q~_i + dK~_i K~_i + q_i Zq_i + k_i Zr_i - k_i Zc_i - dK^_i K^_i
#          (+ sum_j dK^_j K^_j + dgamma_L gamma_L at i = C-1),
# the reverse sum P_m = sum_{i>=m} dG_i equals alpha_m dalpha_m (the terms with both ends
# at or after m cancel), so dalpha_m = P_m / alpha_m for a nonzero gate.  For a zero gate
# P_m = 0 and the derivative is the product with alpha_m left out:
#   dalpha_m = sum_{i>=m} r_(i,m) [sum_{j<m} w_ij r_(m-1,j) + a_i gamma_(m-1)]
#              + r_(L,m) [sum_{j<m} b_j r_(m-1,j) + dgamma_L gamma_(m-1)]
# with w_ij = dA_ij q_i k_j + dD_ij k_i k_j, a_i = dQ~_i q_i + dK~_i k_i, b_j = dK^_j k_j and
# r_(x,y) = prod_{y<l<=x} alpha_l (the products exclusive of m on both sides).
# ---------------------------------------------------------------------------

def _ranges(a):
    """r[i, j] = prod_{j<l<=i} a_l for i >= j (1 on the diagonal, 0 above), [C, C, dk]."""
    C, dk = a.shape
    r = np.zeros((C, C, dk))
    for j in range(C):
        run = np.ones(dk)
        r[j, j] = 1.0
        for i in range(j + 1, C):
            run = run * a[i]
            r[i, j] = run
    return r


def _chunk_fwd_parts(q, k, v, a, beta, S):
    C = q.shape[0]
    r = _ranges(a)
    gam = np.cumprod(a, axis=0)                       # gamma_i = prod_{l<=i}
    rho = r[C - 1]                                     # rho_j = prod_{j<l<=C-1}
    gL = gam[C - 1]
    A = np.einsum("ic,jc,ijc->ij", q, k, r) * np.tril(np.ones((C, C)))
    D = np.einsum("ic,jc,ijc->ij", k, k, r) * np.tril(np.ones((C, C)), -1)
    M = np.linalg.inv(np.eye(C) + beta[:, None] * D)
    Mt = M * beta[None, :]
    Kg, Qg, Kr = k * gam, q * gam, k * rho
    U, W = Mt @ v, Mt @ Kg
    Dl = U - W @ S
    O = Qg @ S + A @ Dl
    Sn = gL[:, None] * S + Kr.T @ Dl
    return dict(r=r, gam=gam, rho=rho, gL=gL, A=A, D=D, M=M, Mt=Mt, Kg=Kg, Qg=Qg, Kr=Kr, W=W, Dl=Dl,
                O=O, S=S, Sn=Sn)


def chunk_backward(q, k, v, a, beta, dO, S0=None, dST=None, C=64, check_zero_formula=False, blocked=False):
    """Gradients for one head through the chunk algebra (fp64).  q, k, a [T, dk]; v, dO
    [T, dv]; beta [T]; S0, dST [dk, dv] or None.  Returns dict dq, dk, dv, dalpha, dbeta,
    dS0.  check_zero_formula: also evaluate the exclusive-product formula for every gate
    (zero or not) and assert it equals P_m / alpha_m where alpha_m != 0.  blocked: take the
    decayed sums and the gate gradient from blocked_decay_grads (the GPU kernel's
    decomposition) instead."""
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, np.float64).copy()
    parts = []
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        pad = lambda x, fill, w: np.concatenate([x[c0:c0 + n], np.full((C - n,) + x.shape[1:], fill)])[:C]
        qc, kc, vc = pad(q, 0.0, dk), pad(k, 0.0, dk), pad(v, 0.0, dv)
        ac, bc, dOc = pad(a, 1.0, dk), pad(beta, 0.0, 1), pad(dO, 0.0, dv)
        p = _chunk_fwd_parts(qc, kc, vc, ac, bc, S)
        p.update(q=qc, k=kc, v=vc, a=ac, beta=bc, dO=dOc, c0=c0, n=n)
        parts.append(p)
        S = p["Sn"]
    out = {x: np.zeros((T, dk)) for x in ("dq", "dk", "dalpha")}
    out["dv"] = np.zeros((T, dv))
    out["dbeta"] = np.zeros(T)
    dSn = np.zeros((dk, dv)) if dST is None else np.asarray(dST, np.float64).copy()
    low, slow = np.tril(np.ones((C, C))), np.tril(np.ones((C, C)), -1)
    for p in reversed(parts):
        S, dO_, qc, kc, vc, ac, bc = p["S"], p["dO"], p["q"], p["k"], p["v"], p["a"], p["beta"]
        r, gam, rho, gL = p["r"], p["gam"], p["rho"], p["gL"]
        dDl = p["Kr"] @ dSn + p["A"].T @ dO_
        dS = gL[:, None] * dSn + p["Qg"].T @ dO_ - p["W"].T @ dDl
        dQg = dO_ @ S.T
        dA = (dO_ @ p["Dl"].T) * low
        dKr = p["Dl"] @ dSn.T
        dgL = (dSn * S).sum(axis=1)
        dW = -dDl @ S.T
        dV = p["Mt"].T @ dDl
        dMt = (dDl @ vc.T + dW @ p["Kg"].T) * low
        dKg = p["Mt"].T @ dW
        dbeta = (dMt * p["M"]).sum(axis=0)
        dM = dMt * bc[None, :]
        dT = -(p["M"].T @ dM @ p["M"].T) * slow
        dbeta = dbeta + (dT * p["D"]).sum(axis=1)
        dD = bc[:, None] * dT
        Zq = np.einsum("ij,jc,ijc->ic", dA, kc, r)
        Zr = np.einsum("ij,jc,ijc->ic", dD, kc, r)
        Zc = np.einsum("ij,ic,ijc->jc", dA, qc, r) + np.einsum("ij,ic,ijc->jc", dD, kc, r)
        if blocked:
            Zq, Zr, Zc, dal_b = blocked_decay_grads(dA, dD, qc, kc, ac, dQg * qc + dKg * kc, dKr * kc, dgL)
        dq = dQg * gam + Zq
        dk_ = dKg * gam + dKr * rho + Zr + Zc
        dG = dQg * p["Qg"] + dKg * p["Kg"] + qc * Zq + kc * Zr - kc * Zc - dKr * p["Kr"]
        dG[C - 1] += (dKr * p["Kr"]).sum(axis=0) + dgL * gL
        P = np.cumsum(dG[::-1], axis=0)[::-1]            # P_m = sum_{i >= m} dG_i
        nz = ac != 0.0
        dal = np.where(nz, P / np.where(nz, ac, 1.0), 0.0)
        if check_zero_formula or (~nz).any():
            w = np.einsum("ij,ic,jc->ijc", dA, qc, kc) + np.einsum("ij,ic,jc->ijc", dD, kc, kc)
            av = dQg * qc + dKg * kc
            bv = dKr * kc
            for m in range(C):
                for c in range(dk):
                    if nz[m, c] and not check_zero_formula:
                        continue
                    gm1 = np.prod(ac[:m, c])                      # gamma_(m-1)
                    left = np.array([np.prod(ac[j + 1:m, c]) for j in range(m)])   # r_(m-1, j)
                    tot = 0.0
                    for i in range(m, C):
                        right = np.prod(ac[m + 1:i + 1, c])                      # r_(i, m)
                        tot += right * ((w[i, :m, c] * left).sum() + av[i, c] * gm1)
                    tot += np.prod(ac[m + 1:, c]) * ((bv[:m, c] * left).sum() + dgL[c] * gm1)
                    if nz[m, c]:
                        assert abs(tot - dal[m, c]) <= 1e-9 * max(1.0, abs(tot)), (m, c, tot, dal[m, c])
                    else:
                        dal[m, c] = tot
        if blocked:
            dal = dal_b
        n, c0 = p["n"], p["c0"]
        out["dq"][c0:c0 + n] = dq[:n]
        out["dk"][c0:c0 + n] = dk_[:n]
        out["dv"][c0:c0 + n] = dV[:n]
        out["dalpha"][c0:c0 + n] = dal[:n]
        out["dbeta"][c0:c0 + n] = dbeta[:n]
        dSn = dS
    out["dS0"] = dSn
    return out


def blocked_decay_grads(dA, dD, q, k, a, av, bv, dgl, x=None):
    """The decayed sums and the gate gradient of one chunk as the GPU gradient kernel forms
    them (fp64), from dA (lower, diagonal included), dD (strictly lower) the gradient of the
    second decayed product sum_c x_ic k_jc r_ijc (x = k, or the GDN-2 erase vector b o k),
    the per-row start-state weights av, the final-state weights bv = d(K o rho) o k and
    dgl = d gamma_last.  Returns Zq, Zr, Zc (the sums sum_j dA_ij k_j r_ij,
    sum_j dD_ij k_j r_ij, sum_i (dA_ij q_i + dD_ij x_i) r_ij) and dalpha, with no division
    by a gate:

    * block products anchored at the 16-row block edges: PA^M = dA[>= s, < s] Khat^M,
      PD^M likewise (Khat^M_j = k_j r(s-1, j)), F^M_j = sum_{i > e} (dA_ij q_i + dD_ij k_i)
      r(i, e), with every r a product of in-block prefix / suffix products and whole
      block totals;
    * per (channel, block): the in-block parts of the sums, and for the gate gradient
      the recursion u_i <- alpha_m u_i + E_im over m, started from the weights of the
      pairs that reach left of the block (g_i), the rows below the block folded into
      its last row (X, f).
    """
    C, dk = q.shape
    NB = C // SUB
    x = k if x is None else x
    pin, sig, pib = np.zeros((C, dk)), np.zeros((C, dk)), np.zeros((NB, dk))
    for I in range(NB):
        p = np.ones(dk)
        for r in range(SUB):
            p = p * a[I * SUB + r]
            pin[I * SUB + r] = p
        pib[I] = p
        sf = np.ones(dk)
        for r in range(SUB - 1, -1, -1):
            sig[I * SUB + r] = sf
            sf = sf * a[I * SUB + r]

    def between(J, I):
        p = np.ones(dk)
        for x in range(J + 1, I):
            p = p * pib[x]
        return p

    PA, PD, F = np.zeros((NB, C, dk)), np.zeros((NB, C, dk)), np.zeros((C, dk))
    for M in range(1, NB):
        s = M * SUB
        khat = np.stack([k[j] * sig[j] * between(j // SUB, M) for j in range(s)])
        PA[M, s:] = dA[s:, :s] @ khat
        PD[M, s:] = dD[s:, :s] @ khat
    for M in range(NB - 1):
        s, e1 = M * SUB, M * SUB + SUB
        rie = np.stack([pin[i] * between(M, i // SUB) for i in range(e1, C)])
        F[s:e1] = dA[e1:, s:e1].T @ (q[e1:] * rie) + dD[e1:, s:e1].T @ (x[e1:] * rie)

    Zq, Zr, Zc, dal = np.zeros((C, dk)), np.zeros((C, dk)), np.zeros((C, dk)), np.zeros((C, dk))
    for M in range(NB):
        s = M * SUB
        al, qv, kv, xv = a[s:s + SUB], q[s:s + SUB], k[s:s + SUB], x[s:s + SUB]
        gs = np.prod(pib[:M], axis=0) if M > 0 else np.ones(dk)
        rend = np.prod(pib[M + 1:], axis=0) if M < NB - 1 else np.ones(dk)
        for r in range(SUB):
            i = s + r
            zq, zr, P = dA[i, i] * kv[r], np.zeros(dk), np.ones(dk)
            for rj in range(r - 1, -1, -1):
                P = P * al[rj + 1]
                zq = zq + dA[i, s + rj] * kv[rj] * P
                zr = zr + dD[i, s + rj] * kv[rj] * P
            if M > 0:
                zq = zq + pin[i] * PA[M, i]
                zr = zr + pin[i] * PD[M, i]
            zc, P = dA[i, i] * qv[r], np.ones(dk)
            for ri in range(r + 1, SUB):
                P = P * al[ri]
                zc = zc + (dA[s + ri, i] * qv[ri] + dD[s + ri, i] * xv[ri]) * P
            if M < NB - 1:
                zc = zc + sig[i] * F[i]
            Zq[i], Zr[i], Zc[i] = zq, zr, zc
        bvs = sum((bv[j] * sig[j] * between(j // SUB, M) for j in range(s)), np.zeros(dk))

        def g_at(i):
            g = av[i] * gs
            if M > 0:
                g = g + q[i] * PA[M, i] + x[i] * PD[M, i]
            if i == C - 1:
                g = g + bvs + dgl * gs
            return g

        u = [g_at(s + r) for r in range(SUB)]
        if M < NB - 1:
            xf = np.zeros(dk)
            for i in range(C - 1, s + SUB - 1, -1):   # sum_{i > e} r(i, e) g_i
                xf = a[i] * (g_at(i) + xf)
            u[SUB - 1] = u[SUB - 1] + xf
            f = [kv[r] * F[s + r] + bv[s + r] * rend for r in range(SUB)]
        else:
            f = [bv[s + r] for r in range(SUB)]
        for m in range(SUB):
            acc = u[SUB - 1]
            for i in range(SUB - 2, m - 1, -1):
                acc = u[i] + al[i + 1] * acc
            dal[s + m] = acc
            for i in range(m + 1, SUB):
                E = (qv[i] * dA[s + i, s + m] + xv[i] * dD[s + i, s + m]) * kv[m]
                if i == SUB - 1:
                    E = E + f[m]
                u[i] = al[m] * u[i] + E
    return Zq, Zr, Zc, dal


def chunk_backward_gdn2(q, k, v, a, erase, write, dO, S0=None, dST=None, C=64, blocked=False):
    """Gated DeltaNet-2 gradients for one head through the chunk algebra (fp64), as the GPU
    kernels form them.  erase [T, dk] (b), write [T, dv] (w).  Per chunk, with e = b o k:
    T = [sum_c e_ic k_jc r_ijc] (j < i), M = (I + T)^-1, W = M (E o gamma), U = M (w o V);
    then Delta, O, S' as for KDA (which is e = beta k, w = beta).  Returns dq, dk, dv,
    dalpha, derase, dwrite, dS0.  blocked: decayed sums and gate gradient from
    blocked_decay_grads with the erase vector as the second product's row operand."""
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, np.float64).copy()
    low, slow = np.tril(np.ones((C, C))), np.tril(np.ones((C, C)), -1)
    parts = []
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        pad = lambda x, fill: np.concatenate([x[c0:c0 + n], np.full((C - n,) + x.shape[1:], fill)])[:C]
        qc, kc, vc, ac = pad(q, 0.0), pad(k, 0.0), pad(v, 0.0), pad(a, 1.0)
        bc, wc, dOc = pad(erase, 0.0), pad(write, 0.0), pad(dO, 0.0)
        r = _ranges(ac)
        gam = np.cumprod(ac, axis=0)
        rho, gL = r[C - 1], gam[C - 1]
        ec = bc * kc
        A = np.einsum("ic,jc,ijc->ij", qc, kc, r) * low
        Tm = np.einsum("ic,jc,ijc->ij", ec, kc, r) * slow
        M = np.linalg.inv(np.eye(C) + Tm)
        Eg, Qg, Kr, WV = ec * gam, qc * gam, kc * rho, wc * vc
        W = M @ Eg
        Dl = M @ WV - W @ S
        parts.append(dict(S=S, q=qc, k=kc, v=vc, a=ac, b=bc, w=wc, e=ec, dO=dOc, r=r, gam=gam, rho=rho, gL=gL,
                          A=A, T=Tm, M=M, Eg=Eg, Qg=Qg, Kr=Kr, WV=WV, W=W, Dl=Dl, c0=c0, n=n))
        S = gL[:, None] * S + Kr.T @ Dl
    out = {x: np.zeros((T, dk)) for x in ("dq", "dk", "dalpha", "derase")}
    out["dv"], out["dwrite"] = np.zeros((T, dv)), np.zeros((T, dv))
    dSn = np.zeros((dk, dv)) if dST is None else np.asarray(dST, np.float64).copy()
    for p in reversed(parts):
        S, dO_, qc, kc, vc, ac, ec = p["S"], p["dO"], p["q"], p["k"], p["v"], p["a"], p["e"]
        r, gam, rho, gL, M = p["r"], p["gam"], p["rho"], p["gL"], p["M"]
        dDl = p["Kr"] @ dSn + p["A"].T @ dO_
        dS = gL[:, None] * dSn + p["Qg"].T @ dO_ - p["W"].T @ dDl
        dQg = dO_ @ S.T
        dA = (dO_ @ p["Dl"].T) * low
        dKr = p["Dl"] @ dSn.T
        dgL = (dSn * S).sum(axis=1)
        dW = -dDl @ S.T
        dWV = M.T @ dDl                       # d(w o V)
        dM = (dDl @ p["WV"].T + dW @ p["Eg"].T) * low
        dEg = M.T @ dW                        # d(E o gamma)
        dT = -(M.T @ dM @ M.T) * slow
        av = dQg * qc + dEg * ec
        bv = dKr * kc
        if blocked:
            Zq, Ze, Zc, dal = blocked_decay_grads(dA, dT, qc, kc, ac, av, bv, dgL, x=ec)
        else:
            Zq = np.einsum("ij,jc,ijc->ic", dA, kc, r)
            Ze = np.einsum("ij,jc,ijc->ic", dT, kc, r)
            Zc = np.einsum("ij,ic,ijc->jc", dA, qc, r) + np.einsum("ij,ic,ijc->jc", dT, ec, r)
            dG = dQg * p["Qg"] + dEg * p["Eg"] + qc * Zq + ec * Ze - kc * Zc - dKr * p["Kr"]
            dG[C - 1] += (dKr * p["Kr"]).sum(axis=0) + dgL * gL
            P = np.cumsum(dG[::-1], axis=0)[::-1]
            nz = ac != 0.0
            dal = np.where(nz, P / np.where(nz, ac, 1.0), 0.0)
        de = dEg * gam + Ze                   # d e, e = b o k
        n, c0 = p["n"], p["c0"]
        out["dq"][c0:c0 + n] = (dQg * gam + Zq)[:n]
        out["dk"][c0:c0 + n] = (dKr * rho + Zc + p["b"] * de)[:n]
        out["derase"][c0:c0 + n] = (kc * de)[:n]
        out["dv"][c0:c0 + n] = (p["w"] * dWV)[:n]
        out["dwrite"][c0:c0 + n] = (vc * dWV)[:n]
        out["dalpha"][c0:c0 + n] = dal[:n]
        dSn = dS
    out["dS0"] = dSn
    return out


# ---- SFDA (complex rotation-decay gates on key-channel pairs) --------------------------
# A real d_k-vector x is read as P = d_k / 2 complex numbers x_p = x_2p + i x_2p+1, the
# state's rows 2p, 2p+1 as one complex row, and the gate of pair p as lam_p, so that the
# decay is z <- lam z.  Real dot products over channels are sums of Re(conj(x_p) y_p).  For
# a product y = x c of complex numbers, the gradient (dL/dRe + i dL/dIm) passes as
# g_x = g_y conj(c); the gate gradient is therefore the conjugate of the real formula's
# exclusive-product sum, with complex weights.

def cx(x):
    """[.., 2P] real pairs -> [.., P] complex."""
    return x[..., 0::2] + 1j * x[..., 1::2]


def pairs(z):
    """[.., P] complex -> [.., 2P] real pairs."""
    out = np.empty(z.shape[:-1] + (2 * z.shape[-1],))
    out[..., 0::2], out[..., 1::2] = z.real, z.imag
    return out


def _rot_rows(g, S):
    """Rows (2p, 2p+1) of S times the complex g_p (g [P], S [2P, dv])."""
    Z = g[:, None] * (S[0::2] + 1j * S[1::2])
    out = np.empty_like(S)
    out[0::2], out[1::2] = Z.real, Z.imag
    return out


def _ranges_cpx(lam):
    C, P = lam.shape
    r = np.zeros((C, C, P), complex)
    for j in range(C):
        run = np.ones(P, complex)
        r[j, j] = 1.0
        for i in range(j + 1, C):
            run = run * lam[i]
            r[i, j] = run
    return r


def blocked_decay_grads_cpx(dA, dD, q, k, lam, av, bv, dgl):
    """Complex form of blocked_decay_grads (q, k, lam, av, bv [C, P] complex; dgl [P]):
    the same block anchoring, with conj(r) on the key side (Zc and its fold term F) and
    conj(q), conj(k) in the pair weights.  Returns Zq, Zr, Zc and the gate gradient as
    dL/dRe + i dL/dIm per pair."""
    C, P = q.shape
    NB = C // SUB
    pin, sig, pib = np.zeros((C, P), complex), np.zeros((C, P), complex), np.zeros((NB, P), complex)
    for I in range(NB):
        p = np.ones(P, complex)
        for r in range(SUB):
            p = p * lam[I * SUB + r]
            pin[I * SUB + r] = p
        pib[I] = p
        sf = np.ones(P, complex)
        for r in range(SUB - 1, -1, -1):
            sig[I * SUB + r] = sf
            sf = sf * lam[I * SUB + r]

    def between(J, I):
        p = np.ones(P, complex)
        for y in range(J + 1, I):
            p = p * pib[y]
        return p

    PA, PD, F = np.zeros((NB, C, P), complex), np.zeros((NB, C, P), complex), np.zeros((C, P), complex)
    for M in range(1, NB):
        s = M * SUB
        khat = np.stack([k[j] * sig[j] * between(j // SUB, M) for j in range(s)])
        PA[M, s:] = dA[s:, :s] @ khat
        PD[M, s:] = dD[s:, :s] @ khat
    for M in range(NB - 1):
        s, e1 = M * SUB, M * SUB + SUB
        rie = np.conj(np.stack([pin[i] * between(M, i // SUB) for i in range(e1, C)]))
        F[s:e1] = dA[e1:, s:e1].T @ (q[e1:] * rie) + dD[e1:, s:e1].T @ (k[e1:] * rie)

    Zq, Zr, Zc = np.zeros((C, P), complex), np.zeros((C, P), complex), np.zeros((C, P), complex)
    dal = np.zeros((C, P), complex)
    for M in range(NB):
        s = M * SUB
        al, qv, kv = lam[s:s + SUB], q[s:s + SUB], k[s:s + SUB]
        gs = np.prod(pib[:M], axis=0) if M > 0 else np.ones(P, complex)
        rend = np.prod(pib[M + 1:], axis=0) if M < NB - 1 else np.ones(P, complex)
        for r in range(SUB):
            i = s + r
            zq, zr, Pr = dA[i, i] * kv[r], np.zeros(P, complex), np.ones(P, complex)
            for rj in range(r - 1, -1, -1):
                Pr = Pr * al[rj + 1]
                zq = zq + dA[i, s + rj] * kv[rj] * Pr
                zr = zr + dD[i, s + rj] * kv[rj] * Pr
            if M > 0:
                zq = zq + pin[i] * PA[M, i]
                zr = zr + pin[i] * PD[M, i]
            zc, Pr = dA[i, i] * qv[r], np.ones(P, complex)
            for ri in range(r + 1, SUB):
                Pr = Pr * al[ri]
                zc = zc + (dA[s + ri, i] * qv[ri] + dD[s + ri, i] * kv[ri]) * np.conj(Pr)
            if M < NB - 1:
                zc = zc + np.conj(sig[i]) * F[i]
            Zq[i], Zr[i], Zc[i] = zq, zr, zc
        bvs = sum((bv[j] * sig[j] * between(j // SUB, M) for j in range(s)), np.zeros(P, complex))

        def g_at(i):
            g = av[i] * gs
            if M > 0:
                g = g + np.conj(q[i]) * PA[M, i] + np.conj(k[i]) * PD[M, i]
            if i == C - 1:
                g = g + bvs + dgl * gs
            return g

        u = [g_at(s + r) for r in range(SUB)]
        if M < NB - 1:
            xf = np.zeros(P, complex)
            for i in range(C - 1, s + SUB - 1, -1):
                xf = lam[i] * (g_at(i) + xf)
            u[SUB - 1] = u[SUB - 1] + xf
            f = [kv[r] * np.conj(F[s + r]) + bv[s + r] * rend for r in range(SUB)]
        else:
            f = [bv[s + r] for r in range(SUB)]
        for m in range(SUB):
            acc = u[SUB - 1]
            for i in range(SUB - 2, m - 1, -1):
                acc = u[i] + al[i + 1] * acc
            dal[s + m] = acc
            for i in range(m + 1, SUB):
                E = (np.conj(qv[i]) * dA[s + i, s + m] + np.conj(kv[i]) * dD[s + i, s + m]) * kv[m]
                if i == SUB - 1:
                    E = E + f[m]
                u[i] = al[m] * u[i] + E
    return Zq, Zr, Zc, np.conj(dal)


def chunk_backward_sfda(q, k, v, lam, beta, dO, S0=None, dST=None, C=64, blocked=False):
    """SFDA gradients for one head through the chunk algebra (fp64).  lam [T, dk] holds
    (Re, Im) of each pair's gate.  Per chunk, with complex ranges r_ij = prod_{j<l<=i} lam_l,
    gamma_i = r_(i,-1), rho_j = r_(C-1,j): Q~ = q conj(gamma), K~g = k conj(gamma),
    K~r = rho k (pairs), A_ij = sum_p Re(conj(q_ip) r_ijp k_jp), D likewise with k_i, and the
    chunk-end decay multiplies the state's row pairs by gamma_last.  Returns dq, dk, dv,
    dalpha (d/dRe, d/dIm in channels 2p, 2p+1), dbeta, dS0.  blocked: decayed sums and
    gate gradient from blocked_decay_grads_cpx."""
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, np.float64).copy()
    low, slow = np.tril(np.ones((C, C))), np.tril(np.ones((C, C)), -1)
    parts = []
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        pad = lambda x, fill: np.concatenate([x[c0:c0 + n], np.full((C - n,) + x.shape[1:], fill)])[:C]
        qc, kc, vc, bc, dOc = pad(q, 0.0), pad(k, 0.0), pad(v, 0.0), pad(beta, 0.0), pad(dO, 0.0)
        lc = np.concatenate([cx(lam[c0:c0 + n]), np.ones((C - n, dk // 2), complex)])
        qh, kh = cx(qc), cx(kc)
        r = _ranges_cpx(lc)
        gam = np.cumprod(lc, axis=0)
        rho, gL = r[C - 1], gam[C - 1]
        A = np.einsum("ip,ijp,jp->ij", np.conj(qh), r, kh).real * low
        D = np.einsum("ip,ijp,jp->ij", np.conj(kh), r, kh).real * slow
        M = np.linalg.inv(np.eye(C) + bc[:, None] * D)
        Mt = M * bc[None, :]
        Qg, Kg, Kr = pairs(qh * np.conj(gam)), pairs(kh * np.conj(gam)), pairs(rho * kh)
        W = Mt @ Kg
        Dl = Mt @ vc - W @ S
        Sn = _rot_rows(gL, S) + Kr.T @ Dl
        parts.append(dict(S=S, q=qh, k=kh, v=vc, lam=lc, beta=bc, dO=dOc, r=r, gam=gam, rho=rho, gL=gL, A=A,
                          D=D, M=M, Mt=Mt, Qg=Qg, Kg=Kg, Kr=Kr, W=W, Dl=Dl, c0=c0, n=n))
        S = Sn
    out = {x: np.zeros((T, dk)) for x in ("dq", "dk", "dalpha")}
    out["dv"], out["dbeta"] = np.zeros((T, dv)), np.zeros(T)
    dSn = np.zeros((dk, dv)) if dST is None else np.asarray(dST, np.float64).copy()
    for p in reversed(parts):
        S, dO_, qh, kh, lc = p["S"], p["dO"], p["q"], p["k"], p["lam"]
        r, gam, rho, gL = p["r"], p["gam"], p["rho"], p["gL"]
        dDl = p["Kr"] @ dSn + p["A"].T @ dO_
        dS = _rot_rows(np.conj(gL), dSn) + p["Qg"].T @ dO_ - p["W"].T @ dDl
        dQg, dKr, dW = dO_ @ S.T, p["Dl"] @ dSn.T, -dDl @ S.T
        dA = (dO_ @ p["Dl"].T) * low
        dV = p["Mt"].T @ dDl
        dMt = (dDl @ p["v"].T + dW @ p["Kg"].T) * low
        dKg = p["Mt"].T @ dW
        dbeta = (dMt * p["M"]).sum(axis=0)
        dT = -(p["M"].T @ (dMt * p["beta"][None, :]) @ p["M"].T) * slow
        dbeta = dbeta + (dT * p["D"]).sum(axis=1)
        dD = p["beta"][:, None] * dT
        dQh, dKgh, dKrh = cx(dQg), cx(dKg), cx(dKr)
        av = dQh * np.conj(qh) + dKgh * np.conj(kh)
        bv = np.conj(dKrh) * kh
        dgl = (np.conj(cx(dSn.T)) * cx(S.T)).sum(axis=0)            # sum_j conj(dS'_j) S_j
        if blocked:
            Zq, Zr, Zc, dlam = blocked_decay_grads_cpx(dA, dD, qh, kh, lc, av, bv, dgl)
        else:
            Zq = np.einsum("ij,ijp,jp->ip", dA, r, kh)
            Zr = np.einsum("ij,ijp,jp->ip", dD, r, kh)
            Zc = np.einsum("ij,ijp,ip->jp", dA, np.conj(r), qh) + np.einsum("ij,ijp,ip->jp", dD, np.conj(r), kh)
            E = np.einsum("ij,ip,jp->ijp", dA, np.conj(qh), kh) + np.einsum("ij,ip,jp->ijp", dD, np.conj(kh), kh)
            dlam = np.zeros((C, dk // 2), complex)
            for m in range(C):
                gm1 = np.prod(lc[:m], axis=0)                                         # gamma_(m-1)
                left = np.stack([np.prod(lc[j + 1:m], axis=0) for j in range(m)]) if m else None
                tot = np.zeros(dk // 2, complex)
                for i in range(m, C):
                    right = np.prod(lc[m + 1:i + 1], axis=0)                           # r_(i, m)
                    inner = av[i] * gm1 + ((E[i, :m] * left).sum(axis=0) if m else 0.0)
                    tot = tot + right * inner
                tail = dgl * gm1 + ((bv[:m] * left).sum(axis=0) if m else 0.0)
                tot = tot + np.prod(lc[m + 1:], axis=0) * tail
                dlam[m] = np.conj(tot)
        dq = pairs(dQh * gam + Zq)
        dk_ = pairs(dKgh * gam + dKrh * np.conj(rho) + Zr + Zc)
        n, c0 = p["n"], p["c0"]
        out["dq"][c0:c0 + n] = dq[:n]
        out["dk"][c0:c0 + n] = dk_[:n]
        out["dv"][c0:c0 + n] = dV[:n]
        out["dalpha"][c0:c0 + n] = pairs(dlam)[:n]
        out["dbeta"][c0:c0 + n] = dbeta[:n]
        dSn = dS
    out["dS0"] = dSn
    return out
