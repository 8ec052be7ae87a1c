/*
 * kda_oracle.c -- plain fp64 CPU oracle for the KDA / CKDA gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the parity reference: only the test
 * suite, the smoke check and the CPU-baseline leg of the benchmark may load
 * it.  It shares no code, header or table with the HIP library.
 *
 * What it computes (one (batch, head) pair at a time, one token at a time):
 *
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *   o_t = S_t^T q_t
 *
 * with S a d_k x d_v matrix (rows = key channels, columns = value channels).
 *   - The recurrence is the real-coordinate form of the update printed on
 *     "Resumen Tecnico: Atencion Delta de Fourier Semidirecta (SFDA)",
 *     section "Arquitectura Central" (phases theta = 0, which the same page's
 *     "Principales Contribuciones" item 1 says recovers KDA), and of the
 *     Gated DeltaNet-2 update on "ملخص تقني: Gated DeltaNet-2", section 1,
 *     with the erase and write gates tied to one scalar beta (the KDA case
 *     stated right after that equation).  The conjugate transposes of the
 *     complex form are plain transposes for real data.
 *   - The decay Diag(alpha_t) acts on the key dimension (rows of S) and is
 *     applied before the erase/write, as D_t is placed in the Gated
 *     DeltaNet-2 equation.
 *   - CKDA allows alpha in [-1, 1] per channel and beta in [0, 2]
 *     ("Complex KDA: ..." page, section "Complex KDA (CKDA) Mimarisi").
 *     Nothing here depends on the range: the oracle is the definition.
 *   - The readout o_t = S_t^T q_t (after the update) is not printed on the
 *     pages; this is the plainest reading (a linear-attention read of the
 *     fixed-size state with the query) and it is the one used throughout.
 *
 * Step order inside one token, written out literally:
 *   1. S <- Diag(alpha) S                       (row i scaled by alpha_i)
 *   2. u <- S^T k                               (read of the old content)
 *   3. S <- S + beta k (v - u)^T                (= (I - beta k k^T) S + beta k v^T)
 *   4. o <- S^T q
 *
 * Columns of S evolve independently (every step above acts on one column at
 * a time), so the work is split over (head, column block) for OpenMP; each
 * column still runs the full serial recurrence over t.
 *
 * Inputs are the exact bytes given to the GPU (bf16 bit patterns or fp32),
 * widened exactly to fp64.  Nothing is normalised or rescaled here.
 *
 * Parity pins: the recurrence (fwd and decode) is pinned by the CPU tests
 * against explicit transition-matrix products, the plain delta rule, pure
 * decay, non-expansiveness, norm preservation and the d=2 rotation.
 *
 * Gated DeltaNet-2 ("ملخص تقني: Gated DeltaNet-2", section 1) splits the scalar
 * beta into an erase gate b_t per key channel and a write gate w_t per value
 * channel:
 *
 *   S_t = (I - k_t (b_t o k_t)^T) D_t S_{t-1} + k_t (w_t o v_t)^T,  D_t = Diag(alpha_t)
 *
 * (o: elementwise product), with the same readout.  kda_oracle_fwd_gdn2 and
 * kda_oracle_decode_gdn2 below run that update one token at a time; the CPU
 * tests pin them against explicit transition-matrix products, against the KDA
 * functions when b = w = beta (the reduction the page states), against the
 * no-erase case (b = 0: a decayed sum of writes) and against a hand-worked
 * two-token case.
 *
 * SFDA with phase control ("Resumen Tecnico: Atencion Delta de Fourier
 * Semidirecta (SFDA)", section "Arquitectura Central"): the real decay
 * Diag(alpha_t) becomes Lambda_t = diag(alpha_t o e^{i theta_t}) in complex
 * coordinates, which the same section says is built in real coordinates as a
 * direct sum of 2 x 2 rotation-decay blocks.  Reading taken here: key channels
 * 2p and 2p+1 form complex coordinate p; the gate of coordinate p is the
 * complex number lambda_p = alpha_p e^{i theta_p}, handed over as its real and
 * imaginary parts in channels 2p and 2p+1 of the gate tensor; k, q, v, beta and
 * the state stay real (the kernel-compatible real family Lambda_t - u_t r_t^*
 * of the same page, section "Expresividad de Estado Finito"), so
 *
 *   S_t = (I - beta_t k_t k_t^T) Lambda_t S_{t-1} + beta_t k_t v_t^T,
 *   (Lambda S)[2p]   = Re(lambda_p) S[2p] - Im(lambda_p) S[2p+1]
 *   (Lambda S)[2p+1] = Im(lambda_p) S[2p] + Re(lambda_p) S[2p+1]
 *
 * (rows 2p, 2p+1 of every column, read as z = S[2p] + i S[2p+1], become
 * lambda_p z).  kda_oracle_fwd_sfda and kda_oracle_decode_sfda run that update;
 * the CPU tests pin them against the KDA functions when every phase is zero
 * (Im lambda = 0, both channels of a pair decayed by Re lambda; the page's
 * "Principales Contribuciones" item 1), against the closed form of pure
 * rotation-decay (beta = 0: z_t = (prod lambda) z_0, with numpy's complex
 * products), against an exact phase-only cyclic counter, against dense real
 * transition matrices and against a hand-worked two-token case.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_BF16 = 0, ORC_F32 = 1, ORC_F64 = 2 };

static double load_elem(const void* base, int dtype, size_t idx) {
    if (dtype == ORC_BF16) {
        uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    if (dtype == ORC_F32) return (double)((const float*)base)[idx];
    return ((const double*)base)[idx];
}

/* One token of the recurrence on columns [j0, j1) of a d_k x d_v state.
 * cpx = 0: Diag(alpha) decay (KDA / CKDA); cpx = 1: SFDA rotation-decay, a[2p] and
 * a[2p+1] being the real and imaginary parts of the gate of coordinate p. */
static void kda_token(double* S, int dk, int dv, int j0, int j1,
                      const double* q, const double* k, const double* v,
                      const double* a, double beta, double* u, double* o, int cpx) {
    /* 1. decay: S <- Diag(alpha) S, or S <- Lambda S (row pairs times lambda_p) */
    if (!cpx) {
        for (int i = 0; i < dk; ++i)
            for (int j = j0; j < j1; ++j) S[(size_t)i * dv + j] *= a[i];
    } else {
        for (int p = 0; p < dk / 2; ++p) {
            const double lr = a[2 * p], li = a[2 * p + 1];
            for (int j = j0; j < j1; ++j) {
                const double x = S[(size_t)(2 * p) * dv + j], y = S[(size_t)(2 * p + 1) * dv + j];
                S[(size_t)(2 * p) * dv + j] = lr * x - li * y;
                S[(size_t)(2 * p + 1) * dv + j] = li * x + lr * y;
            }
        }
    }
    /* 2. read: u = S^T k */
    for (int j = j0; j < j1; ++j) u[j] = 0.0;
    for (int i = 0; i < dk; ++i)
        for (int j = j0; j < j1; ++j) u[j] += k[i] * S[(size_t)i * dv + j];
    /* 3. erase + write: S <- S + beta k (v - u)^T */
    for (int i = 0; i < dk; ++i)
        for (int j = j0; j < j1; ++j)
            S[(size_t)i * dv + j] += beta * k[i] * (v[j] - u[j]);
    /* 4. readout: o = S^T q */
    if (o) {
        for (int j = j0; j < j1; ++j) o[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = j0; j < j1; ++j) o[j] += q[i] * S[(size_t)i * dv + j];
    }
}

static int pick_threads(int nthreads) {
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/*
 * Forward over whole sequences.
 *   q, k, alpha : [B, T, H, dk]   (dtype)
 *   v           : [B, T, H, dv]   (dtype)
 *   beta        : [B, T, H]       (dtype)
 *   S0          : [n_sel, dk, dv] fp64, or NULL for zeros
 *   o_out       : [n_sel, T, dv]  fp64, or NULL
 *   S_out       : [n_sel, dk, dv] fp64, or NULL
 *   sel         : n_sel flat head indices b*H + h, or NULL (then n_sel = B*H)
 *   col_block   : width of the column blocks handed to threads (<= 0: dv)
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
static int fwd_common(int B, int T, int H, int dk, int dv, int dtype,
                      const void* q, const void* k, const void* v,
                      const void* alpha, const void* beta, const double* S0,
                      double* o_out, double* S_out, const int* sel, int n_sel,
                      int col_block, int nthreads, int cpx) {
    if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (cpx && dk % 2) return -1;
    if (dtype < ORC_BF16 || dtype > ORC_F64) return -1;
    if (!sel) n_sel = B * H;
    if (n_sel < 0) return -1;
    if (col_block <= 0 || col_block > dv) col_block = dv;
    const int nblk = (dv + col_block - 1) / col_block;
    const long n_items = (long)n_sel * nblk;
    int err = 0;

#pragma omp parallel num_threads(pick_threads(nthreads))
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
        double* buf = (double*)malloc(sizeof(double) * (size_t)(3 * dk + 3 * dv));
        if (!S || !buf) {
#pragma omp atomic write
            err = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (long it = 0; it < n_items; ++it) {
            if (!S || !buf) continue;
            const int s = (int)(it / nblk);
            const int j0 = (int)(it % nblk) * col_block;
            const int j1 = j0 + col_block < dv ? j0 + col_block : dv;
            const int bh = sel ? sel[s] : s;
            const int b = bh / H, h = bh % H;
            double *qq = buf, *kk = buf + dk, *aa = buf + 2 * dk;
            double *vv = buf + 3 * dk, *u = vv + dv, *oo = u + dv;
            for (int i = 0; i < dk; ++i)
                for (int j = j0; j < j1; ++j)
                    S[(size_t)i * dv + j] = S0 ? S0[((size_t)s * dk + i) * dv + j] : 0.0;
            for (int t = 0; t < T; ++t) {
                const size_t row = ((size_t)b * T + t) * H + h;
                for (int i = 0; i < dk; ++i) {
                    qq[i] = load_elem(q, dtype, row * dk + i);
                    kk[i] = load_elem(k, dtype, row * dk + i);
                    aa[i] = load_elem(alpha, dtype, row * dk + i);
                }
                for (int j = j0; j < j1; ++j) vv[j] = load_elem(v, dtype, row * dv + j);
                const double bt = load_elem(beta, dtype, row);
                kda_token(S, dk, dv, j0, j1, qq, kk, vv, aa, bt, u, o_out ? oo : NULL, cpx);
                if (o_out)
                    for (int j = j0; j < j1; ++j)
                        o_out[((size_t)s * T + t) * dv + j] = oo[j];
            }
            if (S_out)
                for (int i = 0; i < dk; ++i)
                    for (int j = j0; j < j1; ++j)
                        S_out[((size_t)s * dk + i) * dv + j] = S[(size_t)i * dv + j];
        }
        free(S);
        free(buf);
    }
    return err ? -1 : 0;
}

int kda_oracle_fwd(int B, int T, int H, int dk, int dv, int dtype,
                   const void* q, const void* k, const void* v,
                   const void* alpha, const void* beta, const double* S0,
                   double* o_out, double* S_out, const int* sel, int n_sel,
                   int col_block, int nthreads) {
    return fwd_common(B, T, H, dk, dv, dtype, q, k, v, alpha, beta, S0, o_out, S_out, sel, n_sel,
                      col_block, nthreads, 0);
}

/* SFDA forward: as kda_oracle_fwd with alpha [B, T, H, dk] holding the complex gates
 * (real part in channel 2p, imaginary part in channel 2p+1); dk must be even. */
int kda_oracle_fwd_sfda(int B, int T, int H, int dk, int dv, int dtype,
                        const void* q, const void* k, const void* v,
                        const void* lambda, const void* beta, const double* S0,
                        double* o_out, double* S_out, const int* sel, int n_sel,
                        int col_block, int nthreads) {
    return fwd_common(B, T, H, dk, dv, dtype, q, k, v, lambda, beta, S0, o_out, S_out, sel, n_sel,
                      col_block, nthreads, 1);
}

/*
 * One recurrent decode step (the same token body), state carried by caller.
 *   q, k, alpha : [B, H, dk]; v : [B, H, dv]; beta : [B, H]   (dtype)
 *   state       : [n_sel, dk, dv] fp64, updated in place
 *   o_out       : [n_sel, dv] fp64, or NULL
 */
static int decode_common(int B, int H, int dk, int dv, int dtype,
                         const void* q, const void* k, const void* v,
                         const void* alpha, const void* beta, double* state,
                         double* o_out, const int* sel, int n_sel, int nthreads, int cpx) {
    if (B < 0 || H <= 0 || dk <= 0 || dv <= 0 || !state) return -1;
    if (cpx && dk % 2) return -1;
    if (dtype < ORC_BF16 || dtype > ORC_F64) return -1;
    if (!sel) n_sel = B * H;
    if (n_sel < 0) return -1;
    int err = 0;
#pragma omp parallel num_threads(pick_threads(nthreads))
    {
        double* buf = (double*)malloc(sizeof(double) * (size_t)(3 * dk + 3 * dv));
        if (!buf) {
#pragma omp atomic write
            err = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int s = 0; s < n_sel; ++s) {
            if (!buf) continue;
            const int bh = sel ? sel[s] : s;
            double *qq = buf, *kk = buf + dk, *aa = buf + 2 * dk;
            double *vv = buf + 3 * dk, *u = vv + dv, *oo = u + dv;
            for (int i = 0; i < dk; ++i) {
                qq[i] = load_elem(q, dtype, (size_t)bh * dk + i);
                kk[i] = load_elem(k, dtype, (size_t)bh * dk + i);
                aa[i] = load_elem(alpha, dtype, (size_t)bh * dk + i);
            }
            for (int j = 0; j < dv; ++j) vv[j] = load_elem(v, dtype, (size_t)bh * dv + j);
            const double bt = load_elem(beta, dtype, (size_t)bh);
            kda_token(state + (size_t)s * dk * dv, dk, dv, 0, dv, qq, kk, vv, aa, bt, u,
                      o_out ? oo : NULL, cpx);
            if (o_out)
                for (int j = 0; j < dv; ++j) o_out[(size_t)s * dv + j] = oo[j];
        }
        free(buf);
    }
    return err ? -1 : 0;
}

int kda_oracle_decode(int B, int H, int dk, int dv, int dtype,
                      const void* q, const void* k, const void* v,
                      const void* alpha, const void* beta, double* state,
                      double* o_out, const int* sel, int n_sel, int nthreads) {
    return decode_common(B, H, dk, dv, dtype, q, k, v, alpha, beta, state, o_out, sel, n_sel,
                         nthreads, 0);
}

/* One SFDA decode step: lambda [B, H, dk] holds the complex gates as in kda_oracle_fwd_sfda. */
int kda_oracle_decode_sfda(int B, int H, int dk, int dv, int dtype,
                           const void* q, const void* k, const void* v,
                           const void* lambda, const void* beta, double* state,
                           double* o_out, const int* sel, int n_sel, int nthreads) {
    return decode_common(B, H, dk, dv, dtype, q, k, v, lambda, beta, state, o_out, sel, n_sel,
                         nthreads, 1);
}

/* One Gated DeltaNet-2 token on columns [j0, j1): the read goes through the erase
 * gate on the key side, the write through the write gate on the value side. */
static void gdn2_token(double* S, int dk, int dv, int j0, int j1,
                       const double* q, const double* k, const double* v,
                       const double* a, const double* eg, const double* wg,
                       double* u, double* o) {
    /* 1. decay: S <- D S */
    for (int i = 0; i < dk; ++i)
        for (int j = j0; j < j1; ++j) S[(size_t)i * dv + j] *= a[i];
    /* 2. read through the erase gate: u = S^T (b o k) */
    for (int j = j0; j < j1; ++j) u[j] = 0.0;
    for (int i = 0; i < dk; ++i) {
        const double e = eg[i] * k[i];
        for (int j = j0; j < j1; ++j) u[j] += e * S[(size_t)i * dv + j];
    }
    /* 3. erase + write: S <- S + k ((w o v) - u)^T
     *    (= (I - k (b o k)^T) D S + k (w o v)^T with D S from step 1) */
    for (int i = 0; i < dk; ++i)
        for (int j = j0; j < j1; ++j)
            S[(size_t)i * dv + j] += k[i] * (wg[j] * v[j] - u[j]);
    /* 4. readout: o = S^T q */
    if (o) {
        for (int j = j0; j < j1; ++j) o[j] = 0.0;
        for (int i = 0; i < dk; ++i)
            for (int j = j0; j < j1; ++j) o[j] += q[i] * S[(size_t)i * dv + j];
    }
}

/*
 * Gated DeltaNet-2 forward over whole sequences.  As kda_oracle_fwd, with the
 * scalar beta replaced by
 *   erase : [B, T, H, dk]  erase gate b (dtype)
 *   write : [B, T, H, dv]  write gate w (dtype)
 */
int kda_oracle_fwd_gdn2(int B, int T, int H, int dk, int dv, int dtype,
                        const void* q, const void* k, const void* v,
                        const void* alpha, const void* erase, const void* write,
                        const double* S0, double* o_out, double* S_out,
                        const int* sel, int n_sel, int col_block, int nthreads) {
    if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    if (dtype < ORC_BF16 || dtype > ORC_F64) return -1;
    if (!sel) n_sel = B * H;
    if (n_sel < 0) return -1;
    if (col_block <= 0 || col_block > dv) col_block = dv;
    const int nblk = (dv + col_block - 1) / col_block;
    const long n_items = (long)n_sel * nblk;
    int err = 0;

#pragma omp parallel num_threads(pick_threads(nthreads))
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
        double* buf = (double*)malloc(sizeof(double) * (size_t)(4 * dk + 4 * dv));
        if (!S || !buf) {
#pragma omp atomic write
            err = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (long it = 0; it < n_items; ++it) {
            if (!S || !buf) continue;
            const int s = (int)(it / nblk);
            const int j0 = (int)(it % nblk) * col_block;
            const int j1 = j0 + col_block < dv ? j0 + col_block : dv;
            const int bh = sel ? sel[s] : s;
            const int b = bh / H, h = bh % H;
            double *qq = buf, *kk = buf + dk, *aa = buf + 2 * dk, *ee = buf + 3 * dk;
            double *vv = buf + 4 * dk, *ww = vv + dv, *u = ww + dv, *oo = u + dv;
            for (int i = 0; i < dk; ++i)
                for (int j = j0; j < j1; ++j)
                    S[(size_t)i * dv + j] = S0 ? S0[((size_t)s * dk + i) * dv + j] : 0.0;
            for (int t = 0; t < T; ++t) {
                const size_t tok = ((size_t)b * T + t) * H + h;
                for (int i = 0; i < dk; ++i) {
                    qq[i] = load_elem(q, dtype, tok * dk + i);
                    kk[i] = load_elem(k, dtype, tok * dk + i);
                    aa[i] = load_elem(alpha, dtype, tok * dk + i);
                    ee[i] = load_elem(erase, dtype, tok * dk + i);
                }
                for (int j = j0; j < j1; ++j) {
                    vv[j] = load_elem(v, dtype, tok * dv + j);
                    ww[j] = load_elem(write, dtype, tok * dv + j);
                }
                gdn2_token(S, dk, dv, j0, j1, qq, kk, vv, aa, ee, ww, u, o_out ? oo : NULL);
                if (o_out)
                    for (int j = j0; j < j1; ++j)
                        o_out[((size_t)s * T + t) * dv + j] = oo[j];
            }
            if (S_out)
                for (int i = 0; i < dk; ++i)
                    for (int j = j0; j < j1; ++j)
                        S_out[((size_t)s * dk + i) * dv + j] = S[(size_t)i * dv + j];
        }
        free(S);
        free(buf);
    }
    return err ? -1 : 0;
}

/* One Gated DeltaNet-2 decode step: erase [B, H, dk], write [B, H, dv]. */
int kda_oracle_decode_gdn2(int B, int H, int dk, int dv, int dtype,
                           const void* q, const void* k, const void* v,
                           const void* alpha, const void* erase, const void* write,
                           double* state, double* o_out, const int* sel, int n_sel,
                           int nthreads) {
    if (B < 0 || H <= 0 || dk <= 0 || dv <= 0 || !state) return -1;
    if (dtype < ORC_BF16 || dtype > ORC_F64) return -1;
    if (!sel) n_sel = B * H;
    if (n_sel < 0) return -1;
    int err = 0;
#pragma omp parallel num_threads(pick_threads(nthreads))
    {
        double* buf = (double*)malloc(sizeof(double) * (size_t)(4 * dk + 4 * dv));
        if (!buf) {
#pragma omp atomic write
            err = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int s = 0; s < n_sel; ++s) {
            if (!buf) continue;
            const int bh = sel ? sel[s] : s;
            double *qq = buf, *kk = buf + dk, *aa = buf + 2 * dk, *ee = buf + 3 * dk;
            double *vv = buf + 4 * dk, *ww = vv + dv, *u = ww + dv, *oo = u + dv;
            for (int i = 0; i < dk; ++i) {
                qq[i] = load_elem(q, dtype, (size_t)bh * dk + i);
                kk[i] = load_elem(k, dtype, (size_t)bh * dk + i);
                aa[i] = load_elem(alpha, dtype, (size_t)bh * dk + i);
                ee[i] = load_elem(erase, dtype, (size_t)bh * dk + i);
            }
            for (int j = 0; j < dv; ++j) {
                vv[j] = load_elem(v, dtype, (size_t)bh * dv + j);
                ww[j] = load_elem(write, dtype, (size_t)bh * dv + j);
            }
            gdn2_token(state + (size_t)s * dk * dv, dk, dv, 0, dv, qq, kk, vv, aa, ee, ww, u,
                       o_out ? oo : NULL);
            if (o_out)
                for (int j = 0; j < dv; ++j) o_out[(size_t)s * dv + j] = oo[j];
        }
        free(buf);
    }
    return err ? -1 : 0;
}

/*
 * Backward of the KDA / CKDA forward: the gradients of
 *   L = sum_t <dO_t, o_t> + <dS_T, S_T>
 * with respect to q, k, v, alpha, beta and S_0, by reverse-mode differentiation of the
 * token recurrence above (the training use of the chunked forward on the GDN-2 page,
 * section 3; the pages print no backward formulas, so this is the plain adjoint of the
 * literal step order).  Per token, with S_prev = S_{t-1} and G the gradient with respect
 * to S_t:
 *   forward   S' = Diag(alpha) S_prev;  u = S'^T k;  delta = v - u;  S_t = S' + beta k delta^T
 *   G        += q dO_t^T                      (o_t = S_t^T q)
 *   dq_t      = S_t dO_t
 *   ddelta    = beta G^T k;   dv_t = ddelta;   dbeta_t = k^T G delta
 *   dk_t      = beta G delta - S' ddelta
 *   dS'       = G - k ddelta^T
 *   dalpha_t  = rowsum(dS' o S_prev)
 *   G         = Diag(alpha) dS'               (now the gradient with respect to S_{t-1})
 * and dS_0 = G after the first token.  The states S_{t-1} are recomputed one 64-token
 * block at a time from checkpoints taken every 64 tokens of a forward sweep.
 *
 *   dO    : [n_sel, T, dv] fp64;  dST : [n_sel, dk, dv] fp64 or NULL (zero)
 *   dq, dk_out, dalpha : [n_sel, T, dk] fp64;  dv_out : [n_sel, T, dv];  dbeta : [n_sel, T]
 *   dS0   : [n_sel, dk, dv] fp64 or NULL
 * Other arguments as kda_oracle_fwd.  Parallel over heads.
 */
/* erase == NULL: KDA / CKDA (beta, dbeta); else Gated DeltaNet-2 (erase, write, derase,
 * dwrite in their place). */
static int bwd_common(int B, int T, int H, int dk, int dv, int dtype,
                      const void* q, const void* k, const void* v,
                      const void* alpha, const void* beta, const void* erase, const void* write,
                      const double* S0, const double* dO, const double* dST,
                      double* dq, double* dk_out, double* dv_out, double* dalpha, double* dbeta,
                      double* derase, double* dwrite,
                      double* dS0, const int* sel, int n_sel, int nthreads, int cpx) {
    const int g2 = erase != NULL;
    if (cpx && (g2 || dk % 2)) return -1;
    if (B < 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0 || !dO) return -1;
    if (!dq || !dk_out || !dv_out || !dalpha) return -1;
    if (g2 ? (!write || !derase || !dwrite) : !dbeta) return -1;
    if (dtype < ORC_BF16 || dtype > ORC_F64) return -1;
    if (!sel) n_sel = B * H;
    if (n_sel < 0) return -1;
    const int BLK = 64;
    const int nblk = (T + BLK - 1) / BLK;
    const size_t SS = (size_t)dk * dv;
    int err = 0;

#pragma omp parallel num_threads(pick_threads(nthreads))
    {
        double* ck = (double*)malloc(sizeof(double) * SS * (size_t)(nblk > 0 ? nblk : 1));
        double* hist = (double*)malloc(sizeof(double) * SS * (size_t)(BLK + 1));
        double* G = (double*)malloc(sizeof(double) * SS);
        double* Sp = (double*)malloc(sizeof(double) * SS);   /* S' of the current token */
        double* buf = (double*)malloc(sizeof(double) * (size_t)(5 * dk + 6 * dv));
        if (!ck || !hist || !G || !Sp || !buf) {
#pragma omp atomic write
            err = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int s = 0; s < n_sel; ++s) {
            if (!ck || !hist || !G || !Sp || !buf) continue;
            const int bh = sel ? sel[s] : s;
            const int b = bh / H, h = bh % H;
            double *qq = buf, *kk = buf + dk, *aa = buf + 2 * dk;
            double *vv = buf + 3 * dk, *u = vv + dv, *del = u + dv, *dd = del + dv, *tmp = dd + dv;
            double *bb = tmp + dv, *ee = bb + dk, *ww = ee + dk;  /* GDN-2: erase gate, b o k, write gate */
            /* forward sweep: checkpoint S at the start of every 64-token block */
            double* S = hist;  /* scratch for the sweep */
            for (size_t x = 0; x < SS; ++x) S[x] = S0 ? S0[(size_t)s * SS + x] : 0.0;
            for (int t = 0; t < T; ++t) {
                if (t % BLK == 0) memcpy(ck + (size_t)(t / BLK) * SS, S, sizeof(double) * SS);
                const size_t row = ((size_t)b * T + t) * H + h;
                for (int i = 0; i < dk; ++i) {
                    qq[i] = load_elem(q, dtype, row * dk + i);
                    kk[i] = load_elem(k, dtype, row * dk + i);
                    aa[i] = load_elem(alpha, dtype, row * dk + i);
                }
                for (int j = 0; j < dv; ++j) vv[j] = load_elem(v, dtype, row * dv + j);
                if (g2) {
                    for (int i = 0; i < dk; ++i) bb[i] = load_elem(erase, dtype, row * dk + i);
                    for (int j = 0; j < dv; ++j) ww[j] = load_elem(write, dtype, row * dv + j);
                    gdn2_token(S, dk, dv, 0, dv, qq, kk, vv, aa, bb, ww, u, NULL);
                } else {
                    kda_token(S, dk, dv, 0, dv, qq, kk, vv, aa, load_elem(beta, dtype, row), u, NULL, cpx);
                }
            }
            /* backward sweep */
            for (size_t x = 0; x < SS; ++x) G[x] = dST ? dST[(size_t)s * SS + x] : 0.0;
            for (int bk = nblk - 1; bk >= 0; --bk) {
                const int t0 = bk * BLK, t1 = t0 + BLK < T ? t0 + BLK : T;
                /* hist[x] = S_{t0 + x - 1}: the states before each token of the block */
                memcpy(hist, ck + (size_t)bk * SS, sizeof(double) * SS);
                for (int t = t0; t < t1 - 1; ++t) {
                    const size_t row = ((size_t)b * T + t) * H + h;
                    for (int i = 0; i < dk; ++i) {
                        qq[i] = load_elem(q, dtype, row * dk + i);
                        kk[i] = load_elem(k, dtype, row * dk + i);
                        aa[i] = load_elem(alpha, dtype, row * dk + i);
                    }
                    for (int j = 0; j < dv; ++j) vv[j] = load_elem(v, dtype, row * dv + j);
                    double* nx = hist + (size_t)(t - t0 + 1) * SS;
                    memcpy(nx, hist + (size_t)(t - t0) * SS, sizeof(double) * SS);
                    if (g2) {
                        for (int i = 0; i < dk; ++i) bb[i] = load_elem(erase, dtype, row * dk + i);
                        for (int j = 0; j < dv; ++j) ww[j] = load_elem(write, dtype, row * dv + j);
                        gdn2_token(nx, dk, dv, 0, dv, qq, kk, vv, aa, bb, ww, u, NULL);
                    } else {
                        kda_token(nx, dk, dv, 0, dv, qq, kk, vv, aa, load_elem(beta, dtype, row), u, NULL, cpx);
                    }
                }
                for (int t = t1 - 1; t >= t0; --t) {
                    const size_t row = ((size_t)b * T + t) * H + h;
                    const double* Sprev = hist + (size_t)(t - t0) * SS;
                    for (int i = 0; i < dk; ++i) {
                        qq[i] = load_elem(q, dtype, row * dk + i);
                        kk[i] = load_elem(k, dtype, row * dk + i);
                        aa[i] = load_elem(alpha, dtype, row * dk + i);
                    }
                    for (int j = 0; j < dv; ++j) vv[j] = load_elem(v, dtype, row * dv + j);
                    const double* dOt = dO + ((size_t)s * T + t) * dv;
                    if (g2) {
                        /* S' = Diag(alpha) S_prev; e = b o k; u = S'^T e; delta = w o v - u;
                         * S_t = S' + k delta^T */
                        for (int i = 0; i < dk; ++i) {
                            bb[i] = load_elem(erase, dtype, row * dk + i);
                            ee[i] = bb[i] * kk[i];
                        }
                        for (int j = 0; j < dv; ++j) ww[j] = load_elem(write, dtype, row * dv + j);
                        for (int i = 0; i < dk; ++i)
                            for (int j = 0; j < dv; ++j) Sp[(size_t)i * dv + j] = Sprev[(size_t)i * dv + j] * aa[i];
                        for (int j = 0; j < dv; ++j) u[j] = 0.0;
                        for (int i = 0; i < dk; ++i)
                            for (int j = 0; j < dv; ++j) u[j] += ee[i] * Sp[(size_t)i * dv + j];
                        for (int j = 0; j < dv; ++j) del[j] = ww[j] * vv[j] - u[j];
                        /* readout: G += q dO^T ; dq = S_t dO */
                        for (int i = 0; i < dk; ++i)
                            for (int j = 0; j < dv; ++j) G[(size_t)i * dv + j] += qq[i] * dOt[j];
                        double* dqg = dq + ((size_t)s * T + t) * dk;
                        for (int i = 0; i < dk; ++i) {
                            double a = 0.0;
                            for (int j = 0; j < dv; ++j) a += (Sp[(size_t)i * dv + j] + kk[i] * del[j]) * dOt[j];
                            dqg[i] = a;
                        }
                        /* ddelta = G^T k ; d(w o v) = ddelta : dv = w o ddelta, dw = v o ddelta */
                        for (int j = 0; j < dv; ++j) dd[j] = 0.0;
                        for (int i = 0; i < dk; ++i)
                            for (int j = 0; j < dv; ++j) dd[j] += G[(size_t)i * dv + j] * kk[i];
                        double* dvg = dv_out + ((size_t)s * T + t) * dv;
                        double* dwg = dwrite + ((size_t)s * T + t) * dv;
                        for (int j = 0; j < dv; ++j) {
                            dvg[j] = ww[j] * dd[j];
                            dwg[j] = vv[j] * dd[j];
                        }
                        /* dk = G delta (write side) + b o de, de = -S' ddelta (read side);
                         * db = k o de */
                        double* dkg = dk_out + ((size_t)s * T + t) * dk;
                        double* dbg = derase + ((size_t)s * T + t) * dk;
                        for (int i = 0; i < dk; ++i) {
                            double w_side = 0.0, de = 0.0;
                            for (int j = 0; j < dv; ++j) {
                                w_side += G[(size_t)i * dv + j] * del[j];
                                de -= Sp[(size_t)i * dv + j] * dd[j];
                            }
                            dkg[i] = w_side + bb[i] * de;
                            dbg[i] = kk[i] * de;
                        }
                        /* dS' = G - e ddelta^T ; dalpha = rowsum(dS' o S_prev) ; G <- Diag(alpha) dS' */
                        double* dag = dalpha + ((size_t)s * T + t) * dk;
                        for (int i = 0; i < dk; ++i) {
                            double a = 0.0;
                            for (int j = 0; j < dv; ++j) {
                                const double g = G[(size_t)i * dv + j] - ee[i] * dd[j];
                                a += Sprev[(size_t)i * dv + j] * g;
                                G[(size_t)i * dv + j] = g * aa[i];
                            }
                            dag[i] = a;
                        }
                        continue;
                    }
                    const double bt = load_elem(beta, dtype, row);
                    /* recompute S' = Diag(alpha) S_prev (SFDA: rows 2p, 2p+1 of every column,
                     * one complex coordinate, times the complex gate aa[2p] + i aa[2p+1]),
                     * u = S'^T k, delta = v - u */
                    if (cpx) {
                        for (int pp = 0; pp < dk / 2; ++pp) {
                            const double lr = aa[2 * pp], li = aa[2 * pp + 1];
                            const double *x0 = Sprev + (size_t)(2 * pp) * dv, *x1 = x0 + dv;
                            double *y0 = Sp + (size_t)(2 * pp) * dv, *y1 = y0 + dv;
                            for (int j = 0; j < dv; ++j) {
                                y0[j] = lr * x0[j] - li * x1[j];
                                y1[j] = li * x0[j] + lr * x1[j];
                            }
                        }
                    } else {
                        for (int i = 0; i < dk; ++i)
                            for (int j = 0; j < dv; ++j) Sp[(size_t)i * dv + j] = aa[i] * Sprev[(size_t)i * dv + j];
                    }
                    for (int j = 0; j < dv; ++j) u[j] = 0.0;
                    for (int i = 0; i < dk; ++i)
                        for (int j = 0; j < dv; ++j) u[j] += kk[i] * Sp[(size_t)i * dv + j];
                    for (int j = 0; j < dv; ++j) del[j] = vv[j] - u[j];
                    /* readout: G += q dO^T ; dq = S_t dO with S_t = S' + beta k delta^T */
                    for (int i = 0; i < dk; ++i)
                        for (int j = 0; j < dv; ++j) G[(size_t)i * dv + j] += qq[i] * dOt[j];
                    double* dqt = dq + ((size_t)s * T + t) * dk;
                    for (int i = 0; i < dk; ++i) {
                        double a = 0.0;
                        for (int j = 0; j < dv; ++j)
                            a += (Sp[(size_t)i * dv + j] + bt * kk[i] * del[j]) * dOt[j];
                        dqt[i] = a;
                    }
                    /* ddelta = beta G^T k ; dv = ddelta ; dbeta = k^T G delta */
                    for (int j = 0; j < dv; ++j) dd[j] = 0.0;
                    for (int i = 0; i < dk; ++i)
                        for (int j = 0; j < dv; ++j) dd[j] += kk[i] * G[(size_t)i * dv + j];
                    double db = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        db += dd[j] * del[j];   /* (G^T k) . delta = k^T G delta */
                        dd[j] *= bt;
                    }
                    dbeta[(size_t)s * T + t] = db;
                    double* dvt = dv_out + ((size_t)s * T + t) * dv;
                    for (int j = 0; j < dv; ++j) dvt[j] = dd[j];
                    /* dk = beta G delta - S' ddelta */
                    double* dkt = dk_out + ((size_t)s * T + t) * dk;
                    for (int i = 0; i < dk; ++i) {
                        double a = 0.0, c = 0.0;
                        for (int j = 0; j < dv; ++j) {
                            a += G[(size_t)i * dv + j] * del[j];
                            c += Sp[(size_t)i * dv + j] * dd[j];
                        }
                        dkt[i] = bt * a - c;
                    }
                    double* dat = dalpha + ((size_t)s * T + t) * dk;
                    if (cpx) {
                        /* dS' = G - k ddelta^T, pair by pair.  S'_0 = lr S_0 - li S_1 and
                         * S'_1 = li S_0 + lr S_1 give dlr = sum_j (g_0 S_0 + g_1 S_1) and
                         * dli = sum_j (g_1 S_0 - g_0 S_1); G <- Lambda^T dS' is
                         * G_0 = lr g_0 + li g_1, G_1 = lr g_1 - li g_0. */
                        for (int pp = 0; pp < dk / 2; ++pp) {
                            const int i0 = 2 * pp, i1 = 2 * pp + 1;
                            const double lr = aa[i0], li = aa[i1];
                            double dre = 0.0, dim = 0.0;
                            for (int j = 0; j < dv; ++j) {
                                const double g0 = G[(size_t)i0 * dv + j] - kk[i0] * dd[j];
                                const double g1 = G[(size_t)i1 * dv + j] - kk[i1] * dd[j];
                                const double s0 = Sprev[(size_t)i0 * dv + j], s1 = Sprev[(size_t)i1 * dv + j];
                                dre += g0 * s0 + g1 * s1;
                                dim += g1 * s0 - g0 * s1;
                                G[(size_t)i0 * dv + j] = lr * g0 + li * g1;
                                G[(size_t)i1 * dv + j] = lr * g1 - li * g0;
                            }
                            dat[i0] = dre;
                            dat[i1] = dim;
                        }
                        continue;
                    }
                    /* dS' = G - k ddelta^T ; dalpha = rowsum(dS' o S_prev) ; G <- Diag(alpha) dS' */
                    for (int i = 0; i < dk; ++i) {
                        double a = 0.0;
                        for (int j = 0; j < dv; ++j) {
                            const double g = G[(size_t)i * dv + j] - kk[i] * dd[j];
                            a += g * Sprev[(size_t)i * dv + j];
                            G[(size_t)i * dv + j] = aa[i] * g;
                        }
                        dat[i] = a;
                    }
                    (void)tmp;
                }
            }
            if (dS0)
                for (size_t x = 0; x < SS; ++x) dS0[(size_t)s * SS + x] = G[x];
        }
        free(ck);
        free(hist);
        free(G);
        free(Sp);
        free(buf);
    }
    return err ? -1 : 0;
}

int kda_oracle_bwd(int B, int T, int H, int dk, int dv, int dtype,
                   const void* q, const void* k, const void* v,
                   const void* alpha, const void* beta, const double* S0,
                   const double* dO, const double* dST,
                   double* dq, double* dk_out, double* dv_out, double* dalpha, double* dbeta,
                   double* dS0, const int* sel, int n_sel, int nthreads) {
    if (!beta) return -1;
    return bwd_common(B, T, H, dk, dv, dtype, q, k, v, alpha, beta, NULL, NULL, S0, dO, dST, dq, dk_out, dv_out,
                      dalpha, dbeta, NULL, NULL, dS0, sel, n_sel, nthreads, 0);
}

/* Gated DeltaNet-2 backward: the same reverse sweep through gdn2_token (erase gate b per
 * key channel on the read, write gate w per value channel on the write).  erase [B, T, H,
 * dk], write [B, T, H, dv] (dtype); derase [n_sel, T, dk], dwrite [n_sel, T, dv] fp64 out,
 * in place of dbeta.  Other arguments as kda_oracle_bwd. */
int kda_oracle_bwd_gdn2(int B, int T, int H, int dk, int dv, int dtype,
                        const void* q, const void* k, const void* v, const void* alpha,
                        const void* erase, const void* write, const double* S0,
                        const double* dO, const double* dST,
                        double* dq, double* dk_out, double* dv_out, double* dalpha,
                        double* derase, double* dwrite, double* dS0,
                        const int* sel, int n_sel, int nthreads) {
    if (!erase || !write) return -1;
    return bwd_common(B, T, H, dk, dv, dtype, q, k, v, alpha, NULL, erase, write, S0, dO, dST, dq, dk_out, dv_out,
                      dalpha, NULL, derase, dwrite, dS0, sel, n_sel, nthreads, 0);
}

/* SFDA backward: the reverse sweep with the rotation-decay step of kda_oracle_fwd_sfda.
 * lambda [B, T, H, dk] holds the complex gates (real part in channel 2p, imaginary part in
 * channel 2p+1); dlambda [n_sel, T, dk] returns d/dRe in channel 2p and d/dIm in channel
 * 2p+1.  Per token, for coordinate p with S' = Lambda S_prev and dS' = G - k ddelta^T:
 * dRe = sum over columns of (dS'_2p S_prev,2p + dS'_2p+1 S_prev,2p+1), dIm = sum of
 * (dS'_2p+1 S_prev,2p - dS'_2p S_prev,2p+1), and G <- Lambda^T dS'.  dk must be even;
 * other arguments as kda_oracle_bwd. */
int kda_oracle_bwd_sfda(int B, int T, int H, int dk, int dv, int dtype,
                        const void* q, const void* k, const void* v,
                        const void* lambda, const void* beta, const double* S0,
                        const double* dO, const double* dST,
                        double* dq, double* dk_out, double* dv_out, double* dlambda, double* dbeta,
                        double* dS0, const int* sel, int n_sel, int nthreads) {
    if (!beta) return -1;
    return bwd_common(B, T, H, dk, dv, dtype, q, k, v, lambda, beta, NULL, NULL, S0, dO, dST, dq, dk_out, dv_out,
                      dlambda, dbeta, NULL, NULL, dS0, sel, n_sel, nthreads, 1);
}
