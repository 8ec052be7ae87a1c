// kda_chunk.hip -- fused chunkwise-parallel WY forward of the KDA / CKDA recurrence.
//
// Math (per (b, h), chunk of C = 64 positions, start state S [d_k x d_v]):
//   r_ij  = prod_{m=j+1..i} alpha_m           (per key channel; r_ii = 1)
//   T_ij  = beta_i sum_c k_ic k_jc r_ijc      (j < i)       -- strictly lower
//   A_ij  = sum_c q_ic k_jc r_ijc             (j <= i)
//   M     = (I + T)^-1,  U = M diag(beta) V,  W = M diag(beta) (K o gamma)
//   Delta = U - W S
//   O     = (Q o gamma) S + A Delta
//   S    <- diag(gamma_last) S + (K o rho)^T Delta
// with gamma_i = r_{i,-1} and rho_j = r_{C-1,j}.  This is the chunk-WY product
// form on the SFDA page ("El Teorema de Chunk-WY Constructivo": the product of
// a chunk's transitions is a diagonal part minus a correction of rank at most
// C; "Principales Contribuciones" item 3: the chunk acts on its start state as
// S -> P S + B with B from a zero start) and the decay-absorbed WY construction
// with its lower-triangular (I + T)^-1 solve on the Gated DeltaNet-2 page
// (section 3, efficient chunkwise parallel training).
//
// Gate prefix without division.  Every decay factor is a running product of
// gates over a range, kept in fp32: the sign is exact, a zero gate makes every
// product through it exactly zero, and no ratio gamma_i / gamma_j is ever
// formed.  The fp32 value itself is the "sign + log2-magnitude" encoding
// (sign bit, exponent, mantissa); a running product is one full-rate multiply
// per step where an exp/log pair would cost two quarter-rate transcendentals.
// Products are local to 16-row sub-blocks so that every matrix-core operand
// has magnitude <= 1:
//   * off-diagonal 16x16 tiles (I > J): r_ij = F_i * Pi_IJ * Bk_j, with F the
//     prefix product from the start of block I, Bk the suffix product to the
//     end of block J, Pi_IJ the whole blocks in between;
//   * a diagonal tile's pair (i, j) is split at the highest bit where the
//     local indices differ (lam = 8, 4, 2, 1): r_ij = F^lam_i * B^lam_j, the
//     prefix / suffix products inside aligned lam-segments; one matrix-core
//     pass per level, the level picked per element.
//
// (I + T)^-1: the four diagonal 16x16 blocks by forward substitution held in
// registers (one lane per column; the rows of T are broadcast across the
// 16-lane DPP row), the off-diagonal blocks by fp32 matrix-core products in
// three dependency stages, M_IJ = -N_II sum_{K=J}^{I-1} T_IK M_KJ.
//
// Layout of the work: one workgroup per (b, h, value tile of VT columns) with
// VT / 16 waves; wave w owns value columns [16 w, 16 w + 16) of the tile.  A
// head's tiles are placed on one XCD (shared L2 for the re-read q, k, alpha).
// The fp32 state stays in registers for the whole sequence in accumulator
// layout, and an accumulator pair is directly a matrix-core B fragment (the
// k-slot order is permuted to match).  q, k, alpha, beta, v of the next chunk
// are prefetched into registers while the current chunk computes.
#include <stdlib.h>

#include <type_traits>

#include "kda_common.h"
#include "kda_internal.h"
#include "kda_record.h"
#include "kda_tile.h"

namespace kda {

// The rounding residual of Frag::from_acc(a, b) (bf16): the fragment of x - bf16(x) for
// the same eight values, given the rounded fragment h.
template <typename T>
__device__ __forceinline__ void residual_frag(const Frag<T>& h, const f32x4_t& a, const f32x4_t& b, Frag<T>& r) {
  const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    r.w[e] = pack_bf16x2(x[2 * e] - __uint_as_float(h.w[e] << 16), x[2 * e + 1] - __uint_as_float(h.w[e] & 0xFFFF0000u));
}

namespace {

template <typename T, int DK, int VT>
struct Cfg {
  static constexpr int ES = Elem<T>::kBytes;
  static constexpr int NW = VT / 16;
  static constexpr int NT = NW * 64;
  static constexpr int KS = DK / 32;          // k-steps over key channels
  static constexpr int RS_DK = DK * ES + 16;  // [pos][channel] rows (padded)
  static constexpr int RS_C = C * ES + 16;    // [channel][pos] and [pos][pos] rows of T type
  static constexpr int RS_VT = VT * ES + 16;  // [pos][value col]
  static constexpr int RS_F = C * 4 + 16;     // fp32 [pos][pos]
  static constexpr int RS_MB = SUB * 4 + 16;  // fp32 transposed 16x16 blocks
  // region R_IN: q, k, alpha -> later v tile (VV), M (MM, fp32), M~ (MT); O staging over VV
  static constexpr int SZ_IN_A = 3 * C * RS_DK;
  static constexpr int OFF_VV = 0;
  static constexpr int OFF_MM = OFF_VV + C * RS_VT;
  static constexpr int OFF_MT = OFF_MM + C * RS_F;
  static constexpr int SZ_IN_B = OFF_MT + C * RS_C;
  static constexpr int SZ_IN = SZ_IN_A > SZ_IN_B ? SZ_IN_A : SZ_IN_B;
  // region R_OP: Xq16, Xk16, Y16 -> later Q o gamma (QG), (K o gamma)^T (KGT), (K o rho)^T (KRT)
  static constexpr int SZ_OP_A = 3 * C * RS_DK;
  static constexpr int OFF_QG = 0;
  static constexpr int OFF_KGT = OFF_QG + C * RS_DK;
  static constexpr int OFF_KRT = OFF_KGT + DK * RS_C;
  static constexpr int SZ_OP_B = OFF_KRT + DK * RS_C;
  static constexpr int SZ_OP = SZ_OP_A > SZ_OP_B ? SZ_OP_A : SZ_OP_B;
  // region R_L: level operands (2 levels x 4 blocks x (16 A rows + 8 B rows))
  //   -> later D (fp32: T before its beta row scale), A~ (AT), transposed inverse blocks (MB);
  //      W over D once the inverse is done
  static constexpr int LVL_ROWS = 24;
  static constexpr int SZ_L_A = 2 * NB * LVL_ROWS * RS_DK;
  static constexpr int OFF_TT = 0;
  static constexpr int OFF_AT = OFF_TT + C * RS_F;
  static constexpr int OFF_MB = OFF_AT + C * RS_C;
  static constexpr int NMB = 5;  // N00, N11, N22, M10, M20, each stored transposed
  static constexpr int SZ_L_B = OFF_MB + NMB * SUB * RS_MB;
  static constexpr int SZ_L = SZ_L_A > SZ_L_B ? SZ_L_A : SZ_L_B;
  // small fp32 tables
  static constexpr int BASE_IN = 0;
  static constexpr int BASE_OP = BASE_IN + SZ_IN;
  static constexpr int BASE_L = BASE_OP + SZ_OP;
  static constexpr int BASE_GT = BASE_L + SZ_L;         // block totals g[4][DK]
  static constexpr int BASE_GC = BASE_GT + 4 * DK * 4;  // gamma of the last row [DK]
  static constexpr int BASE_BETA = BASE_GC + DK * 4;    // beta [C]
  static constexpr int LDS = BASE_BETA + C * 4;
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(C * RS_DK <= C * RS_F, "W fits over D");
  // prefetch vectors (16 B) per thread
  static constexpr int VROW_K = DK * ES / 16;  // 16-byte vectors per q/k/alpha row
  static constexpr int VROW_V = VT * ES / 16;  // 16-byte vectors per row of the v tile
  static constexpr int VPT = C * VROW_K / NT;
  static constexpr int VPT_V = C * VROW_V / NT;
  static_assert(VPT * NT == C * VROW_K && VPT_V * NT == C * VROW_V, "prefetch split");
  // gate passes: (block, channel pair) items; with enough threads two roles split the work
  static constexpr int NITEM = NB * DK / 2;
  static constexpr bool SPLIT = NT >= 2 * NITEM;
  static_assert(NITEM <= NT, "one gate item per thread");
};

}  // namespace

// PREP = false: the fused single-pass forward (state in registers, outputs written).
// PREP = true : the parallel first pass of the two-pass forward: every workgroup takes a
//               run of `cpw` chunks of one head and writes each chunk's record (-W, Q o gamma,
//               (K o rho)^T, A~, M~, gamma_last) to `ws` for the state pass.
// G2 = true (with PREP): Gated DeltaNet-2 records.  The erase gate b scales the key on
//               the read side only, e = b o k: T_ij = sum_c e_ic k_jc r_ijc and W = M (E o gamma),
//               with no beta (M~ = M); the write side (K o rho, A) keeps k.
template <typename T, int DK, int VT, bool PREP, bool G2 = false>
__global__ __launch_bounds__((VT / 16) * 64) void chunk_fwd_kernel(
    const void* __restrict__ gq, const void* __restrict__ gk, const void* __restrict__ gv,
    const void* __restrict__ galpha, const void* __restrict__ gbeta, const float* s0,
    void* __restrict__ go, float* sT, float* __restrict__ dbg, int Tlen, int H, int DV, int BH,
    char* __restrict__ ws, int cpw, const void* __restrict__ gerase, const int* __restrict__ cu,
    const int* __restrict__ ctab, const int* __restrict__ ctotal, int gmax) {
  static_assert(PREP || !G2, "the Gated DeltaNet-2 gates run on the two-pass path");
  // cu != NULL (PREP only): packed variable-length batch; chunk indices are global
  // (ctab[c] = (sequence, chunk of that sequence)) and records are [H][gmax]
  using K = Cfg<T, DK, VT>;
  using R = Raw<T>;
  constexpr int ES = K::ES;
  constexpr int NT = K::NT;
  constexpr int NW = K::NW;
  constexpr int LDF = K::RS_F / 4;
  extern __shared__ __align__(16) char smem[];
  char* const R_IN = smem + K::BASE_IN;
  char* const R_OP = smem + K::BASE_OP;
  char* const R_L = smem + K::BASE_L;
  float* const GT = (float*)(smem + K::BASE_GT);
  float* const GC = (float*)(smem + K::BASE_GC);
  float* const BETA = (float*)(smem + K::BASE_BETA);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int g = lane >> 4;
  const int n = lane & 15;
  // block -> (head, value tile); a head's tiles land on one XCD when the grid allows it
  const int NVT = PREP ? 1 : DV / VT;
  const int nchunks = cu ? gmax : (Tlen + C - 1) / C;
  int bh, vt, c_begin, c_end;
  {
    const int bid = blockIdx.x;
    if (PREP) {
      const int nseg = (nchunks + cpw - 1) / cpw;
      bh = bid / nseg;
      vt = 0;
      c_begin = (bid % nseg) * cpw;
      c_end = min(cu ? *ctotal : nchunks, c_begin + cpw);
    } else {
      if (NVT > 1 && (BH & 7) == 0) {
        const int r = bid >> 3;
        vt = r % NVT;
        bh = (r / NVT) * 8 + (bid & 7);
      } else {
        bh = bid / NVT;
        vt = bid % NVT;
      }
      c_begin = 0;
      c_end = nchunks;
    }
  }
  const int b = bh / H, h = bh % H;  // varlen: bh = h (b = 0)
  const int v0 = vt * VT;
  auto row_base = [&](int t) -> size_t { return ((size_t)b * Tlen + t) * H + h; };
  // where chunk c lies: token rows sbase + t0 .. of a sequence of len rows, record rec
  struct Geo {
    size_t sbase;
    int len, t0;
    size_t rec;
  };
  auto geo = [&](int c) -> Geo {
    if (cu) {
      const int sq = ctab[2 * c], lc = ctab[2 * c + 1];
      return Geo{(size_t)cu[sq], cu[sq + 1] - cu[sq], lc * C, (size_t)h * gmax + c};
    }
    return Geo{(size_t)b * Tlen, Tlen, c * C, (size_t)bh * nchunks + c};
  };
  auto grow = [&](const Geo& gm, int t) -> size_t { return (gm.sbase + t) * H + h; };

  // ---------------- state tiles: rows 16 r + 4 g + e (key channels), column v0 + 16 wave + n
  f32x4_t S[DK / 16];
#pragma unroll
  for (int r = 0; r < DK / 16; ++r) S[r] = zero4();
  if (!PREP && s0) {
#pragma unroll
    for (int r = 0; r < DK / 16; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[r][e] = s0[((size_t)bh * DK + 16 * r + 4 * g + e) * DV + v0 + 16 * wave + n];
  }

  // ---------------- prefetch registers.  Loads are unconditional (rows past the end
  // are clamped to the last row and replaced when staged) so that no wait is forced
  // at issue time.
  uint4 pq[K::VPT], pk[K::VPT], pa[K::VPT], pv[K::VPT_V];
  uint32_t pb = 0u;  // raw beta bits, converted when staged
  // (G2) erase gate of this thread's gate item (16 rows x 2 channels), one chunk ahead
  typename Raw<T>::type pe[G2 ? SUB : 1], er_raw[G2 ? SUB : 1];
  const int item_g = K::SPLIT ? tid % K::NITEM : tid;
  const bool item_ok = K::SPLIT ? (tid < 2 * K::NITEM) : (tid < K::NITEM);
  auto issue_qka = [&](int c) {
    const Geo gn = geo(c);
    const int t0 = gn.t0;
#pragma unroll
    for (int i = 0; i < K::VPT; ++i) {
      const int j = tid + NT * i;
      const int row = j / K::VROW_K, c16 = j % K::VROW_K;
      const size_t off = grow(gn, min(t0 + row, gn.len - 1)) * DK * ES + (size_t)c16 * 16;
      pq[i] = *(const uint4*)((const char*)gq + off);
      pk[i] = *(const uint4*)((const char*)gk + off);
      pa[i] = *(const uint4*)((const char*)galpha + off);
    }
    if constexpr (!G2) {
      const size_t ib = grow(gn, min(t0 + (tid & (C - 1)), gn.len - 1));
      pb = ES == 2 ? (uint32_t)((const uint16_t*)gbeta)[ib] : ((const uint32_t*)gbeta)[ib];
    } else if (item_ok) {
      const int bI = item_g / (DK / 2), cp = item_g % (DK / 2);
#pragma unroll
      for (int m = 0; m < SUB; ++m)
        pe[m] = R::ld((const char*)gerase + grow(gn, min(t0 + SUB * bI + m, gn.len - 1)) * DK * ES + 2 * cp * ES);
    }
  };
  auto issue_v = [&](int c) {
    const int t0 = c * C;
#pragma unroll
    for (int i = 0; i < K::VPT_V; ++i) {
      const int j = tid + NT * i;
      const int row = j / K::VROW_V, c16 = j % K::VROW_V;
      pv[i] = *(const uint4*)((const char*)gv + row_base(min(t0 + row, Tlen - 1)) * DV * ES + (size_t)v0 * ES +
                              (size_t)c16 * 16);
    }
  };
  if (c_begin < c_end) {
    issue_qka(c_begin);
    if (!PREP) issue_v(c_begin);
  }

  // gate-pass item: (block iI, channels 2 icp, 2 icp + 1); roles 0 / 1 split the passes
  const int item = K::SPLIT ? tid % K::NITEM : tid;
  const int role = K::SPLIT ? tid / K::NITEM : 2;  // 2: this thread takes both roles
  const bool has_item = K::SPLIT ? (tid < 2 * K::NITEM) : (tid < K::NITEM);
  const bool r0 = has_item && role != 1;
  const bool r1 = has_item && role != 0;
  const int iI = item / (DK / 2);
  const int icp = item % (DK / 2);
  const int item_off = (SUB * iI) * K::RS_DK + 2 * icp * ES;

  for (int chunk = c_begin; chunk < c_end; ++chunk) {
    const Geo gm = geo(chunk);
    const int t0 = gm.t0;
    const int nv = min(C, gm.len - t0);
    // ================= phase 0: staged inputs -> LDS (padded rows: q = k = 0, alpha = 1, beta = 0)
    __syncthreads();
#pragma unroll
    for (int i = 0; i < K::VPT; ++i) {
      const int j = tid + NT * i;
      const int row = j / K::VROW_K, c16 = j % K::VROW_K;
      const bool ok = t0 + row < gm.len;
      const uint32_t one = R::kOneWord;
      const int off = row * K::RS_DK + c16 * 16;
      *(uint4*)(R_IN + 0 * C * K::RS_DK + off) = ok ? pq[i] : make_uint4(0, 0, 0, 0);
      *(uint4*)(R_IN + 1 * C * K::RS_DK + off) = ok ? pk[i] : make_uint4(0, 0, 0, 0);
      *(uint4*)(R_IN + 2 * C * K::RS_DK + off) = ok ? pa[i] : make_uint4(one, one, one, one);
    }
    if (tid < C) BETA[tid] = (t0 + tid < gm.len) ? (G2 ? 1.f : __uint_as_float(ES == 2 ? pb << 16 : pb)) : 0.f;
    if constexpr (G2) {
#pragma unroll
      for (int m = 0; m < SUB; ++m) er_raw[m] = pe[m];
    }
    __syncthreads();
    if (chunk + 1 < c_end) issue_qka(chunk + 1);

    const char* const Qs = R_IN;
    const char* const Ks = R_IN + C * K::RS_DK;
    const char* const As = R_IN + 2 * C * K::RS_DK;

    // item registers: alpha (fp32), q and k (packed), loaded in one batch per phase
    typename R::type qr[SUB], kr_raw[SUB];
    float al[SUB][2];
    // the key as the erase side reads it: k (KDA), b o k (Gated DeltaNet-2)
    auto read_key = [&](int m, float& e0, float& e1) {
      R::unpack(kr_raw[m], e0, e1);
      if constexpr (G2) {
        float b0, b1;
        R::unpack(er_raw[m], b0, b1);
        e0 *= b0;
        e1 *= b1;
      }
    };
    auto ld_item = [&](bool with_qk) {
#pragma unroll
      for (int m = 0; m < SUB; ++m) {
        R::unpack(R::ld(As + item_off + m * K::RS_DK), al[m][0], al[m][1]);
        if (with_qk) {
          qr[m] = R::ld(Qs + item_off + m * K::RS_DK);
          kr_raw[m] = R::ld(Ks + item_off + m * K::RS_DK);
        }
      }
    };

    // level operand writer: slot ls (0/1), level lam, for the item's block
    auto write_levels = [&](int ls, int lam) {
      char* LA = R_L + (size_t)(ls * NB + iI) * K::LVL_ROWS * K::RS_DK + 2 * icp * ES;
      char* LB = LA + 16 * K::RS_DK;
      float f0 = 1.f, f1 = 1.f;
#pragma unroll
      for (int m = 0; m < SUB; ++m) {
        if (m & lam) {
          if ((m & (lam - 1)) == 0) {
            f0 = al[m][0];
            f1 = al[m][1];
          } else {
            f0 *= al[m][0];
            f1 *= al[m][1];
          }
          const int u = (m / (2 * lam)) * lam + (m & (lam - 1));
          float q0, q1, k0, k1;
          R::unpack(qr[m], q0, q1);
          read_key(m, k0, k1);
          R::st(LA + u * K::RS_DK, q0 * f0, q1 * f1);
          R::st(LA + (8 + u) * K::RS_DK, k0 * f0, k1 * f1);
        }
      }
      float b0 = 1.f, b1 = 1.f;
#pragma unroll
      for (int m = SUB - 1; m >= 0; --m) {
        if (!(m & lam)) {
          if ((m & (lam - 1)) == lam - 1) {
            b0 = 1.f;
            b1 = 1.f;
          } else {
            b0 *= al[m + 1][0];
            b1 *= al[m + 1][1];
          }
          const int v = (m / (2 * lam)) * lam + (m & (lam - 1));
          float k0, k1;
          R::unpack(kr_raw[m], k0, k1);
          R::st(LB + v * K::RS_DK, k0 * b0, k1 * b1);
        }
      }
    };

    // ================= phase B: 16-block anchored operands (role 0) + level 8 / 4 operands (role 1)
    if (has_item) {
      ld_item(true);
      if (r0) {
        char* Xq = R_OP + item_off;
        char* Xk = R_OP + C * K::RS_DK + item_off;
        char* Y = R_OP + 2 * C * K::RS_DK + item_off;
        float f0 = 1.f, f1 = 1.f;
#pragma unroll
        for (int m = 0; m < SUB; ++m) {
          f0 *= al[m][0];
          f1 *= al[m][1];
          float q0, q1, k0, k1;
          R::unpack(qr[m], q0, q1);
          read_key(m, k0, k1);
          R::st(Xq + m * K::RS_DK, q0 * f0, q1 * f1);
          R::st(Xk + m * K::RS_DK, k0 * f0, k1 * f1);
        }
        *(float2*)(GT + iI * DK + 2 * icp) = make_float2(f0, f1);  // the block's gate total
        float b0 = 1.f, b1 = 1.f;
#pragma unroll
        for (int m = SUB - 1; m >= 0; --m) {
          float k0, k1;
          R::unpack(kr_raw[m], k0, k1);
          R::st(Y + m * K::RS_DK, k0 * b0, k1 * b1);
          b0 *= al[m][0];
          b1 *= al[m][1];
        }
      }
      if (r1) {
        write_levels(0, 8);
        write_levels(1, 4);
      }
    }
    __syncthreads();

    // ================= phase M1: off-diagonal tiles and level 8 / 4 passes
    constexpr int NJ1 = 14;
    constexpr int MJ1 = (NJ1 + NW - 1) / NW;
    f32x4_t r1a[MJ1], r1t[MJ1];
#pragma unroll
    for (int s = 0; s < MJ1; ++s) {
      const int j = wave + s * NW;
      r1a[s] = zero4();
      r1t[s] = zero4();
      if (j < 6) {
        const int I = kOffI[j], J = kOffJ[j], pi = kOffPi[j];
        const char* Xq = R_OP + (16 * I + n) * K::RS_DK;
        const char* Xk = R_OP + C * K::RS_DK + (16 * I + n) * K::RS_DK;
        const char* Y = R_OP + 2 * C * K::RS_DK + (16 * J + n) * K::RS_DK;
        Frag<T> fa[K::KS], fk[K::KS], fb[K::KS];
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) {
          const int c0 = 32 * ks + 8 * g;
          fb[ks].load8(Y + c0 * ES);
          fa[ks].load8(Xq + c0 * ES);
          fk[ks].load8(Xk + c0 * ES);
        }
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) {
          if (pi >= 0) {
            // whole blocks between J and I: g1 (pi 0), g1 g2 (pi 1), g2 (pi 2)
            const int c0 = 32 * ks + 8 * g;
            const float* G1 = GT + (pi == 2 ? 2 : 1) * DK + c0;
            float4 p0 = *(const float4*)G1, p1 = *(const float4*)(G1 + 4);
            if (pi == 1) {
              const float4 e0 = *(const float4*)(GT + 2 * DK + c0), e1 = *(const float4*)(GT + 2 * DK + c0 + 4);
              p0 = make_float4(p0.x * e0.x, p0.y * e0.y, p0.z * e0.z, p0.w * e0.w);
              p1 = make_float4(p1.x * e1.x, p1.y * e1.y, p1.z * e1.z, p1.w * e1.w);
            }
            const float pv8[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
            fb[ks].scale(pv8);
          }
          mma(r1a[s], fa[ks], fb[ks]);
          mma(r1t[s], fk[ks], fb[ks]);
        }
      } else if (j < NJ1) {
        const int ls = (j - 6) / NB, I = (j - 6) % NB;
        const char* LA = R_L + (size_t)(ls * NB + I) * K::LVL_ROWS * K::RS_DK;
        const char* LB = LA + 16 * K::RS_DK;
        Frag<T> fa[K::KS], fb[K::KS];
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) {
          const int c0 = 32 * ks + 8 * g;
          fa[ks].load8(LA + n * K::RS_DK + c0 * ES);
          if (n < 8)
            fb[ks].load8(LB + n * K::RS_DK + c0 * ES);
          else
            fb[ks].zero();
        }
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) mma(r1a[s], fa[ks], fb[ks]);
      }
    }
    __syncthreads();

    // ================= phase C: gamma / rho operands (role 0) + level 2 / 1 operands (role 1)
    if (has_item) {
      ld_item(true);
      if (r0) {
        const float2 t0v = *(const float2*)(GT + 2 * icp), t1v = *(const float2*)(GT + DK + 2 * icp);
        const float2 t2v = *(const float2*)(GT + 2 * DK + 2 * icp), t3v = *(const float2*)(GT + 3 * DK + 2 * icp);
        float Gp[2], Rp[2];
        Gp[0] = iI == 0 ? 1.f : iI == 1 ? t0v.x : iI == 2 ? t0v.x * t1v.x : t0v.x * t1v.x * t2v.x;
        Gp[1] = iI == 0 ? 1.f : iI == 1 ? t0v.y : iI == 2 ? t0v.y * t1v.y : t0v.y * t1v.y * t2v.y;
        Rp[0] = iI == 3 ? 1.f : iI == 2 ? t3v.x : iI == 1 ? t2v.x * t3v.x : t1v.x * t2v.x * t3v.x;
        Rp[1] = iI == 3 ? 1.f : iI == 2 ? t3v.y : iI == 1 ? t2v.y * t3v.y : t1v.y * t2v.y * t3v.y;
        if (iI == 3) *(float2*)(GC + 2 * icp) = make_float2(Gp[0] * t3v.x, Gp[1] * t3v.y);  // gamma_last
        char* QG = R_OP + K::OFF_QG + item_off;
        // (K o gamma)^T and (K o rho)^T rows of the item's two channels, positions 16 iI ..
        // 16 iI + 15: written as 8-position row segments
        char* pg0 = R_OP + K::OFF_KGT + (2 * icp) * K::RS_C + (SUB * iI) * ES;
        char* pr0 = R_OP + K::OFF_KRT + (2 * icp) * K::RS_C + (SUB * iI) * ES;
        float f0 = Gp[0], f1 = Gp[1];
#pragma unroll
        for (int h8 = 0; h8 < SUB; h8 += 8) {
          float g8a[8], g8b[8];
#pragma unroll
          for (int mm = 0; mm < 8; ++mm) {
            const int m = h8 + mm;
            f0 *= al[m][0];
            f1 *= al[m][1];
            float q0, q1, k0, k1;
            R::unpack(qr[m], q0, q1);
            read_key(m, k0, k1);
            R::st(QG + m * K::RS_DK, q0 * f0, q1 * f1);
            g8a[mm] = k0 * f0;
            g8b[mm] = k1 * f1;
          }
          st_row8<T>(pg0 + h8 * ES, g8a);
          st_row8<T>(pg0 + K::RS_C + h8 * ES, g8b);
        }
        float b0 = Rp[0], b1 = Rp[1];
#pragma unroll
        for (int h8 = SUB - 8; h8 >= 0; h8 -= 8) {
          float r8a[8], r8b[8];
#pragma unroll
          for (int mm = 7; mm >= 0; --mm) {
            const int m = h8 + mm;
            float k0, k1;
            R::unpack(kr_raw[m], k0, k1);
            r8a[mm] = k0 * b0;
            r8b[mm] = k1 * b1;
            b0 *= al[m][0];
            b1 *= al[m][1];
          }
          st_row8<T>(pr0 + h8 * ES, r8a);
          st_row8<T>(pr0 + K::RS_C + h8 * ES, r8b);
        }
      }
      if (r1) {
        write_levels(0, 2);
        write_levels(1, 1);
      }
    }
    __syncthreads();

    // ================= phase M2: level 2 / 1 passes + level 0 (diagonal of A)
    constexpr int NJ2 = 12;
    constexpr int MJ2 = (NJ2 + NW - 1) / NW;
    f32x4_t r2[MJ2];
#pragma unroll
    for (int s = 0; s < MJ2; ++s) {
      const int j = wave + s * NW;
      r2[s] = zero4();
      if (j < NJ2) {
        const char* pa_;
        const char* pb_;
        bool use_b = true;
        if (j < 8) {
          const int ls = j / NB, I = j % NB;
          pa_ = R_L + (size_t)(ls * NB + I) * K::LVL_ROWS * K::RS_DK + n * K::RS_DK;
          pb_ = R_L + (size_t)(ls * NB + I) * K::LVL_ROWS * K::RS_DK + (16 + n) * K::RS_DK;
          use_b = n < 8;
        } else {
          const int I = j - 8;
          pa_ = Qs + (16 * I + n) * K::RS_DK;
          pb_ = Ks + (16 * I + n) * K::RS_DK;
        }
        Frag<T> fa[K::KS], fb[K::KS];
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) {
          const int c0 = 32 * ks + 8 * g;
          fa[ks].load8(pa_ + c0 * ES);
          if (use_b)
            fb[ks].load8(pb_ + c0 * ES);
          else
            fb[ks].zero();
        }
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) mma(r2[s], fa[ks], fb[ks]);
      }
    }
    __syncthreads();

    // ================= phase D: scatter D (fp32, T before its beta row scale) and A~
    float* TT = (float*)(R_L + K::OFF_TT);
    char* AT = R_L + K::OFF_AT;
    // level results: D[u][v] holds the A entry (u < 8) or D entry (u >= 8) of upper row
    // rank u & 7 and lower row rank v, valid when both lie in one 2 lam block
    auto put_level_t = [&](auto lam_c, const f32x4_t& acc, int I) {
      constexpr int lam = decltype(lam_c)::value;
      if (n < 8) {
        const int v = n;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 4 * g + e;
          const int u = row & 7;
          if ((u / lam) == (v / lam)) {
            const int mu = (u / lam) * 2 * lam + lam + (u % lam);
            const int ml = (v / lam) * 2 * lam + (v % lam);
            const int gi = 16 * I + mu, gj = 16 * I + ml;
            if (row < 8)
              st_elem(AT + gi * K::RS_C + gj * ES, acc[e], ES);
            else
              TT[gi * LDF + gj] = acc[e];
          }
        }
      }
    };
    auto put_level = [&](const f32x4_t& acc, int lam, int I) {
      if (lam == 8)
        put_level_t(std::integral_constant<int, 8>(), acc, I);
      else if (lam == 4)
        put_level_t(std::integral_constant<int, 4>(), acc, I);
      else if (lam == 2)
        put_level_t(std::integral_constant<int, 2>(), acc, I);
      else
        put_level_t(std::integral_constant<int, 1>(), acc, I);
    };
#pragma unroll
    for (int s = 0; s < MJ1; ++s) {
      const int j = wave + s * NW;
      if (j < 6) {
        const int I = kOffI[j], J = kOffJ[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int gi = 16 * I + 4 * g + e, gj = 16 * J + n;
          st_elem(AT + gi * K::RS_C + gj * ES, r1a[s][e], ES);
          TT[gi * LDF + gj] = r1t[s][e];
        }
      } else if (j < NJ1) {
        const int ls = (j - 6) / NB, I = (j - 6) % NB;
        put_level(r1a[s], ls == 0 ? 8 : 4, I);
      }
    }
#pragma unroll
    for (int s = 0; s < MJ2; ++s) {
      const int j = wave + s * NW;
      if (j < 8) {
        const int ls = j / NB, I = j % NB;
        put_level(r2[s], ls == 0 ? 2 : 1, I);
      } else if (j < NJ2) {
        const int I = j - 8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 4 * g + e;
          if (row <= n) st_elem(AT + (16 * I + row) * K::RS_C + (16 * I + n) * ES, row == n ? r2[s][e] : 0.f, ES);
        }
      }
    }
    for (int x = tid; x < 6 * 16 * 2; x += NT) {  // 6 tiles x 16 rows x 2 segments of 8
      const int t = x >> 5, i = (x >> 1) & 15, j0 = 8 * (x & 1);
      const float z8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      st_row8<T>(AT + (16 * kUpI[t] + i) * K::RS_C + (16 * kUpJ[t] + j0) * ES, z8);
    }
    // v tile of this chunk -> LDS, then prefetch the next chunk's
    if (!PREP) {
#pragma unroll
      for (int i = 0; i < K::VPT_V; ++i) {
        const int j = tid + NT * i;
        const int row = j / K::VROW_V, c16 = j % K::VROW_V;
        *(uint4*)(R_IN + K::OFF_VV + row * K::RS_VT + c16 * 16) =
            (t0 + row < Tlen) ? pv[i] : make_uint4(0, 0, 0, 0);
      }
      if (chunk + 1 < c_end) issue_v(chunk + 1);
    }
    __syncthreads();

    if (!PREP && dbg && vt == 0) {
      float* Dp = dbg + ((size_t)bh * nchunks + chunk) * 4 * C * C;
      for (int x = tid; x < C * C; x += NT) {
        const int i = x / C, j = x % C;
        Dp[x] = j < i ? BETA[i] * TT[i * LDF + j] : 0.f;
        Dp[C * C + x] = j <= i ? Elem<T>::load(AT + i * K::RS_C, j) : 0.f;
      }
    }

    // O = (Q o gamma) S does not depend on the inverse: waves 1.. do it while wave 0
    // runs the diagonal-block substitution, wave 0 in the second off-diagonal stage.
    f32x4_t Ot[NB];
    auto q_times_S = [&]() {
      Frag<T> bs[K::KS];
#pragma unroll
      for (int ks = 0; ks < K::KS; ++ks) bs[ks].from_acc(S[2 * ks], S[2 * ks + 1]);
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        Ot[I] = zero4();
        const char* qrow = R_OP + K::OFF_QG + (16 * I + n) * K::RS_DK;
        Frag<T> fq[K::KS];
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) {
          const int c0 = 32 * ks + 4 * g;
          fq[ks].load4x2(qrow + c0 * ES, qrow + (c0 + 16) * ES);
        }
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) mma(Ot[I], fq[ks], bs[ks]);
      }
    };
    if (!PREP && wave != 0) q_times_S();

    // ================= phase I: M = (I + T)^-1 with T = diag(beta) D
    float* MM = (float*)(R_IN + K::OFF_MM);
    char* MB = R_L + K::OFF_MB;  // transposed 16x16 blocks: 0 N00, 1 N11, 2 N22, 3 M10, 4 M20
    auto mb_row = [&](int blk, int r) -> float* { return (float*)(MB + (blk * SUB + r) * K::RS_MB); };
    if (wave == 0) {
      // diagonal blocks: lane = (block I, column col); it also holds row `col` of T_II
      const int I = lane >> 4, col = lane & 15;
      const float* drow = TT + (16 * I + col) * LDF + 16 * I;
      const float bcol = BETA[16 * I + col];
      float tr[SUB];
#pragma unroll
      for (int p4 = 0; p4 < SUB; p4 += 4) {
        const float4 w4 = *(const float4*)(drow + p4);
        tr[p4] = w4.x;
        tr[p4 + 1] = w4.y;
        tr[p4 + 2] = w4.z;
        tr[p4 + 3] = w4.w;
      }
#pragma unroll
      for (int p = 0; p < SUB; ++p) tr[p] = p < col ? bcol * tr[p] : 0.f;
      float x[SUB], nx[SUB];  // column of N_II and its negation (accumulated with fmac)
#define KDA_FS_ROW(i)                                                                        \
  {                                                                                          \
    float acc = (col == i) ? 1.f : 0.f;                                                      \
    _Pragma("unroll") for (int p = 0; p < i; ++p) acc = fmaf(row_bcast<i>(tr[p]), nx[p], acc); \
    x[i] = acc;                                                                              \
    nx[i] = -acc;                                                                            \
  }
      KDA_FS_ROW(0) KDA_FS_ROW(1) KDA_FS_ROW(2) KDA_FS_ROW(3) KDA_FS_ROW(4) KDA_FS_ROW(5) KDA_FS_ROW(6)
      KDA_FS_ROW(7) KDA_FS_ROW(8) KDA_FS_ROW(9) KDA_FS_ROW(10) KDA_FS_ROW(11) KDA_FS_ROW(12) KDA_FS_ROW(13)
      KDA_FS_ROW(14) KDA_FS_ROW(15)
#undef KDA_FS_ROW
#pragma unroll
      for (int i = 0; i < SUB; ++i) MM[(16 * I + i) * LDF + 16 * I + col] = x[i];
      if (I < 3) {
        float* dst = mb_row(I, col);
#pragma unroll
        for (int p4 = 0; p4 < SUB; p4 += 4) *(float4*)(dst + p4) = make_float4(x[p4], x[p4 + 1], x[p4 + 2], x[p4 + 3]);
      }
    }
    __syncthreads();
    // off-diagonal blocks.  In product instruction s the k-slot is 4 g + s, so an
    // accumulator tile is directly the B operand of the next product.
    auto a_T = [&](int I, int Kb, float (&a)[4]) {  // row n of T_IK = beta_i D_IK
      const float4 w4 = *(const float4*)(TT + (16 * I + n) * LDF + 16 * Kb + 4 * g);
      const float bi = BETA[16 * I + n];
      a[0] = bi * w4.x;
      a[1] = bi * w4.y;
      a[2] = bi * w4.z;
      a[3] = bi * w4.w;
    };
    auto b_MB = [&](int blk, float (&bb)[4]) {  // B = a block whose transpose is stored in MB
      const float4 w4 = *(const float4*)(mb_row(blk, n) + 4 * g);
      bb[0] = w4.x;
      bb[1] = w4.y;
      bb[2] = w4.z;
      bb[3] = w4.w;
    };
    auto mm4_acc = [&](f32x4_t& acc, const float (&a)[4], const f32x4_t& bacc) {
      const float bb[4] = {bacc[0], bacc[1], bacc[2], bacc[3]};
      mm4(acc, a, bb);
    };
    auto neg_N_times = [&](int I, const f32x4_t& z) -> f32x4_t {  // -N_II z
      const float4 w4 = *(const float4*)(MM + (16 * I + n) * LDF + 16 * I + 4 * g);
      const float a[4] = {w4.x, w4.y, w4.z, w4.w};
      f32x4_t r = zero4();
      mm4_acc(r, a, z);
      return -r;
    };
    auto put_M = [&](int I, int J, const f32x4_t& m, int blk) {
#pragma unroll
      for (int e = 0; e < 4; ++e) MM[(16 * I + 4 * g + e) * LDF + 16 * J + n] = m[e];
      if (blk >= 0) *(float4*)(mb_row(blk, n) + 4 * g) = make_float4(m[0], m[1], m[2], m[3]);
    };
    f32x4_t keep = zero4();  // partial sum carried across the stages (waves 0 and 3)
    {
      float a[4], bb[4];
      if (wave == 0) {  // M10, then P30 = T30 N00 + T31 M10
        f32x4_t z = zero4();
        a_T(1, 0, a);
        b_MB(0, bb);
        mm4(z, a, bb);
        const f32x4_t m10 = neg_N_times(1, z);
        put_M(1, 0, m10, 3);
        a_T(3, 0, a);
        b_MB(0, bb);
        mm4(keep, a, bb);
        a_T(3, 1, a);
        mm4_acc(keep, a, m10);
      } else if (wave == 1) {  // M21, then M31 = -N33 (T31 N11 + T32 M21)
        f32x4_t z = zero4();
        a_T(2, 1, a);
        b_MB(1, bb);
        mm4(z, a, bb);
        const f32x4_t m21 = neg_N_times(2, z);
        put_M(2, 1, m21, -1);
        f32x4_t p = zero4();
        a_T(3, 1, a);
        b_MB(1, bb);
        mm4(p, a, bb);
        a_T(3, 2, a);
        mm4_acc(p, a, m21);
        put_M(3, 1, neg_N_times(3, p), -1);
      } else if (wave == 2) {  // M32
        f32x4_t z = zero4();
        a_T(3, 2, a);
        b_MB(2, bb);
        mm4(z, a, bb);
        put_M(3, 2, neg_N_times(3, z), -1);
      } else if (wave == 3) {  // P20 = T20 N00
        a_T(2, 0, a);
        b_MB(0, bb);
        mm4(keep, a, bb);
      }
    }
    __syncthreads();
    if (!PREP && wave == 0) q_times_S();  // wave 0's share, in the stage where it is otherwise idle
    if (wave == 3) {  // M20 = -N22 (P20 + T21 M10)
      float a[4], bb[4];
      a_T(2, 1, a);
      b_MB(3, bb);
      mm4(keep, a, bb);
      put_M(2, 0, neg_N_times(2, keep), 4);
    }
    __syncthreads();
    if (wave == 0) {  // M30 = -N33 (P30 + T32 M20)
      float a[4], bb[4];
      a_T(3, 2, a);
      b_MB(4, bb);
      mm4(keep, a, bb);
      put_M(3, 0, neg_N_times(3, keep), -1);
    }
    __syncthreads();
    // M~ = M diag(beta), lower incl. diagonal, as matrix-core operand (8 columns per step)
    char* MT = R_IN + K::OFF_MT;
#pragma unroll
    for (int x = tid; x < C * C / 8; x += NT) {
      const int i = x / (C / 8), j0 = 8 * (x % (C / 8));
      const float4 m0 = *(const float4*)(MM + i * LDF + j0), m1 = *(const float4*)(MM + i * LDF + j0 + 4);
      const float4 b0 = *(const float4*)(BETA + j0), b1 = *(const float4*)(BETA + j0 + 4);
      float v8[8] = {m0.x * b0.x, m0.y * b0.y, m0.z * b0.z, m0.w * b0.w,
                     m1.x * b1.x, m1.y * b1.y, m1.z * b1.z, m1.w * b1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (j0 + e > i) v8[e] = 0.f;
      st_row8<T>(MT + i * K::RS_C + j0 * ES, v8);
    }
    if (!PREP && dbg && vt == 0) {
      float* Dp = dbg + ((size_t)bh * nchunks + chunk) * 4 * C * C + 2 * C * C;
      for (int x = tid; x < C * C; x += NT) {
        const int i = x / C, j = x % C;
        Dp[x] = j <= i ? MM[i * LDF + j] : 0.f;
      }
    }
    __syncthreads();

    // ================= phase W: W = M~ (K o gamma) -> -W in LDS;  U_w = M~ V[:, w] in registers
    char* WW = R_L + K::OFF_TT;
    f32x4_t Dl[NB];
    {
      Frag<T> am[NB][2];
#pragma unroll
      for (int I = 0; I < NB; ++I)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (ks == 0 || I >= 2)
            am[I][ks].load8(MT + (16 * I + n) * K::RS_C + (32 * ks + 8 * g) * ES);
          else
            am[I][ks].zero();
        }
      constexpr int NCT = DK / 16;
      for (int cn = wave; cn < NCT; cn += NW) {
        Frag<T> bk[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          bk[ks].load8(R_OP + K::OFF_KGT + (16 * cn + n) * K::RS_C + (32 * ks + 8 * g) * ES);
#pragma unroll
        for (int I = 0; I < NB; ++I) {
          f32x4_t acc = zero4();
          mma(acc, am[I][0], bk[0]);
          if (I >= 2) mma(acc, am[I][1], bk[1]);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            st_elem(WW + (16 * I + 4 * g + e) * K::RS_DK + (16 * cn + n) * ES, -acc[e], ES);
          if (!PREP && dbg && vt == 0 && cn < 4) {
            float* Dp = dbg + ((size_t)bh * nchunks + chunk) * 4 * C * C + 3 * C * C;
#pragma unroll
            for (int e = 0; e < 4; ++e) Dp[(16 * I + 4 * g + e) * C + 16 * cn + n] = acc[e];
          }
        }
      }
      if constexpr (!PREP) {
        // U for this wave's value columns
        Frag<T> bv[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          bv[ks].load_col8(R_IN + K::OFF_VV + (32 * ks + 8 * g) * K::RS_VT + (16 * wave + n) * ES, K::RS_VT);
#pragma unroll
        for (int I = 0; I < NB; ++I) {
          Dl[I] = zero4();
          mma(Dl[I], am[I][0], bv[0]);
          if (I >= 2) mma(Dl[I], am[I][1], bv[1]);
        }
      }
    }
    __syncthreads();
    if constexpr (PREP) {
      // the chunk's record for the state pass: -W, Q o gamma, (K o rho)^T, A~, M~, gamma_last
      // (the LDS tiles are copied whole, padded rows and all: the record is their image)
      using RL = RecordLayout<T, DK>;
      static_assert(RL::RS_DK == K::RS_DK && RL::RS_C == K::RS_C, "record rows match the LDS tiles");
      char* rec = ws + gm.rec * RL::BYTES;
      copy_flat<NT>(rec + RL::WW, WW, RL::QG - RL::WW, tid);
      copy_flat<NT>(rec + RL::QG, R_OP + K::OFF_QG, RL::KRT - RL::QG, tid);
      copy_flat<NT>(rec + RL::KRT, R_OP + K::OFF_KRT, RL::AT - RL::KRT, tid);
      copy_flat<NT>(rec + RL::AT, AT, RL::MT - RL::AT, tid);
      copy_flat<NT>(rec + RL::MT, MT, RL::GC - RL::MT, tid);
      copy_flat<NT>(rec + RL::GC, (const char*)GC, RL::IMG - RL::GC, tid);
      continue;
    }

    // ================= phase S: Delta = U - W S ; O = (Q o gamma) S + A Delta ; S update
    // (bf16: S in W S and Delta in the state update enter as a bf16 pair, value and
    // rounding residual, so that their roundings do not accumulate along the chain where the
    // transitions are orthogonal; the readout A Delta takes the single bf16 value)
    {
      constexpr bool kPair = std::is_same<T, bf16_t>::value;
      Frag<T> bs[K::KS], bsl[K::KS];
#pragma unroll
      for (int ks = 0; ks < K::KS; ++ks) {
        bs[ks].from_acc(S[2 * ks], S[2 * ks + 1]);
        if constexpr (kPair) residual_frag(bs[ks], S[2 * ks], S[2 * ks + 1], bsl[ks]);
      }
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        const char* wrow = WW + (16 * I + n) * K::RS_DK;
        Frag<T> fw[K::KS];
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) {
          const int c0 = 32 * ks + 4 * g;
          fw[ks].load4x2(wrow + c0 * ES, wrow + (c0 + 16) * ES);
        }
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) {
          mma(Dl[I], fw[ks], bs[ks]);
          if constexpr (kPair) mma(Dl[I], fw[ks], bsl[ks]);
        }
      }
      Frag<T> bd[2], bdl[2];
      bd[0].from_acc(Dl[0], Dl[1]);
      bd[1].from_acc(Dl[2], Dl[3]);
      if constexpr (kPair) {
        residual_frag(bd[0], Dl[0], Dl[1], bdl[0]);
        residual_frag(bd[1], Dl[2], Dl[3], bdl[1]);
      }
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        const char* arow = AT + (16 * I + n) * K::RS_C;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          if (s2 == 0 || I >= 2) {
            const int p0 = 32 * s2 + 4 * g;
            Frag<T> fa;
            fa.load4x2(arow + p0 * ES, arow + (p0 + 16) * ES);
            mma(Ot[I], fa, bd[s2]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < DK / 16; ++r) {
        const float4 gc = *(const float4*)(GC + 16 * r + 4 * g);
        S[r][0] *= gc.x;
        S[r][1] *= gc.y;
        S[r][2] *= gc.z;
        S[r][3] *= gc.w;
        const char* krow = R_OP + K::OFF_KRT + (16 * r + n) * K::RS_C;
        Frag<T> fa[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int p0 = 32 * s2 + 4 * g;
          fa[s2].load4x2(krow + p0 * ES, krow + (p0 + 16) * ES);
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          mma(S[r], fa[s2], bd[s2]);
          if constexpr (kPair) mma(S[r], fa[s2], bdl[s2]);
        }
      }
      // stage O (over the consumed v tile)
#pragma unroll
      for (int I = 0; I < NB; ++I)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          st_elem(R_IN + K::OFF_VV + (16 * I + 4 * g + e) * K::RS_VT + (16 * wave + n) * ES, Ot[I][e], ES);
    }
    __syncthreads();
    // ================= phase O: coalesced store of the chunk's outputs
    for (int j = tid; j < C * K::VROW_V; j += NT) {
      const int row = j / K::VROW_V, c16 = j % K::VROW_V;
      if (row < nv)
        *(uint4*)((char*)go + row_base(t0 + row) * DV * ES + (size_t)v0 * ES + (size_t)c16 * 16) =
            *(const uint4*)(R_IN + K::OFF_VV + row * K::RS_VT + c16 * 16);
    }
  }

  if (!PREP && sT) {
#pragma unroll
    for (int r = 0; r < DK / 16; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sT[((size_t)bh * DK + 16 * r + 4 * g + e) * DV + v0 + 16 * wave + n] = S[r][e];
  }
}

template <typename T, int DK, int VT>
static hipError_t launch_chunk_t(const ChunkArgs& a) {
  using K = Cfg<T, DK, VT>;
  auto kern = chunk_fwd_kernel<T, DK, VT, false>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, K::LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int BH = a.B * a.H;
  hipLaunchKernelGGL(kern, dim3(BH * (a.dv / VT)), dim3(K::NT), K::LDS, (hipStream_t)a.stream, a.q, a.k, a.v,
                     a.alpha, a.beta, a.s0, a.o, a.sT, a.dbg, a.T, a.H, a.dv, BH, (char*)nullptr, 0,
                     (const void*)nullptr, (const int*)nullptr, (const int*)nullptr, (const int*)nullptr, 0);
  return hipGetLastError();
}

// Value-tile width: narrow tiles (more workgroups; the gate work is repeated per
// tile) when the (b, h) count alone cannot fill the chip's 256 compute units.
static int pick_vt(const ChunkArgs& a) {
  if (a.vt_override == 64 || a.vt_override == 128) return a.vt_override <= a.dv ? a.vt_override : a.dv;
  if (a.dv == 64) return 64;
  return (long)a.B * a.H >= 256 ? 128 : 64;
}

hipError_t launch_chunk(const ChunkArgs& a) {
  if (a.B * a.H == 0) return hipSuccess;
  const int vt = pick_vt(a);
  if (!a.bf16) {
    // fp32 operands double every LDS buffer: only d_k = d_v = 64 fits
    if (a.dk == 64 && a.dv == 64) return launch_chunk_t<float, 64, 64>(a);
    return hipErrorInvalidValue;
  }
  if (a.dk == 64) return vt == 64 ? launch_chunk_t<bf16_t, 64, 64>(a) : launch_chunk_t<bf16_t, 64, 128>(a);
  return vt == 64 ? launch_chunk_t<bf16_t, 128, 64>(a) : launch_chunk_t<bf16_t, 128, 128>(a);
}

// ---------------------------------------------------------------------------
// Two-pass forward, first pass: records of every chunk of every head, in parallel.
template <typename T, int DK, bool G2>
static hipError_t launch_prep_t(const ChunkArgs& a, char* ws, int cpw) {
  using K = Cfg<T, DK, 64>;
  auto kern = chunk_fwd_kernel<T, DK, 64, true, G2>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, K::LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  // varlen: workgroups over (head, runs of global chunks); BH = H, b = 0
  const int BH = a.cu ? a.H : a.B * a.H;
  const int nchunks = a.cu ? a.gmax : (a.T + C - 1) / C;
  const int nseg = (nchunks + cpw - 1) / cpw;
  if ((long)BH * nseg == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(BH * nseg), dim3(K::NT), K::LDS, (hipStream_t)a.stream, a.q, a.k, a.v, a.alpha,
                     a.beta, a.s0, a.o, a.sT, (float*)nullptr, a.T, a.H, a.dv, BH, ws, cpw, a.erase, a.cu, a.ctab,
                     a.ctab_total, a.gmax);
  return hipGetLastError();
}

template <bool G2>
static hipError_t launch_prep_g(const ChunkArgs& a, void* ws, int cpw) {
  return a.dk == 64 && a.dv == 64 ? launch_prep_t<float, 64, G2>(a, (char*)ws, cpw) : hipErrorInvalidValue;
}

// bf16 records (WalkRecord) come from the kernel sized for two workgroups per compute
// unit; the first half of the fused kernel writes the fp32 ones (RecordLayout)
hipError_t launch_prep(const ChunkArgs& a, void* ws, int cpw) {
  if (a.bf16) return launch_records(a, ws, cpw);
  if (a.cpx) return hipErrorInvalidValue;
  return a.erase ? launch_prep_g<true>(a, ws, cpw) : launch_prep_g<false>(a, ws, cpw);
}

size_t record_bytes(bool bf16, int dk) {
  if (!bf16) return RecordLayout<float, 64>::BYTES;
  return dk == 64 ? WalkRecord<64>::BYTES : WalkRecord<128>::BYTES;
}

}  // namespace kda
