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
// Layout of the work: one workgroup per (b, h) with DV / 16 waves; wave w owns
// value columns [16 w, 16 w + 16).  The fp32 state stays in registers for the
// whole sequence in accumulator layout (8 tiles of 16x16 at d_k = 128), and an
// accumulator pair is directly a matrix-core B fragment (the k-slot order is
// permuted to match).  q, k, alpha, beta, v of the next chunk are prefetched
// into registers while the current chunk computes.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int C = 64;
constexpr int SUB = 16;
constexpr int NB = C / SUB;

// Off-diagonal tile jobs (I, J) and which block-product Pi they need
// (-1: adjacent, none; 0: g1; 1: g1 g2; 2: g2).
__constant__ int kOffI[6] = {1, 2, 3, 2, 3, 3};
__constant__ int kOffJ[6] = {0, 1, 2, 0, 1, 0};
__constant__ int kOffPi[6] = {-1, -1, -1, 0, 2, 1};

template <typename T, int DK, int DV>
struct Cfg {
  static constexpr int ES = Elem<T>::kBytes;
  static constexpr int NW = DV / 16;
  static constexpr int NT = NW * 64;
  static constexpr int KS = DK / 32;  // k-steps over key channels
  static constexpr int RS_DK = DK * ES + 16;  // [pos][channel] rows (padded)
  static constexpr int RS_C = C * ES + 16;    // [channel][pos] and [pos][pos] rows of T type
  static constexpr int RS_DV = DV * ES + 16;  // [pos][value col]
  static constexpr int RS_F = C * 4 + 16;     // fp32 [pos][pos]
  // region R_IN: q, k, alpha -> later v (VV), M (MM, fp32), M~ (MT)
  static constexpr int SZ_IN_A = 3 * C * RS_DK;
  static constexpr int OFF_VV = 0;
  static constexpr int OFF_MM = OFF_VV + C * RS_DV;
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
  // region R_L: level operands (2 levels x 4 blocks x (16 A rows + 8 B rows)) -> later T, A (fp32), A~ (AT)
  static constexpr int LVL_ROWS = 24;
  static constexpr int SZ_L_A = 2 * NB * LVL_ROWS * RS_DK;
  static constexpr int OFF_TT = 0;          // later also W (WW) once T is consumed
  static constexpr int OFF_AA = OFF_TT + C * RS_F;  // later E = N_II T_IK blocks
  static constexpr int OFF_AT = OFF_AA + C * RS_F;
  static constexpr int SZ_L_B = OFF_AT + C * RS_C;
  static constexpr int SZ_L = SZ_L_A > SZ_L_B ? SZ_L_A : SZ_L_B;
  // small fp32 tables
  static constexpr int BASE_IN = 0;
  static constexpr int BASE_OP = BASE_IN + SZ_IN;
  static constexpr int BASE_L = BASE_OP + SZ_OP;
  static constexpr int BASE_GT = BASE_L + SZ_L;       // block totals g[4][DK]
  static constexpr int BASE_PI = BASE_GT + 4 * DK * 4;  // Pi tables [3][DK]
  static constexpr int BASE_GC = BASE_PI + 3 * DK * 4;  // gamma of the last row [DK]
  static constexpr int BASE_BETA = BASE_GC + DK * 4;    // beta [C]
  static constexpr int LDS = BASE_BETA + C * 4;
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(C * RS_DK <= C * RS_F, "W fits over T");
  // prefetch vectors (16 B) per thread
  static constexpr int VROW_K = DK * ES / 16;  // 16-byte vectors per q/k/alpha row
  static constexpr int VROW_V = DV * ES / 16;
  static constexpr int VPT = C * VROW_K / NT;
  static constexpr int VPT_V = C * VROW_V / NT;
  static_assert(VPT * NT == C * VROW_K && VPT_V * NT == C * VROW_V, "prefetch split");
  static constexpr int NITEM = NB * DK / 2;  // (block, channel pair) items of the gate passes
  static_assert(NITEM <= NT, "one gate item per thread");
};

template <typename T>
struct Pair;  // two adjacent channels of one row
template <>
struct Pair<bf16_t> {
  __device__ __forceinline__ static void load(const char* p, float& a, float& b) {
    uint32_t w = *(const uint32_t*)p;
    a = __uint_as_float(w << 16);
    b = __uint_as_float(w & 0xFFFF0000u);
  }
  __device__ __forceinline__ static void store(char* p, float a, float b) {
    *(uint32_t*)p = pack_bf16x2(a, b);
  }
};
template <>
struct Pair<float> {
  __device__ __forceinline__ static void load(const char* p, float& a, float& b) {
    float2 w = *(const float2*)p;
    a = w.x;
    b = w.y;
  }
  __device__ __forceinline__ static void store(char* p, float a, float b) {
    *(float2*)p = make_float2(a, b);
  }
};

__device__ __forceinline__ void st_elem_bf16_or_f32(char* p, float x, int es) {
  if (es == 2)
    *(uint16_t*)p = f32_to_bf16(x);
  else
    *(float*)p = x;
}

}  // namespace

template <typename T, int DK, int DV>
__global__ __launch_bounds__((DV / 16) * 64) void chunk_fwd_kernel(
    const void* __restrict__ gq, const void* __restrict__ gk, const void* __restrict__ gv,
    const void* __restrict__ galpha, const void* __restrict__ gbeta, const float* s0,
    void* __restrict__ go, float* sT, float* __restrict__ dbg, int Tlen, int H) {
  using K = Cfg<T, DK, DV>;
  constexpr int ES = K::ES;
  constexpr int NT = K::NT;
  constexpr int NW = K::NW;
  extern __shared__ __align__(16) char smem[];
  char* const R_IN = smem + K::BASE_IN;
  char* const R_OP = smem + K::BASE_OP;
  char* const R_L = smem + K::BASE_L;
  float* const GT = (float*)(smem + K::BASE_GT);
  float* const PI = (float*)(smem + K::BASE_PI);
  float* const GC = (float*)(smem + K::BASE_GC);
  float* const BETA = (float*)(smem + K::BASE_BETA);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh % H;
  const int nchunks = (Tlen + C - 1) / C;

  // ---------------- state tiles (rows 16 r .. of key channels, columns 16 wave + n)
  f32x4_t S[DK / 16];
#pragma unroll
  for (int r = 0; r < DK / 16; ++r) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      S[r][e] = s0 ? s0[((size_t)bh * DK + 16 * r + 4 * g + e) * DV + 16 * wave + n] : 0.f;
  }

  // ---------------- prefetch registers
  uint4 pq[K::VPT], pk[K::VPT], pa[K::VPT], pv[K::VPT_V];
  float pb = 0.f;
  auto row_base = [&](int t) -> size_t { return ((size_t)b * Tlen + t) * H + h; };
  auto issue_qka = [&](int c) {
    const int t0 = c * C;
#pragma unroll
    for (int i = 0; i < K::VPT; ++i) {
      const int j = tid + NT * i;
      const int row = j / K::VROW_K, c16 = j % K::VROW_K;
      if (t0 + row < Tlen) {
        const size_t off = row_base(t0 + row) * DK * ES + (size_t)c16 * 16;
        pq[i] = *(const uint4*)((const char*)gq + off);
        pk[i] = *(const uint4*)((const char*)gk + off);
        pa[i] = *(const uint4*)((const char*)galpha + off);
      } else {
        pq[i] = make_uint4(0, 0, 0, 0);
        pk[i] = make_uint4(0, 0, 0, 0);
        // alpha = 1 on padded rows: identity transitions
        const uint32_t one = ES == 2 ? 0x3F803F80u : 0x3F800000u;
        pa[i] = make_uint4(one, one, one, one);
      }
    }
    if (tid < C) pb = (t0 + tid < Tlen) ? Elem<T>::load(gbeta, row_base(t0 + tid)) : 0.f;
  };
  auto issue_v = [&](int c) {
    const int t0 = c * C;
#pragma unroll
    for (int i = 0; i < K::VPT_V; ++i) {
      const int j = tid + NT * i;
      const int row = j / K::VROW_V, c16 = j % K::VROW_V;
      pv[i] = (t0 + row < Tlen)
                  ? *(const uint4*)((const char*)gv + row_base(t0 + row) * DV * ES + (size_t)c16 * 16)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  if (nchunks > 0) {
    issue_qka(0);
    issue_v(0);
  }

  // gate-pass item: (block I, channel pair cp)
  const bool has_item = tid < K::NITEM;
  const int iI = tid / (DK / 2);
  const int icp = tid % (DK / 2);

  for (int chunk = 0; chunk < nchunks; ++chunk) {
    const int t0 = chunk * C;
    const int nv = min(C, Tlen - t0);
    // ================= phase 0: staged inputs -> LDS
    __syncthreads();
#pragma unroll
    for (int i = 0; i < K::VPT; ++i) {
      const int j = tid + NT * i;
      const int row = j / K::VROW_K, c16 = j % K::VROW_K;
      const int off = row * K::RS_DK + c16 * 16;
      *(uint4*)(R_IN + 0 * C * K::RS_DK + off) = pq[i];
      *(uint4*)(R_IN + 1 * C * K::RS_DK + off) = pk[i];
      *(uint4*)(R_IN + 2 * C * K::RS_DK + off) = pa[i];
    }
    if (tid < C) BETA[tid] = pb;
    __syncthreads();
    if (chunk + 1 < nchunks) issue_qka(chunk + 1);

    const char* const Qs = R_IN;
    const char* const Ks = R_IN + C * K::RS_DK;
    const char* const As = R_IN + 2 * C * K::RS_DK;

    // ================= phase A: block totals of the gates
    // gate-pass item (block iI, channels 2 icp, 2 icp + 1); alpha / q / k are
    // re-read from LDS in every gate phase rather than held across barriers.
    const int item_off = (SUB * iI) * K::RS_DK + 2 * icp * ES;
    auto ld_alpha = [&](float (&al)[SUB][2]) {
#pragma unroll
      for (int m = 0; m < SUB; ++m) Pair<T>::load(As + item_off + m * K::RS_DK, al[m][0], al[m][1]);
    };
    auto ld_q = [&](int m, float& a, float& b) { Pair<T>::load(Qs + item_off + m * K::RS_DK, a, b); };
    auto ld_k = [&](int m, float& a, float& b) { Pair<T>::load(Ks + item_off + m * K::RS_DK, a, b); };
    if (has_item) {
      float al[SUB][2];
      ld_alpha(al);
      float g0 = 1.f, g1 = 1.f;
#pragma unroll
      for (int m = 0; m < SUB; ++m) {
        g0 *= al[m][0];
        g1 *= al[m][1];
      }
      GT[iI * DK + 2 * icp] = g0;
      GT[iI * DK + 2 * icp + 1] = g1;
    }
    __syncthreads();

    // chunk-level products for the item's channels
    float Gp[2] = {1.f, 1.f}, Rp[2] = {1.f, 1.f};
    if (has_item) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int c = 2 * icp + e;
        const float t0v = GT[c], t1v = GT[DK + c], t2v = GT[2 * DK + c], t3v = GT[3 * DK + c];
        Gp[e] = iI == 0 ? 1.f : iI == 1 ? t0v : iI == 2 ? t0v * t1v : t0v * t1v * t2v;
        Rp[e] = iI == 3 ? 1.f : iI == 2 ? t3v : iI == 1 ? t2v * t3v : t1v * t2v * t3v;
        if (iI == 0) {
          PI[0 * DK + c] = t1v;
          PI[1 * DK + c] = t1v * t2v;
          PI[2 * DK + c] = t2v;
          GC[c] = t0v * t1v * t2v * t3v;
        }
      }
    }

    // level operand writer: slot ls (0/1), block I, level lam
    auto write_levels = [&](const float (&al)[SUB][2], int ls, int lam) {
      char* LA = R_L + (size_t)(ls * NB + iI) * K::LVL_ROWS * K::RS_DK;
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
          ld_q(m, q0, q1);
          ld_k(m, k0, k1);
          Pair<T>::store(LA + u * K::RS_DK + 2 * icp * ES, q0 * f0, q1 * f1);
          Pair<T>::store(LA + (8 + u) * K::RS_DK + 2 * icp * ES, k0 * f0, k1 * f1);
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
          ld_k(m, k0, k1);
          Pair<T>::store(LB + v * K::RS_DK + 2 * icp * ES, k0 * b0, k1 * b1);
        }
      }
    };

    // ================= phase B: 16-block anchored operands + level 8 / 4 operands
    if (has_item) {
      float al[SUB][2];
      ld_alpha(al);
      char* Xq = R_OP;
      char* Xk = R_OP + C * K::RS_DK;
      char* Y = R_OP + 2 * C * K::RS_DK;
      float f0 = 1.f, f1 = 1.f;
#pragma unroll
      for (int m = 0; m < SUB; ++m) {
        f0 *= al[m][0];
        f1 *= al[m][1];
        float q0, q1, k0, k1;
        ld_q(m, q0, q1);
        ld_k(m, k0, k1);
        Pair<T>::store(Xq + item_off + m * K::RS_DK, q0 * f0, q1 * f1);
        Pair<T>::store(Xk + item_off + m * K::RS_DK, k0 * f0, k1 * f1);
      }
      float b0 = 1.f, b1 = 1.f;
#pragma unroll
      for (int m = SUB - 1; m >= 0; --m) {
        float k0, k1;
        ld_k(m, k0, k1);
        Pair<T>::store(Y + item_off + m * K::RS_DK, k0 * b0, k1 * b1);
        b0 *= al[m][0];
        b1 *= al[m][1];
      }
      write_levels(al, 0, 8);
      write_levels(al, 1, 4);
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
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) {
          const int c0 = 32 * ks + 8 * g;
          Frag<T> fa, fk, fb;
          fb.load8(Y + c0 * ES);
          if (pi >= 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) fb.set(e, fb.get(e) * PI[pi * DK + c0 + e]);
          }
          fa.load8(Xq + c0 * ES);
          fk.load8(Xk + c0 * ES);
          mma(r1a[s], fa, fb);
          mma(r1t[s], fk, fb);
        }
      } else if (j < NJ1) {
        const int ls = (j - 6) / NB, I = (j - 6) % NB;
        const char* LA = R_L + (size_t)(ls * NB + I) * K::LVL_ROWS * K::RS_DK;
        const char* LB = LA + 16 * K::RS_DK;
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) {
          const int c0 = 32 * ks + 8 * g;
          Frag<T> fa, fb;
          fa.load8(LA + n * K::RS_DK + c0 * ES);
          if (n < 8)
            fb.load8(LB + n * K::RS_DK + c0 * ES);
          else
            fb.zero();
          mma(r1a[s], fa, fb);
        }
      }
    }
    __syncthreads();

    // ================= phase C: gamma / rho operands + level 2 / 1 operands
    if (has_item) {
      float al[SUB][2];
      ld_alpha(al);
      char* QG = R_OP + K::OFF_QG;
      char* KGT = R_OP + K::OFF_KGT;
      char* KRT = R_OP + K::OFF_KRT;
      char* kg_row0 = KGT + (2 * icp) * K::RS_C + (SUB * iI) * ES;
      char* kg_row1 = kg_row0 + K::RS_C;
      char* kr_row0 = KRT + (2 * icp) * K::RS_C + (SUB * iI) * ES;
      char* kr_row1 = kr_row0 + K::RS_C;
      float f0 = Gp[0], f1 = Gp[1];
      float p0 = 0.f, p1 = 0.f;  // previous position's values (pairs of positions per store)
#pragma unroll
      for (int m = 0; m < SUB; ++m) {
        f0 *= al[m][0];
        f1 *= al[m][1];
        float q0, q1, k0, k1;
        ld_q(m, q0, q1);
        ld_k(m, k0, k1);
        Pair<T>::store(QG + item_off + m * K::RS_DK, q0 * f0, q1 * f1);
        if (m & 1) {
          Pair<T>::store(kg_row0 + (m - 1) * ES, p0, k0 * f0);
          Pair<T>::store(kg_row1 + (m - 1) * ES, p1, k1 * f1);
        } else {
          p0 = k0 * f0;
          p1 = k1 * f1;
        }
      }
      float b0 = Rp[0], b1 = Rp[1];
#pragma unroll
      for (int m = SUB - 1; m >= 0; --m) {
        float k0, k1;
        ld_k(m, k0, k1);
        if (m & 1) {
          p0 = k0 * b0;
          p1 = k1 * b1;
        } else {
          Pair<T>::store(kr_row0 + m * ES, k0 * b0, p0);
          Pair<T>::store(kr_row1 + m * ES, k1 * b1, p1);
        }
        b0 *= al[m][0];
        b1 *= al[m][1];
      }
      write_levels(al, 0, 2);
      write_levels(al, 1, 1);
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
      if (j < 8) {
        const int ls = j / NB, I = j % NB;
        const char* LA = R_L + (size_t)(ls * NB + I) * K::LVL_ROWS * K::RS_DK;
        const char* LB = LA + 16 * K::RS_DK;
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) {
          const int c0 = 32 * ks + 8 * g;
          Frag<T> fa, fb;
          fa.load8(LA + n * K::RS_DK + c0 * ES);
          if (n < 8)
            fb.load8(LB + n * K::RS_DK + c0 * ES);
          else
            fb.zero();
          mma(r2[s], fa, fb);
        }
      } else if (j < NJ2) {
        const int I = j - 8;
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) {
          const int c0 = 32 * ks + 8 * g;
          Frag<T> fa, fb;
          fa.load8(Qs + (16 * I + n) * K::RS_DK + c0 * ES);
          fb.load8(Ks + (16 * I + n) * K::RS_DK + c0 * ES);
          mma(r2[s], fa, fb);
        }
      }
    }
    __syncthreads();

    // ================= phase D: scatter T and A (fp32) and stage v
    float* TT = (float*)(R_L + K::OFF_TT);
    float* AA = (float*)(R_L + K::OFF_AA);
    constexpr int LDF = K::RS_F / 4;
    auto put_level = [&](const f32x4_t& acc, int lam, int I) {
      if (n < 8) {
        const int v = n;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 4 * g + e;
          const int u = row & 7;
          if (u / lam == v / lam) {
            const int mu = (u / lam) * 2 * lam + lam + (u % lam);
            const int ml = (v / lam) * 2 * lam + (v % lam);
            const int gi = 16 * I + mu, gj = 16 * I + ml;
            if (row < 8)
              AA[gi * LDF + gj] = acc[e];
            else
              TT[gi * LDF + gj] = BETA[gi] * acc[e];
          }
        }
      }
    };
#pragma unroll
    for (int s = 0; s < MJ1; ++s) {
      const int j = wave + s * NW;
      if (j < 6) {
        const int I = kOffI[j], J = kOffJ[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int gi = 16 * I + 4 * g + e, gj = 16 * J + n;
          AA[gi * LDF + gj] = r1a[s][e];
          TT[gi * LDF + gj] = BETA[gi] * r1t[s][e];
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
        for (int e = 0; e < 4; ++e)
          if (4 * g + e == n) AA[(16 * I + n) * LDF + 16 * I + n] = r2[s][e];
      }
    }
    // v of this chunk -> LDS, then prefetch the next chunk's v
#pragma unroll
    for (int i = 0; i < K::VPT_V; ++i) {
      const int j = tid + NT * i;
      const int row = j / K::VROW_V, c16 = j % K::VROW_V;
      *(uint4*)(R_IN + K::OFF_VV + row * K::RS_DV + c16 * 16) = pv[i];
    }
    if (chunk + 1 < nchunks) issue_v(chunk + 1);
    __syncthreads();

    if (dbg) {
      float* D = dbg + ((size_t)bh * nchunks + chunk) * 4 * C * C;
      for (int x = tid; x < C * C; x += NT) {
        const int i = x / C, j = x % C;
        D[x] = j < i ? TT[i * LDF + j] : 0.f;
        D[C * C + x] = j <= i ? AA[i * LDF + j] : 0.f;
      }
    }

    // ================= phase I: M = (I + T)^-1
    float* MM = (float*)(R_IN + K::OFF_MM);
    char* MT = R_IN + K::OFF_MT;
    char* AT = R_L + K::OFF_AT;
    if (wave == 0) {
      // diagonal blocks by forward substitution: lane = (block, column)
      const int I = lane >> 4, col = lane & 15;
      float x[SUB];
#pragma unroll
      for (int i = 0; i < SUB; ++i) {
        const float* trow = TT + (16 * I + i) * LDF + 16 * I;
        float acc = (i == col) ? 1.f : 0.f;
#pragma unroll
        for (int p = 0; p < i; ++p) acc -= trow[p] * x[p];
        x[i] = acc;
      }
#pragma unroll
      for (int i = 0; i < SUB; ++i) MM[(16 * I + i) * LDF + 16 * I + col] = x[i];
    } else {
      // A~ = A (lower incl. diagonal) as matrix-core operand
      for (int x = tid - 64; x < C * C; x += NT - 64) {
        const int i = x / C, j = x % C;
        st_elem_bf16_or_f32(AT + i * K::RS_C + j * ES, j <= i ? AA[i * LDF + j] : 0.f, ES);
      }
    }
    __syncthreads();
    // E_IK = N_II T_IK for K < I, into the A buffer (A~ already formed)
    float* EE = AA;
    for (int x = tid; x < 6 * 256; x += NT) {
      const int blk = x >> 8, i = (x >> 4) & 15, r = x & 15;
      const int I = kOffI[blk], Kb = kOffJ[blk];
      float acc = 0.f;
#pragma unroll
      for (int p = 0; p < SUB; ++p) acc += MM[(16 * I + i) * LDF + 16 * I + p] * TT[(16 * I + p) * LDF + 16 * Kb + r];
      EE[(16 * I + i) * LDF + 16 * Kb + r] = acc;
    }
    __syncthreads();
    // block rows: M_IJ = -sum_{K=J}^{I-1} E_IK M_KJ
#pragma unroll
    for (int I = 1; I < NB; ++I) {
      for (int x = tid; x < I * 256; x += NT) {
        const int J = x >> 8, i = (x >> 4) & 15, j = x & 15;
        float acc = 0.f;
        for (int Kb = J; Kb < I; ++Kb) {
#pragma unroll
          for (int r = 0; r < SUB; ++r)
            acc += EE[(16 * I + i) * LDF + 16 * Kb + r] * MM[(16 * Kb + r) * LDF + 16 * J + j];
        }
        MM[(16 * I + i) * LDF + 16 * J + j] = -acc;
      }
      __syncthreads();
    }
    // M~ = M diag(beta), lower incl. diagonal, as matrix-core operand
    for (int x = tid; x < C * C; x += NT) {
      const int i = x / C, j = x % C;
      st_elem_bf16_or_f32(MT + i * K::RS_C + j * ES, j <= i ? MM[i * LDF + j] * BETA[j] : 0.f, ES);
    }
    if (dbg) {
      float* D = dbg + ((size_t)bh * nchunks + chunk) * 4 * C * C + 2 * C * C;
      for (int x = tid; x < C * C; x += NT) {
        const int i = x / C, j = x % C;
        D[x] = j <= i ? MM[i * LDF + j] : 0.f;
      }
    }
    __syncthreads();

    // ================= phase W: W = M~ (K o gamma) -> -W in LDS;  U_w = M~ V[:, w] in registers
    char* WW = R_L + K::OFF_TT;
    {
      constexpr int NCT = DK / 16;
      for (int t = wave; t < NB * NCT; t += NW) {
        const int I = t / NCT, cn = t % NCT;
        f32x4_t acc = zero4();
        const int nks = I < 2 ? 1 : 2;
        for (int ks = 0; ks < nks; ++ks) {
          Frag<T> fa, fb;
          fa.load8(MT + (16 * I + n) * K::RS_C + (32 * ks + 8 * g) * ES);
          fb.load8(R_OP + K::OFF_KGT + (16 * cn + n) * K::RS_C + (32 * ks + 8 * g) * ES);
          mma(acc, fa, fb);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
          st_elem_bf16_or_f32(WW + (16 * I + 4 * g + e) * K::RS_DK + (16 * cn + n) * ES, -acc[e], ES);
        if (dbg && cn < 4) {
          float* D = dbg + ((size_t)bh * nchunks + chunk) * 4 * C * C + 3 * C * C;
#pragma unroll
          for (int e = 0; e < 4; ++e) D[(16 * I + 4 * g + e) * C + 16 * cn + n] = acc[e];
        }
      }
    }
    f32x4_t Dl[NB];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      Dl[I] = zero4();
      const int nks = I < 2 ? 1 : 2;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks < nks) {
          Frag<T> fa, fb;
          fa.load8(MT + (16 * I + n) * K::RS_C + (32 * ks + 8 * g) * ES);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            fb.set(e, Elem<T>::load(R_IN + K::OFF_VV + (32 * ks + 8 * g + e) * K::RS_DV, 16 * wave + n));
          mma(Dl[I], fa, fb);
        }
      }
    }
    __syncthreads();

    // ================= phase S: Delta = U - W S ; O = (Q o gamma) S + A Delta ; S update
    {
      Frag<T> bs[K::KS];
#pragma unroll
      for (int ks = 0; ks < K::KS; ++ks) bs[ks].from_acc(S[2 * ks], S[2 * ks + 1]);
      f32x4_t Ot[NB];
#pragma unroll
      for (int I = 0; I < NB; ++I) {
        Ot[I] = zero4();
        const char* wrow = WW + (16 * I + n) * K::RS_DK;
        const char* qrow = R_OP + K::OFF_QG + (16 * I + n) * K::RS_DK;
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) {
          const int c0 = 32 * ks + 4 * g;
          Frag<T> fw, fq;
          fw.load4x2(wrow + c0 * ES, wrow + (c0 + 16) * ES);
          fq.load4x2(qrow + c0 * ES, qrow + (c0 + 16) * ES);
          mma(Dl[I], fw, bs[ks]);
          mma(Ot[I], fq, bs[ks]);
        }
      }
      Frag<T> bd[2];
      bd[0].from_acc(Dl[0], Dl[1]);
      bd[1].from_acc(Dl[2], Dl[3]);
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
#pragma unroll
        for (int e = 0; e < 4; ++e) S[r][e] *= GC[16 * r + 4 * g + e];
        const char* krow = R_OP + K::OFF_KRT + (16 * r + n) * K::RS_C;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int p0 = 32 * s2 + 4 * g;
          Frag<T> fa;
          fa.load4x2(krow + p0 * ES, krow + (p0 + 16) * ES);
          mma(S[r], fa, bd[s2]);
        }
      }
      // stage O (reuses the v slot of R_IN: v is consumed)
#pragma unroll
      for (int I = 0; I < NB; ++I)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          st_elem_bf16_or_f32(R_IN + K::OFF_VV + (16 * I + 4 * g + e) * K::RS_DV + (16 * wave + n) * ES,
                              Ot[I][e], ES);
    }
    __syncthreads();
    // ================= phase O: coalesced store of the chunk's outputs
    for (int j = tid; j < C * K::VROW_V; j += NT) {
      const int row = j / K::VROW_V, c16 = j % K::VROW_V;
      if (row < nv)
        *(uint4*)((char*)go + row_base(t0 + row) * DV * ES + (size_t)c16 * 16) =
            *(const uint4*)(R_IN + K::OFF_VV + row * K::RS_DV + c16 * 16);
    }
  }

  if (sT) {
#pragma unroll
    for (int r = 0; r < DK / 16; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) sT[((size_t)bh * DK + 16 * r + 4 * g + e) * DV + 16 * wave + n] = S[r][e];
  }
}

template <typename T, int DK, int DV>
static hipError_t launch_chunk_t(const ChunkArgs& a) {
  using K = Cfg<T, DK, DV>;
  auto kern = chunk_fwd_kernel<T, DK, DV>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, K::LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(a.B * a.H), dim3(K::NT), K::LDS, (hipStream_t)a.stream, a.q, a.k, a.v,
                     a.alpha, a.beta, a.s0, a.o, a.sT, a.dbg, a.T, a.H);
  return hipGetLastError();
}

hipError_t launch_chunk(const ChunkArgs& a) {
  if (a.B * a.H == 0) return hipSuccess;
  if (!a.bf16) {
    // fp32 operands double every LDS buffer: only d_k = d_v = 64 fits
    if (a.dk == 64 && a.dv == 64) return launch_chunk_t<float, 64, 64>(a);
    return hipErrorInvalidValue;
  }
  if (a.dk == 64 && a.dv == 64) return launch_chunk_t<bf16_t, 64, 64>(a);
  if (a.dk == 64 && a.dv == 128) return launch_chunk_t<bf16_t, 64, 128>(a);
  if (a.dk == 128 && a.dv == 64) return launch_chunk_t<bf16_t, 128, 64>(a);
  return launch_chunk_t<bf16_t, 128, 128>(a);
}

}  // namespace kda
