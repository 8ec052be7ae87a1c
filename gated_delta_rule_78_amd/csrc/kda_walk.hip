// kda_walk.hip -- second pass of the two-pass chunk forward for bf16 inputs: the walk of
// the state along the chunks of each (b, h, value tile).
//
// Per chunk, with the fp32 state S [d_k x VT] in registers (matrix-core accumulator
// layout), the chunk's record (A, M~ = (I + T)^-1 diag(beta) as a bf16 pair) and the
// chunk's q, k, alpha, v:
//   R     = V - (K o gamma) S
//   Delta = M~ R                              (= M~ V - M~ (K o gamma) S = U - W S)
//   O     = (Q o gamma) S + A Delta
//   S    <- diag(gamma_last) S + (K o rho)^T Delta
// which is the chunk's exact affine transfer (SFDA page, "Principales Contribuciones"
// item 3; the chunk-WY form of "El Teorema de Chunk-WY Constructivo" with the decay
// absorbed into the triangular solve as on the Gated DeltaNet-2 page, section 3).
//
// Precision.  Where the transitions are orthogonal (CKDA page, "Complex KDA (CKDA)
// Mimarisi": |alpha| = 1 per channel, beta in {0, 2}) the state never decays, so every
// rounding of a quantity that multiplies S is carried to the end of the sequence and the
// errors add up like a random walk over the chunks.  The products that feed the state
// therefore take their variable operands as bf16 pairs x = hi + lo (hi = bf16(x),
// lo = bf16(x - hi), about 2^-17 relative): S in R = V - K S, R and M~ in Delta = M~ R,
// Delta in the state update.  The key-side operands (K o gamma, K o rho) are a product
// of bf16 inputs and gate products: exact in bf16 where |alpha| = 1, and where a gate is
// smaller the channel forgets its rounding within a few chunks (bf16 gates below one are
// at most 1 - 2^-9).  The readout products (Q o gamma) S and A Delta take single bf16
// operands: their errors end in the output, not in the state.
//
// Work split in a workgroup: VT / 16 compute waves (16 value columns each) and four
// producer waves.  The producers load the chunk's record (A, M~ hi, M~ lo) and v tile into
// registers a step ahead and write them to the second of two LDS buffer sets (the next
// chunk is assembled while the current one computes), and rebuild the chunk's operands
// Q o gamma, -(K o gamma) and (K o rho)^T and gamma_last from q, k, alpha alone (one gate
// item = 4 rows x 8 channels per lane, loaded a step ahead; the running products across
// row groups are DPP scans).
#include <stdlib.h>

#include "kda_common.h"
#include "kda_internal.h"
#include "kda_record.h"
#include "kda_tile.h"

namespace kda {

namespace {

// LDS stores of the producer waves (operands, record, v tile), written as instructions the
// compiler does not analyse, so that it neither orders them behind the compute waves'
// buffer reads nor waits on them; they complete before the step barrier (lgkmcnt(0)).
__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void lds_st32(void* p, uint32_t v) {
#ifndef KDA_HOST_PASS
  asm volatile("ds_write_b32 %0, %1" ::"v"(lds_off(p)), "v"(v) : "memory");
#endif
}
__device__ __forceinline__ void lds_st64(void* p, float x, float y) {
#ifndef KDA_HOST_PASS
  typedef float f2 __attribute__((ext_vector_type(2)));
  f2 v = {x, y};
  asm volatile("ds_write_b64 %0, %1" ::"v"(lds_off(p)), "v"(v) : "memory");
#endif
}
__device__ __forceinline__ void lds_st128(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
#ifndef KDA_HOST_PASS
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  u4 v = {a, b, c, d};
  asm volatile("ds_write_b128 %0, %1" ::"v"(lds_off(p)), "v"(v) : "memory");
#endif
}

// The gate product v of the lane CTRL's DPP row shift points at (row_shr:d = 0x110 + d,
// row_shl:d = 0x100 + d), or the identity where that lane lies outside the 16-lane row.
template <typename G, int CTRL>
__device__ __forceinline__ G dpp_fill(const G& v) {
  const G one = G::one();
  auto f = [](float old, float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                                 __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
  };
  return G{f(one.x, v.x), f(one.y, v.y)};
}

// Inclusive products along each 16-lane DPP row of eight values: I over the lanes up to
// this one, J over the lanes from this one on (lane i multiplies in lane i -+ d for
// d = 1, 2, 4, 8; a lane whose partner lies outside the row is left as it is).  The 16
// chains are interleaved, so no cross-lane read follows the write of its source closely
// (the leading s_nop covers the inputs' writes).
__device__ __forceinline__ void row_scan16(float (&I)[8], float (&J)[8]) {
#ifndef KDA_HOST_PASS
  asm volatile(
      "s_nop 1\n"
      "v_mul_f32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %1, %1, %1 row_shr:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %2, %2, %2 row_shr:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %3, %3, %3 row_shr:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %4, %4, %4 row_shr:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %5, %5, %5 row_shr:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %6, %6, %6 row_shr:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %7, %7, %7 row_shr:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %8, %8, %8 row_shl:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %9, %9, %9 row_shl:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %10, %10, %10 row_shl:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %11, %11, %11 row_shl:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %12, %12, %12 row_shl:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %13, %13, %13 row_shl:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %14, %14, %14 row_shl:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %15, %15, %15 row_shl:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %1, %1, %1 row_shr:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %2, %2, %2 row_shr:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %3, %3, %3 row_shr:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %4, %4, %4 row_shr:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %5, %5, %5 row_shr:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %6, %6, %6 row_shr:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %7, %7, %7 row_shr:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %8, %8, %8 row_shl:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %9, %9, %9 row_shl:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %10, %10, %10 row_shl:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %11, %11, %11 row_shl:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %12, %12, %12 row_shl:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %13, %13, %13 row_shl:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %14, %14, %14 row_shl:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %15, %15, %15 row_shl:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %1, %1, %1 row_shr:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %2, %2, %2 row_shr:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %3, %3, %3 row_shr:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %4, %4, %4 row_shr:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %5, %5, %5 row_shr:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %6, %6, %6 row_shr:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %7, %7, %7 row_shr:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %8, %8, %8 row_shl:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %9, %9, %9 row_shl:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %10, %10, %10 row_shl:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %11, %11, %11 row_shl:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %12, %12, %12 row_shl:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %13, %13, %13 row_shl:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %14, %14, %14 row_shl:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %15, %15, %15 row_shl:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %0, %0, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %1, %1, %1 row_shr:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %2, %2, %2 row_shr:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %3, %3, %3 row_shr:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %4, %4, %4 row_shr:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %5, %5, %5 row_shr:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %6, %6, %6 row_shr:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %7, %7, %7 row_shr:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %8, %8, %8 row_shl:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %9, %9, %9 row_shl:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %10, %10, %10 row_shl:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %11, %11, %11 row_shl:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %12, %12, %12 row_shl:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %13, %13, %13 row_shl:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %14, %14, %14 row_shl:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %15, %15, %15 row_shl:8 row_mask:0xf bank_mask:0xf\n"
      : "+v"(I[0]), "+v"(I[1]), "+v"(I[2]), "+v"(I[3]), "+v"(I[4]), "+v"(I[5]), "+v"(I[6]), "+v"(I[7]), "+v"(J[0]), "+v"(J[1]), "+v"(J[2]), "+v"(J[3]), "+v"(J[4]), "+v"(J[5]), "+v"(J[6]), "+v"(J[7]));
#endif
}

// A workgroup barrier that waits for this wave's LDS operations only.
__device__ __forceinline__ void lds_barrier_only() {
#ifndef KDA_HOST_PASS
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
#endif
}

template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

// fp32 pair -> bf16 pair hi = bf16(x) and the rounding residual lo = bf16(x - hi)
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(x0, x1);
  lo = pack_bf16x2(x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xFFFF0000u));
}

// Two accumulator tiles (rows 4g + e of tile a, rows 16 + 4g + e of tile b, column n) as
// the hi and lo B fragments of one 32-deep product step (k-slots 4g + e and 16 + 4g + e;
// the A side loads the matching columns, so the k-slot order is free).
__device__ __forceinline__ void split_acc(const f32x4_t& a, const f32x4_t& b, Frag<bf16_t>& hi, Frag<bf16_t>& lo) {
  split_pair(a[0], a[1], hi.w[0], lo.w[0]);
  split_pair(a[2], a[3], hi.w[1], lo.w[1]);
  split_pair(b[0], b[1], hi.w[2], lo.w[2]);
  split_pair(b[2], b[3], hi.w[3], lo.w[3]);
}

template <int DK, int VT>
struct WCfg {
  using RL = WalkRecord<DK>;
  static constexpr int NW = VT / 16;  // compute waves
  static constexpr int NP = 4;        // producer waves
  static constexpr int NT = (NW + NP) * 64;
  static constexpr int KS = DK / 32;
  static constexpr int RS_Q = DK * 2 + 16;  // [pos][channel] rows of Q o gamma, -(K o gamma)
  static constexpr int RS_KT = C * 2;       // [channel][pos] rows of (K o rho)^T, 16-byte units swizzled
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_K = OFF_Q + C * RS_Q;
  static constexpr int OFF_KT = OFF_K + C * RS_Q;
  static constexpr int OFF_G = OFF_KT + DK * RS_KT;  // gamma_last, fp32 [DK]
  static constexpr int OPS = OFF_G + DK * 4;
  static constexpr int RS_V = VT * 2;  // v tile rows (dense: filled by DMA), reused for O
  static constexpr int UPR = RS_V / 16;
  static constexpr int V_BYTES = C * RS_V;
  static constexpr int N_DMA_REC = RL::DMA / 1024;
  static constexpr int N_DMA_V = C * UPR / 64;
  static constexpr int NITEM = 2 * DK;  // gate items: 16 row groups x DK / 8 channel groups
  static_assert(NITEM <= NP * 64, "one gate item per producer lane");
  static_assert(N_DMA_V * 64 == C * UPR, "v tile split");
  static_assert(2 * (OPS + RL::DMA + V_BYTES) <= 160 * 1024, "LDS budget");
  // byte offset of the 16-byte unit u of (K o rho)^T row c: the unit index is XORed with
  // bits 1..3 of the row, so the sixteen rows a matrix-core fragment load touches (and
  // the two rows a gate item writes) spread over all LDS banks without row padding
  __device__ static constexpr int kt_unit(int c, int u) { return c * RS_KT + 16 * (u ^ ((c >> 1) & 7)); }
  // v tile: LDS unit u of row r holds the tile's 16-byte unit u ^ vsw(r) (the DMA and the
  // output store apply the same permutation), so the four row groups 4g + e that a
  // fragment's lanes read fall on different banks
  __device__ static constexpr int vsw(int r) { return ((r >> 2) & 3) * 2 & (UPR - 1); }
};

// flags of a split walk (launch_walk_split): no output stores; v read as zero; start from
// the identity; only the last segment writes the end state, indexed by (b, h); the start
// state indexed by (b, h) (S_0 itself); the end state written as the next segment's start
enum : int { kSegNoOut = 1, kSegZeroV = 2, kSegIdentity = 4, kSegLastOnly = 8, kSegS0Head = 16, kSegEndNext = 32 };
// what a walk computes (a compile-time choice: the split walk's first two passes skip the
// work they would discard): everything; the state only (outputs neither formed nor
// stored, no Q o gamma); the state only with v = 0 (no v tile either)
enum : int { kWalkFull = 0, kWalkState = 1, kWalkTransfer = 2 };

__device__ __forceinline__ void fence_sched() {
#ifndef KDA_HOST_PASS
  __builtin_amdgcn_sched_barrier(0);
#endif
}

// One chunk of the walk for compute wave `wave` (value columns 16 wave + n of the tile):
// operands in `ops`, record (A, MH, ML) in `rec`, v tile in `vv` (rows past the end of the
// sequence hold zeros); S advances one chunk and the outputs are staged over this wave's
// own (consumed) columns of `vv`.
template <int DK, int VT, bool G2, bool CPX, int MODE>
__device__ __forceinline__ void walk_chunk(const char* ops, const char* rec, char* vv, const float (&wf)[16],
                                           f32x4_t (&S)[DK / 16], int wave, int g, int n) {
  constexpr bool kOut = MODE == kWalkFull;    // outputs formed and staged
  constexpr bool kV = MODE != kWalkTransfer;  // v read
  using K = WCfg<DK, VT>;
  using RL = typename K::RL;
  constexpr int KS = K::KS;
  const char* OQ = ops + K::OFF_Q;
  const char* OK = ops + K::OFF_K;
  const char* OKT = ops + K::OFF_KT;
  const float* OG = (const float*)(ops + K::OFF_G);
  const int col = 16 * wave + n;

  // (one base address for this lane's column of the v tile, rows at immediate offsets; the
  // tile is read whole: the producers store the rows past the end, and the whole tile when
  // v is read as zero, as zeros, so no per-row address, mask or branch).
  // Rows 16 I + 4g + e share the unit permutation of row 4g (vsw depends on bits 2, 3).
  char* const vb = vv + 4 * g * K::RS_V + 16 * ((col >> 3) ^ K::vsw(4 * g)) + (col & 7) * 2;
  // The operand fragments of each group of products are loaded one group ahead and the
  // scheduling fences keep them there: with one compute wave per SIMD little else hides
  // the LDS latency.
  auto ld_kq = [&](int ks, Frag<bf16_t> (&fk)[NB], Frag<bf16_t> (&fq)[NB]) __attribute__((always_inline)) {
    const int c0 = 32 * ks + 4 * g;
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      const char* krow = OK + (16 * I + n) * K::RS_Q;
      const char* qrow = OQ + (16 * I + n) * K::RS_Q;
      fk[I].load4x2(krow + c0 * 2, krow + (c0 + 16) * 2);
      if constexpr (kOut) fq[I].load4x2(qrow + c0 * 2, qrow + (c0 + 16) * 2);
    }
  };
  // (I, s2) of the six lower 16 x 32 blocks of a 64 x 64 record matrix
  auto blk_I = [](int j) { return j < 2 ? j : 2 + (j - 2) / 2; };
  auto blk_s = [](int j) { return j < 2 ? 0 : (j - 2) % 2; };
  auto ld_rec = [&](int mat, int j, Frag<bf16_t>& f) __attribute__((always_inline)) {
    const int I = blk_I(j), s2 = blk_s(j);
    f.load4x2(rec + mat + RL::at(16 * I + n, 32 * s2 + 4 * g), rec + mat + RL::at(16 * I + n, 32 * s2 + 16 + 4 * g));
  };
  auto ld_kt = [&](int r, Frag<bf16_t> (&fk)[2]) __attribute__((always_inline)) {
    const int kc = 16 * r + n;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      // positions 32 s2 + 4g .. +3 and 32 s2 + 16 + 4g .. +3: units 4 s2 + g / 2 and + 2, half g & 1
      const int u = 4 * s2 + (g >> 1), h8 = 8 * (g & 1);
      fk[s2].load4x2(OKT + K::kt_unit(kc, u) + h8, OKT + K::kt_unit(kc, u + 2) + h8);
    }
  };

  // R = V - (K o gamma) (S_hi + S_lo)  (the operand tile holds -(K o gamma)); O = (Q o gamma) S_hi
  f32x4_t Rr[NB], O[NB];
  Frag<bf16_t> fk[2][NB], fq[2][NB];
  ld_kq(0, fk[0], fq[0]);
#pragma unroll
  for (int I = 0; I < NB; ++I) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (kV && !G2) {
        Rr[I][e] = bf16_to_f32(*(const uint16_t*)(vb + (16 * I + e) * K::RS_V));
      } else {
        Rr[I][e] = 0.f;  // (Gated DeltaNet-2: w o V is added after the products below)
      }
    }
    O[I] = zero4();
  }
  fence_sched();
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (ks + 1 < KS) ld_kq(ks + 1, fk[(ks + 1) & 1], fq[(ks + 1) & 1]);
    fence_sched();
    // S as hi / lo B fragments (k-slots: rows 32 ks + 4g + e and 32 ks + 16 + 4g + e)
    Frag<bf16_t> bsh, bsl;
    split_acc(S[2 * ks], S[2 * ks + 1], bsh, bsl);
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      mma(Rr[I], fk[ks & 1][I], bsh);
      if constexpr (kOut) mma(O[I], fq[ks & 1][I], bsh);
      mma(Rr[I], fk[ks & 1][I], bsl);
    }
    fence_sched();
  }

  if constexpr (kV && G2) {  // R += w o V: the write gates' loads have had the products' time
#pragma unroll
    for (int I = 0; I < NB; ++I)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Rr[I][e] += bf16_to_f32(*(const uint16_t*)(vb + (16 * I + e) * K::RS_V)) * wf[4 * I + e];
      }
  }

  // Delta = M~ R over the lower blocks (I, s2) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1):
  // M~_hi R_hi + M~_hi R_lo + M~_lo R_hi
  Frag<bf16_t> fh[6], fl[6];
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    ld_rec(RL::MH, j, fh[j]);
    ld_rec(RL::ML, j, fl[j]);
  }
  fence_sched();
  Frag<bf16_t> brh[2], brl[2];
  split_acc(Rr[0], Rr[1], brh[0], brl[0]);
  split_acc(Rr[2], Rr[3], brh[1], brl[1]);
  f32x4_t D[NB];
#pragma unroll
  for (int I = 0; I < NB; ++I) D[I] = zero4();
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    const int I = blk_I(j), s2 = blk_s(j);
    mma(D[I], fh[j], brh[s2]);
    mma(D[I], fh[j], brl[s2]);
    mma(D[I], fl[j], brh[s2]);
  }
  // the readout block's and the first state row block's operands, in flight meanwhile
  Frag<bf16_t> fa[6], ft[2][2];
  if constexpr (kOut) {
#pragma unroll
    for (int j = 0; j < 6; ++j) ld_rec(RL::A, j, fa[j]);
  }
  ld_kt(0, ft[0]);
  fence_sched();

  // O += A Delta_hi
  Frag<bf16_t> bdh[2], bdl[2];
  split_acc(D[0], D[1], bdh[0], bdl[0]);
  split_acc(D[2], D[3], bdh[1], bdl[1]);
  if constexpr (kOut) {
#pragma unroll
    for (int j = 0; j < 6; ++j) mma(O[blk_I(j)], fa[j], bdh[blk_s(j)]);
  }

  // S <- diag(gamma_last) S + (K o rho)^T (Delta_hi + Delta_lo)
  float4 gl[2];
  gl[0] = *(const float4*)(OG + 4 * g);
#pragma unroll
  for (int r = 0; r < DK / 16; ++r) {
    if (r + 1 < DK / 16) {
      gl[(r + 1) & 1] = *(const float4*)(OG + 16 * (r + 1) + 4 * g);
      ld_kt(r + 1, ft[(r + 1) & 1]);
    }
    const float4 c = gl[r & 1];
    fence_sched();
    if constexpr (CPX) {  // rows (2p, 2p+1) are one complex coordinate, turned by gamma_last
      const float s0 = S[r][0], s1 = S[r][1], s2 = S[r][2], s3 = S[r][3];
      S[r][0] = c.x * s0 - c.y * s1;
      S[r][1] = c.y * s0 + c.x * s1;
      S[r][2] = c.z * s2 - c.w * s3;
      S[r][3] = c.w * s2 + c.z * s3;
    } else {
      S[r][0] *= c.x;
      S[r][1] *= c.y;
      S[r][2] *= c.z;
      S[r][3] *= c.w;
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      mma(S[r], ft[r & 1][s2], bdh[s2]);
      mma(S[r], ft[r & 1][s2], bdl[s2]);
    }
    fence_sched();
  }

  // O over this wave's own (already consumed) v columns
  if constexpr (kOut) {
#pragma unroll
    for (int I = 0; I < NB; ++I)
#pragma unroll
      for (int e = 0; e < 4; e += 2) {  // rows e and e + 1 rounded by one conversion
        const uint32_t w = pack_bf16x2(O[I][e], O[I][e + 1]);
        *(uint16_t*)(vb + (16 * I + e) * K::RS_V) = (uint16_t)w;
        *(uint16_t*)(vb + (16 * I + e + 1) * K::RS_V) = (uint16_t)(w >> 16);
      }
  }
}

}  // namespace

// The walk of one workgroup: `bid` numbers it among the launch's workgroups of this mode;
// ops_a ... v_b are its LDS buffers (distinct __shared__ arrays of the calling kernel).
// Chains: the (b, h) pairs, times nsub segments seg_lo ... seg_lo + nsub - 1 of the nseg
// segments of segc chunks each when the walk is split.
template <int DK, int VT, bool G2, bool CPX, int MODE>
__device__ __forceinline__ void walk_body(
    char* ops_a, char* ops_b, char* rec_a, char* rec_b, char* v_a, char* v_b, const int bid,
    const char* __restrict__ ws, const void* __restrict__ gq, const void* __restrict__ gk,
    const void* __restrict__ galpha, const void* __restrict__ gerase, const void* __restrict__ gv,
    const void* __restrict__ gw, const float* s0, void* __restrict__ go, float* sT, int Tlen, int H, int DV,
    int BH, const int* __restrict__ cu, const int* __restrict__ cbase, int gmax, int nseg, int segc, int flags,
    int nsub, int seg_lo, int c0, int c1) {
  using K = WCfg<DK, VT>;
  using RL = typename K::RL;
  using R = Raw<bf16_t>;
  using G = Gp2<CPX>;
  constexpr int NW = K::NW;
  constexpr int NP = K::NP;
  constexpr int NT = K::NT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool producer = wave >= NW;
  const int pw = wave - NW;  // producer index
  const int g = lane >> 4;
  const int n = lane & 15;
  const int NVT = DV / VT;
  // the value tiles of one chain (or segment) read the same records and share an XCD
  const int BHs = BH * nsub;
  int bhs, vt;
  {
    if (NVT > 1 && (BHs & 7) == 0) {
      const int r = bid >> 3;
      vt = r % NVT;
      bhs = (r / NVT) * 8 + (bid & 7);
    } else {
      bhs = bid / NVT;
      vt = bid % NVT;
    }
  }
  const int bh = bhs / nsub, seg = seg_lo + (bhs - bh * nsub);
  // the sequence this workgroup walks: batch row b of length Tlen, or (packed varlen
  // batch, cu != NULL) sequence b = bh / H of length cu[b + 1] - cu[b]
  const int b = bh / H, h = bh % H;
  const int v0 = vt * VT;
  size_t sbase;
  int slen;
  const char* rec0;
  if (cu) {
    sbase = (size_t)cu[b];
    slen = cu[b + 1] - cu[b];
    rec0 = ws + ((size_t)h * gmax + cbase[b]) * RL::BYTES;
  } else {
    sbase = (size_t)b * Tlen;
    slen = Tlen;
    rec0 = ws + (size_t)bh * ((Tlen + C - 1) / C) * RL::BYTES;
  }
  if (nseg > 1) {  // this workgroup's segment: c0 chunks, c1 chunks, then segc chunks each
    const int cb = seg == 0 ? 0 : seg == 1 ? c0 : c0 + c1 + (seg - 2) * segc;
    const int cl = seg == 0 ? c0 : seg == 1 ? c1 : segc;
    rec0 += (size_t)cb * RL::BYTES;
    sbase += (size_t)cb * C;
    slen = max(0, min(slen - cb * C, cl * C));
  }
  const int nchunks = (slen + C - 1) / C;
  const size_t sidx = (size_t)bh * nseg + seg;  // start / end state index: (b, h), or (b, h, segment)
  constexpr bool kOut = MODE == kWalkFull;    // outputs formed and stored
  constexpr bool kV = MODE != kWalkTransfer;  // v read
  const bool zero_v = !kV || (flags & kSegZeroV) != 0, no_out = !kOut || (flags & kSegNoOut) != 0;

  f32x4_t S[DK / 16];
#pragma unroll
  for (int r = 0; r < DK / 16; ++r) S[r] = zero4();
  if ((flags & kSegIdentity) && !producer) {  // S = I (the walk then yields the transfer P)
#pragma unroll
    for (int r = 0; r < DK / 16; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[r][e] = 16 * r + 4 * g + e == v0 + 16 * wave + n ? 1.f : 0.f;
  } else if (s0 && !producer) {
    const size_t si0 = (flags & kSegS0Head) ? (size_t)bh : sidx;
#pragma unroll
    for (int r = 0; r < DK / 16; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[r][e] = s0[(si0 * DK + 16 * r + 4 * g + e) * DV + v0 + 16 * wave + n];
  }

  // ---- producer side: lane pt holds one gate item (4 rows x 8 channels) when pt < NITEM
  const int pt = tid - NW * 64;
  const bool has_item = producer && pt < K::NITEM;
  // Transfers of producer wave pw per step: ND DMA instructions (1 KiB each) and NS output
  // stores.  DMA index i < N_DMA_V is v unit i, the rest are record units; indices past
  // the last repeat the last record unit (the same bytes to the same place).  Output unit
  // j of the wave is v unit pw + NP j, which this wave reads out before its own DMA
  // overwrites it, so no workgroup barrier sits between the two.  The counts are the same
  // on every step: the tail repeats the last chunk's transfers into buffers nobody reads,
  // and the stores of a step with nothing to write are dropped by the buffer range check.
  // The vector-memory counter, which retires in issue order, then holds a known number of
  // operations at every wait (the barrier's and the compiler's).
  constexpr int NVU = kV ? K::N_DMA_V : 0;  // v units moved per step
  constexpr int NU = NVU + K::N_DMA_REC;
  // a wave's unit slots: NVJ v slots (unit pw + NP j), then NRJ record slots (unit
  // pw + NP j' of the record, the last one repeated past the end)
  constexpr int NVJ = (NVU + NP - 1) / NP;
  constexpr int NRJ = (K::N_DMA_REC + NP - 1) / NP;
  constexpr int ND = NVJ + NRJ;
  constexpr int NS = (K::N_DMA_V + NP - 1) / NP;
  static_assert(NS >= 1 && NS <= 2, "one or two output units per producer wave");
  typedef uint32_t u32x4o __attribute__((ext_vector_type(4)));
  u32x4o ov0 = {0u, 0u, 0u, 0u}, ov1 = ov0;
  // the wave's output units of the tile staged in `vv` into registers (then lgkmcnt(0):
  // the DMA that follows may overwrite them)
  auto read_o = [&](const char* vv) __attribute__((always_inline)) {
    ov0 = *(const u32x4o*)(vv + (min(pw, K::N_DMA_V - 1) * 64 + lane) * 16);
    if constexpr (NS > 1) ov1 = *(const u32x4o*)(vv + (min(pw + NP, K::N_DMA_V - 1) * 64 + lane) * 16);
#ifndef KDA_HOST_PASS
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
#endif
  };
  // ... and out to o rows of chunk c (when `any`): rows past the end fall outside the
  // buffer range and are dropped
  auto write_o = [&](int c, bool any) __attribute__((always_inline)) {
    const int t0 = max(c, 0) * C;
    const int nv = min(C, slen - t0);
    const uint32_t rs = (uint32_t)H * DV * 2;
    // (the descriptor fields are wave-uniform: made explicit, or the compiler loops over
    // lanes to build a scalar descriptor)
    const uint64_t ba = (uint64_t)((char*)go + ((sbase + t0) * H + h) * DV * 2 + (size_t)v0 * 2);
    char* base = (char*)(((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(ba >> 32)) << 32) |
                         (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ba));
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int x = pw + NP * j;
      const int num = __builtin_amdgcn_readfirstlane(any && x < K::N_DMA_V && nv > 0 ? (int)((nv - 1) * rs) + VT * 2 : 0);
      const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, num, 0x00020000);
      const int sl = min(x, K::N_DMA_V - 1) * 64 + lane;
      const int row = sl / K::UPR, u = (sl % K::UPR) ^ K::vsw(row);
      __builtin_amdgcn_raw_buffer_store_b128(j == 0 ? ov0 : ov1, rsrc, (int)(row * rs) + u * 16, 0, 0);
    }
  };
  // The record and v tile of a chunk move through the producers' registers: unit j of
  // wave pw (16 bytes per lane, 1 KiB per wave) is loaded two steps before use and written
  // to LDS one step before use, so a load has a whole step to land and the step barrier
  // waits for LDS writes only.  (With DMA into LDS the barrier must wait for the DMA, and
  // with it every load issued before it.)  Unit i < NVU is v unit i, the rest record
  // units; the v tile comes from the record itself when v is read as zero (the bytes go
  // unused, the stores write zeros).
  static_assert(ND <= 8, "unit registers");
  typedef uint32_t u32x16u __attribute__((ext_vector_type(16)));
  struct USet {
    u32x16u lo, hi;  // units 0..3, 4..7
  };
  USet us0, us1;
  auto load_units = [&](int c, USet& us) __attribute__((always_inline)) {
    const char* rc = rec0 + (size_t)c * RL::BYTES;
    const int t0 = c * C;
#pragma unroll
    for (int j = 0; j < ND; ++j) {
      const char* src;
      if (j < NVJ) {  // v slot (when the wave has no unit there, a record unit again)
        const int i = pw + NP * j;
        const int sl = min(i, K::N_DMA_V - 1) * 64 + lane;
        const int row = sl / K::UPR, u = (sl % K::UPR) ^ K::vsw(row);
        const size_t gr = (sbase + min(t0 + row, slen - 1)) * H + h;
        src = zero_v ? rc + lane * 16 : (const char*)gv + (gr * DV + v0) * 2 + (size_t)u * 16;
        if (NVU % NP != 0 && i >= NVU) src = rc + lane * 16;
      } else {
        const int r = min(pw + NP * (j - NVJ), K::N_DMA_REC - 1);
        src = rc + r * 1024 + lane * 16;
      }
      const uint4 x = *(const uint4*)src;
      u32x16u& d = j < 4 ? us.lo : us.hi;
      const int o = 4 * (j & 3);
      d[o] = x.x;
      d[o + 1] = x.y;
      d[o + 2] = x.z;
      d[o + 3] = x.w;
    }
  };
  // (v rows at or past `nvrow`, the rows of the chunk that exist, or all of them when v is
  // read as zero, are stored as zeros: the compute waves read the tile unmasked)
  auto store_units = [&](const USet& us, char* rec_dst, char* v_dst, int nvrow) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < ND; ++j) {
      char* dst;
      bool zero = false;
      if (j < NVJ) {
        const int i = pw + NP * j;
        dst = v_dst + i * 1024;
        const int row = (min(i, K::N_DMA_V - 1) * 64 + lane) / K::UPR;
        zero = row >= nvrow;
        if (NVU % NP != 0 && i >= NVU) {  // (the record's first unit again)
          dst = rec_dst;
          zero = false;
        }
      } else {
        dst = rec_dst + min(pw + NP * (j - NVJ), K::N_DMA_REC - 1) * 1024;
      }
      const u32x16u& d = j < 4 ? us.lo : us.hi;
      const int o = 4 * (j & 3);
      lds_st128(dst + lane * 16, zero ? 0u : d[o], zero ? 0u : d[o + 1], zero ? 0u : d[o + 2], zero ? 0u : d[o + 3]);
    }
  };
  auto v_rows = [&](int c) { return zero_v ? 0 : slen - c * C; };
  // Gate items: lane (rg, cg) = (lane & 15, lane >> 4) of producer wave pw holds rows
  // 4 rg .. 4 rg + 3 of channels c0 = 32 pw + 8 cg .. c0 + 7 (one 16-byte vector per row
  // and tensor: few, wide loads).  The 16 row groups of a channel group are the 16 lanes of
  // one DPP row, so the gate products across row groups are 4-step scans along that row.
  // The raw rows sit in two register sets that alternate by chunk: chunk c + 2's inputs
  // load into the set chunk c vacated while chunk c + 1's are turned into operands, so a
  // load has a whole step to land.  Rows past the end are clamped to the last row
  // (unconditional loads) and given gate 1 when used.  (Native vectors, not arrays: arrays
  // captured by the lambdas stay in scratch memory.)
  typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  struct PSet {
    u32x16 q, k, a;  // dword 4 j + p: row 4 rg + j, channels c0 + 2p, c0 + 2p + 1
    int nrow;           // rows of the loaded chunk that exist
  };
  PSet ps0, ps1;
  ps0.nrow = ps1.nrow = 0;
  // row j of the lane's row group (4 rg + j) of chunk c into `ps`
  auto load_row = [&](int c, PSet& ps, int j) __attribute__((always_inline)) {
    // the lane's row group and channels from an opaque copy of the thread index: the row
    // offsets are then recomputed per chunk instead of hoisted out of the loop and spilled
    // (a reload would wait for every load in flight)
    int t = threadIdx.x - NW * 64;
    asm volatile("" : "+v"(t));
    const int rg = t & 15, c0 = 32 * (t >> 6) + 8 * ((t >> 4) & 3);
    const int t0 = c * C;
    const size_t base = ((sbase + t0) * H + h) * DK * 2;
    const uint32_t rs = (uint32_t)H * DK * 2;
    ps.nrow = slen - t0;
    const uint32_t off = (uint32_t)min(4 * rg + j, ps.nrow - 1) * rs + 2 * c0;
    if constexpr (kOut) {
      const u32x4v q4 = *(const u32x4v*)((const char*)gq + base + off);
#pragma unroll
      for (int p = 0; p < 4; ++p) ps.q[4 * j + p] = q4[p];
    }
    const u32x4v k4 = *(const u32x4v*)((const char*)gk + base + off);
    const u32x4v a4 = *(const u32x4v*)((const char*)galpha + base + off);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      ps.k[4 * j + p] = k4[p];
      ps.a[4 * j + p] = a4[p];
    }
  };
  auto load_rows = [&](int c, PSet& ps) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) load_row(c, ps, j);
  };
  // the operands of the chunk loaded in `ps` into `ops`, bf16: Q o gamma and -(E o gamma)
  // rows (E: k, or b o k for Gated DeltaNet-2), (K o rho)^T columns, gamma_last
  // hook(j), j = 0..3, runs at four points spread over the work (the step's transfers,
  // issued in parts between the arithmetic)
  auto form = [&](const PSet& ps, char* ops, int cf, auto&& hook) __attribute__((always_inline)) {
    int t = threadIdx.x - NW * 64;
    asm volatile("" : "+v"(t));
    const int rg = t & 15, c0 = 32 * (t >> 6) + 8 * ((t >> 4) & 3);
    // (Gated DeltaNet-2) the erase gates of chunk cf, the one being formed: one register
    // set, loaded here and first used after the gate scans
    u32x16 ev;
    if constexpr (G2) {
      const size_t base = ((sbase + cf * C) * H + h) * DK * 2;
      const uint32_t rs = (uint32_t)H * DK * 2;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t off = (uint32_t)min(4 * rg + j, slen - cf * C - 1) * rs + 2 * c0;
        const u32x4v e4 = *(const u32x4v*)((const char*)gerase + base + off);
#pragma unroll
        for (int p = 0; p < 4; ++p) ev[4 * j + p] = e4[p];
      }
    }
    hook(0);
    constexpr uint32_t kOne = CPX ? 0x00003F80u : R::kOneWord;
    // gates (channel pair p of row j), the products inside the row group: prefix P (rows
    // up to j) and exclusive suffix B (rows after j), then across the groups
    G al[4][4], P[4][4], B[4][4], X[4], Y[4], tot[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int p = 0; p < 4; ++p) R::unpack(4 * rg + j < ps.nrow ? ps.a[4 * j + p] : kOne, al[j][p].x, al[j][p].y);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      P[0][p] = al[0][p];
      P[1][p] = P[0][p] * al[1][p];
      P[2][p] = P[1][p] * al[2][p];
      P[3][p] = P[2][p] * al[3][p];
      B[3][p] = G::one();
      B[2][p] = al[3][p];
      B[1][p] = al[2][p] * al[3][p];
      B[0][p] = al[1][p] * B[1][p];
    }
    // inclusive scans of the group totals along the DPP row: I (groups up to rg), J
    // (groups from rg on); X, Y their exclusive forms
    if constexpr (!CPX) {
      float I[8], J[8];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        I[2 * p] = J[2 * p] = P[3][p].x;
        I[2 * p + 1] = J[2 * p + 1] = P[3][p].y;
      }
      row_scan16(I, J);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        tot[p] = G{I[2 * p], I[2 * p + 1]};
        X[p] = dpp_fill<G, 0x111>(tot[p]);
        Y[p] = dpp_fill<G, 0x101>(G{J[2 * p], J[2 * p + 1]});
      }
    } else {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        G I = P[3][p], J = P[3][p];
        I = I * dpp_fill<G, 0x111>(I);
        J = J * dpp_fill<G, 0x101>(J);
        I = I * dpp_fill<G, 0x112>(I);
        J = J * dpp_fill<G, 0x102>(J);
        I = I * dpp_fill<G, 0x114>(I);
        J = J * dpp_fill<G, 0x104>(J);
        I = I * dpp_fill<G, 0x118>(I);
        J = J * dpp_fill<G, 0x108>(J);
        X[p] = dpp_fill<G, 0x111>(I);
        Y[p] = dpp_fill<G, 0x101>(J);
        tot[p] = I;
      }
    }
    typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
    u32x2v kt[4][2];  // (K o rho)^T: channel 2p + c2, rows (4rg, 4rg+1), (4rg+2, 4rg+3)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j > 0) hook(j);
      uint32_t wq[4], wk[4];
      float kr[4][2];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const G gm = X[p] * P[j][p], rh = Y[p] * B[j][p];
        float k0, k1, e0, e1, r0, r1;
        R::unpack(ps.k[4 * j + p], k0, k1);
        e0 = k0;
        e1 = k1;
        if constexpr (G2) {
          float b0, b1;
          R::unpack(ev[4 * j + p], b0, b1);
          e0 *= b0;
          e1 *= b1;
        }
        if constexpr (kOut) {
          float q0, q1;
          R::unpack(ps.q[4 * j + p], q0, q1);
          gm.row(q0, q1, r0, r1);
          wq[p] = pack_bf16x2(r0, r1);
        }
        gm.row(e0, e1, r0, r1);
        wk[p] = pack_bf16x2(-r0, -r1);
        rh.col(k0, k1, kr[p][0], kr[p][1]);
      }
      const int row = 4 * rg + j;
      if constexpr (kOut) lds_st128(ops + K::OFF_Q + row * K::RS_Q + 2 * c0, wq[0], wq[1], wq[2], wq[3]);
      lds_st128(ops + K::OFF_K + row * K::RS_Q + 2 * c0, wk[0], wk[1], wk[2], wk[3]);
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const float v = kr[p][c2];
          if (j == 0) kt[p][c2][0] = __float_as_uint(v);
          if (j == 1) kt[p][c2][0] = pack_bf16x2(__uint_as_float(kt[p][c2][0]), v);
          if (j == 2) kt[p][c2][1] = __float_as_uint(v);
          if (j == 3) kt[p][c2][1] = pack_bf16x2(__uint_as_float(kt[p][c2][1]), v);
        }
    }
    char* ktb = ops + K::OFF_KT;
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int ch = c0 + 2 * p + c2;
        lds_st64(ktb + K::kt_unit(ch, rg >> 1) + 8 * (rg & 1), __uint_as_float(kt[p][c2][0]),
                 __uint_as_float(kt[p][c2][1]));
      }
    if (rg == 15) {  // gamma_last: the inclusive product over every row group
      float* og = (float*)(ops + K::OFF_G) + c0;
      lds_st128(og, __float_as_uint(tot[0].x), __float_as_uint(tot[0].y), __float_as_uint(tot[1].x),
                __float_as_uint(tot[1].y));
      lds_st128(og + 4, __float_as_uint(tot[2].x), __float_as_uint(tot[2].y), __float_as_uint(tot[3].x),
                __float_as_uint(tot[3].y));
    }
  };

  // (compute waves, G2) the write gate of this lane's rows 16 I + 4 g + e and column of
  // chunk c, rows past the end clamped to the last row (their v rows read as zero)
  float wf[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) wf[i] = 0.f;
  auto load_w = [&](int c) __attribute__((always_inline)) {
    const int t0 = c * C, col = v0 + 16 * wave + n;
#pragma unroll
    for (int I = 0; I < NB; ++I)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const size_t row = sbase + min(t0 + 16 * I + 4 * g + e, slen - 1);
        wf[4 * I + e] = bf16_to_f32(((const uint16_t*)gw)[(row * H + h) * DV + col]);
      }
  };

  // The two roles run separate loops (so the compiler sees their registers as never live
  // at once); both pass the same barriers: one per chunk, and one at the end.
  // Step c: the compute waves walk chunk c from buffers P (operands, record, v tile); the
  // producers store chunk c - 1's outputs out of buffers Q, stream chunk c + 1's record and v
  // tile into Q, build its operands there, and load chunk c + 2's inputs.
  if (producer) {
    // (items: whether the wave holds gate items, a compile-time constant so that no
    // branch around a transfer blurs the counts)
    auto run = [&](auto items) __attribute__((always_inline)) {
      constexpr bool kItems = decltype(items)::value;
      const int last = nchunks - 1;
      load_units(0, us0);
      if constexpr (kItems) load_rows(0, ps0);
      load_units(min(1, last), us1);
      if constexpr (kItems) load_rows(min(1, last), ps1);
      if constexpr (kOut) write_o(0, false);  // (issues the step's store count; writes nothing)
      store_units(us0, rec_a, v_a, v_rows(0));
      if constexpr (kItems) form(ps0, ops_a, 0, [](int) {});
      // step c: the outputs of chunk c - 1 out of buffers Q, chunk c + 2's rows into the
      // register set chunk c vacated (psN) while chunk c + 1's operands are formed from
      // psP into Q, then chunk c + 1's record and v tile (loaded a step ago) into Q, and
      // chunk c + 2's units into usN.  The barrier waits for the LDS writes only: a load
      // issued in step c is first needed in step c + 1, and the compute waves never wait
      // for one.
      auto pstep = [&](int c, PSet& psP, PSet& psN, USet& usP, USet& usN, char* opsQ, char* recQ, char* vQ)
          __attribute__((always_inline)) {
        lds_barrier_only();
        if constexpr (kOut) read_o(vQ);
        fence_sched();
        if constexpr (kOut) write_o(c - 1, c > 0 && !no_out);
        fence_sched();
        if constexpr (kItems) {
          const int cl = min(c + 2, last);
          form(psP, opsQ, min(c + 1, last), [&](int j) __attribute__((always_inline)) {
            fence_sched();
            load_row(cl, psN, j);
            fence_sched();
          });
        }
        fence_sched();
        store_units(usP, recQ, vQ, v_rows(min(c + 1, last)));
        fence_sched();
        load_units(min(c + 2, last), usN);
      };
      for (int chunk = 0; chunk < nchunks; chunk += 2) {
        pstep(chunk, ps1, ps0, us1, us0, ops_b, rec_b, v_b);
        if (chunk + 1 >= nchunks) break;
        pstep(chunk + 1, ps0, ps1, us0, us1, ops_a, rec_a, v_a);
      }
      full_barrier();
      if constexpr (kOut) {
        read_o((last & 1) ? v_b : v_a);
        write_o(last, !no_out);
      }
    };
    if (nchunks > 0) {
      if (has_item)
        run(BoolC<true>{});
      else
        run(BoolC<false>{});
    }
  } else {
    if (G2 && !zero_v && nchunks > 0) load_w(0);
    auto cstep = [&](int c, const char* opsP, const char* recP, char* vP) __attribute__((always_inline)) {
      // chunk c landed and its operands are in place.  (The compute waves' own memory
      // operations are only the write-gate loads, which the walk waits for where it uses
      // them, after the state products: the barrier does not wait for them.)
      lds_barrier_only();
      walk_chunk<DK, VT, G2, CPX, MODE>(opsP, recP, vP, wf, S, wave, g, n);
      if (G2 && !zero_v && c + 1 < nchunks) load_w(c + 1);
    };
    for (int chunk = 0; chunk < nchunks; chunk += 2) {
      cstep(chunk, ops_a, rec_a, v_a);
      if (chunk + 1 >= nchunks) break;
      cstep(chunk + 1, ops_b, rec_b, v_b);
    }
    if (nchunks > 0) lds_barrier_only();  // the last outputs are staged
  }

  const bool last_only = (flags & kSegLastOnly) != 0;
  if (sT && !producer && (!last_only || seg == nseg - 1)) {
    const size_t oi = last_only ? (size_t)bh : (flags & kSegEndNext) ? sidx + 1 : sidx;
#pragma unroll
    for (int r = 0; r < DK / 16; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) sT[(oi * DK + 16 * r + 4 * g + e) * DV + v0 + 16 * wave + n] = S[r][e];
  }
}

#define KDA_WALK_LDS(K, RL)                              \
  __shared__ __align__(16) char ops_a[K::OPS];           \
  __shared__ __align__(16) char ops_b[K::OPS];           \
  __shared__ __align__(16) char rec_a[RL::DMA];          \
  __shared__ __align__(16) char rec_b[RL::DMA];          \
  __shared__ __align__(16) char v_a[K::V_BYTES];         \
  __shared__ __align__(16) char v_b[K::V_BYTES];

// One walk per workgroup.  Separate LDS objects per buffer, so that reads of one buffer
// are not ordered behind the loads (or the operand stores) still filling the other.
template <int DK, int VT, bool G2, bool CPX, int MODE>
__global__ __launch_bounds__((VT / 16 + 4) * 64) void chunk_walk_kernel(
    const char* __restrict__ ws, const void* __restrict__ gq, const void* __restrict__ gk,
    const void* __restrict__ galpha, const void* __restrict__ gerase, const void* __restrict__ gv,
    const void* __restrict__ gw, const float* s0, void* __restrict__ go, float* sT, int Tlen, int H, int DV,
    int BH, const int* __restrict__ cu, const int* __restrict__ cbase, int gmax, int nseg, int segc, int flags,
    int nsub, int seg_lo, int c0, int c1) {
  using K = WCfg<DK, VT>;
  using RL = typename K::RL;
  KDA_WALK_LDS(K, RL)
  walk_body<DK, VT, G2, CPX, MODE>(ops_a, ops_b, rec_a, rec_b, v_a, v_b, blockIdx.x, ws, gq, gk, galpha, gerase, gv,
                                   gw, s0, go, sT, Tlen, H, DV, BH, cu, cbase, gmax, nseg, segc, flags, nsub, seg_lo,
                                   c0, c1);
}

// A launch of a split walk over nseg segments (d_k = 128, 64 columns) that runs two walks
// side by side: the first `nfirst` workgroups walk segment seg_first in full (outputs
// stored) from its start state (S_0 indexed by (b, h) for segment 0, else Sst), writing
// the end state to Sst as segment seg_first + 1's start; the others run MODE2 (end states
// from zero, or transfers from the identity) over segments seg_lo ... seg_lo + nsub - 1,
// writing to out2 (d_v2 columns per state).  Segments 0 and 1 are walked this way, one in
// each of the first two launches, so neither needs an end state from zero nor a transfer.
template <bool G2, bool CPX, int MODE2>
__global__ __launch_bounds__((64 / 16 + 4) * 64) void chunk_walk_pair_kernel(
    const char* __restrict__ ws, const void* __restrict__ gq, const void* __restrict__ gk,
    const void* __restrict__ galpha, const void* __restrict__ gerase, const void* __restrict__ gv,
    const void* __restrict__ gw, const float* s_first, void* __restrict__ go, float* Sst, float* out2, int Tlen,
    int H, int DV, int DV2, int BH, int nseg, int segc, int c0, int c1, int nfirst, int seg_first, int flags2,
    int nsub, int seg_lo) {
  using K = WCfg<128, 64>;
  using RL = typename K::RL;
  KDA_WALK_LDS(K, RL)
  const int bid = blockIdx.x;
  if (bid < nfirst)
    walk_body<128, 64, G2, CPX, kWalkFull>(ops_a, ops_b, rec_a, rec_b, v_a, v_b, bid, ws, gq, gk, galpha, gerase,
                                           gv, gw, s_first, go, Sst, Tlen, H, DV, BH, nullptr, nullptr, 0, nseg, segc,
                                           (seg_first == 0 ? kSegS0Head : 0) | kSegEndNext, 1, seg_first, c0, c1);
  else
    walk_body<128, 64, G2, CPX, MODE2>(ops_a, ops_b, rec_a, rec_b, v_a, v_b, bid - nfirst, ws, gq, gk, galpha, gerase,
                                       gv, gw, nullptr, go, out2, Tlen, H, DV2, BH, nullptr, nullptr, 0, nseg, segc,
                                       flags2, nsub, seg_lo, c0, c1);
}
#undef KDA_WALK_LDS

// Start states of the segments of a split walk: Sst[b, h, g + 1] = P_g Sst[b, h, g] + B_g
// for g = g0 ... G - 2, from Sst[b, h, g0] (g0 > 0: segment g0's start, already written by
// the full walk of segment g0 - 1; g0 = 0: S_0 or zero, copied there), where B_g is segment g's end state from a zero
// start and P_g (d_k x d_k) its end state from the identity with v = 0 -- the affine
// transfer of a block of the SFDA page ("Principales Contribuciones", item 3), applied
// segment by segment.  One workgroup per (b, h, 16 state columns), fp32: P_g is staged in
// LDS (P_(g+1) loads into registers while segment g is applied) and each thread carries
// DK / 32 rows of the product as independent sums.
constexpr int kScanThreads = 512;

template <int DK>
__global__ __launch_bounds__(kScanThreads) void seg_scan_kernel(const float* __restrict__ s0, const float* __restrict__ P,
                                                     const float* __restrict__ Bst, float* __restrict__ Sst, int G,
                                                     int DV, int g0) {
  constexpr int LP = DK + 4;  // P rows in LDS: four rows a wave reads at once on distinct banks
  __shared__ float sP[DK * LP];
  __shared__ float sS[DK][17];
  const int nsl = DV / 16, bh = blockIdx.x / nsl, c0 = (blockIdx.x % nsl) * 16;
  constexpr int NR = kScanThreads / 16;  // row groups
  const int tid = threadIdx.x, c = tid & 15, r0 = tid >> 4;  // rows r0 + NR j
  constexpr int RJ = DK / NR;
  constexpr int NV4 = DK * DK / 4 / kScanThreads;  // float4 of P per thread
  const size_t SS = (size_t)DK * DV;
  // (a native vector, not an array: an array carried across the loop stays in scratch)
  typedef float pvec __attribute__((ext_vector_type(4 * NV4)));
  pvec pf;
  auto load_p = [&](int gi) __attribute__((always_inline)) {
    const float4* src = (const float4*)(P + ((size_t)bh * G + gi) * DK * DK);
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
      const float4 v = src[tid + kScanThreads * i];
      pf[4 * i] = v.x;
      pf[4 * i + 1] = v.y;
      pf[4 * i + 2] = v.z;
      pf[4 * i + 3] = v.w;
    }
  };
  auto store_p = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
      const int x = tid + kScanThreads * i, row = x / (DK / 4), col = 4 * (x % (DK / 4));
      *(float4*)(sP + row * LP + col) = make_float4(pf[4 * i], pf[4 * i + 1], pf[4 * i + 2], pf[4 * i + 3]);
    }
  };
  float* out0 = Sst + ((size_t)bh * G + g0) * SS;
#pragma unroll
  for (int j = 0; j < RJ; ++j) {
    const int r = r0 + NR * j;
    if (g0) {
      sS[r][c] = out0[(size_t)r * DV + c0 + c];
    } else {
      const float x = s0 ? s0[((size_t)bh * DK + r) * DV + c0 + c] : 0.f;
      sS[r][c] = x;
      out0[(size_t)r * DV + c0 + c] = x;
    }
  }
  if (G > g0 + 1) {
    load_p(g0);
    store_p();
  }
  for (int gi = g0; gi + 1 < G; ++gi) {
    __syncthreads();  // sP = P_gi, sS = the start state of segment gi
    if (gi + 2 < G) load_p(gi + 1);
    const float* Bg = Bst + ((size_t)bh * G + gi) * SS;
    float acc[RJ];
#pragma unroll
    for (int j = 0; j < RJ; ++j) acc[j] = Bg[(size_t)(r0 + NR * j) * DV + c0 + c];
#pragma unroll 4
    for (int k = 0; k < DK; ++k) {
      const float xk = sS[k][c];
#pragma unroll
      for (int j = 0; j < RJ; ++j) acc[j] += sP[(r0 + NR * j) * LP + k] * xk;
    }
    __syncthreads();
    if (gi + 2 < G) store_p();
    float* outg = Sst + ((size_t)bh * G + gi + 1) * SS;
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
      const int r = r0 + NR * j;
      sS[r][c] = acc[j];
      outg[(size_t)r * DV + c0 + c] = acc[j];
    }
  }
}

template <int DK, int VT, bool G2, bool CPX, int MODE = kWalkFull>
static void walk_launch(const ChunkArgs& a, const void* ws, int nblocks, int BH, int DV, const float* s0, float* sT,
                        int nseg, int segc, int flags, int nsub, int seg_lo, int c0 = 0, int c1 = 0) {
  using K = WCfg<DK, VT>;
  if (nblocks <= 0) return;
  hipLaunchKernelGGL((chunk_walk_kernel<DK, VT, G2, CPX, MODE>), dim3(nblocks), dim3(K::NT), 0, (hipStream_t)a.stream,
                     (const char*)ws, a.q, a.k, a.alpha, a.erase, a.v, a.write, s0, a.o, sT, a.T, a.H, DV, BH, a.cu,
                     a.ctab_base, a.gmax, nseg, segc, flags, nsub, seg_lo, c0, c1);
}

template <int DK, int VT, bool G2, bool CPX>
static hipError_t launch_walk_t(const ChunkArgs& a, const void* ws) {
  // varlen: one chain per (sequence, head): BH = n_seqs * H
  const int BHc = a.cu ? a.n_seqs * a.H : a.B * a.H;
  walk_launch<DK, VT, G2, CPX>(a, ws, BHc * (a.dv / VT), BHc, a.dv, a.s0, a.sT, 1, 0, 0, 1, 0);
  return hipGetLastError();
}

// The split walk (fixed-length batches at d_k = 128, few (b, h) chains, G >= 2 segments
// per chain): four launches, 64 value columns per workgroup, scratch after the records:
// B [BH G][d_k][d_v], P [BH G][d_k][d_k], segment start states [BH G][d_k][d_v] (index 0
// unused).  Segment 0 is walked in full from S_0 beside the end states of segments
// 2 ... G - 2, segment 1 in full from the start that gives beside their transfers; the
// scan then forms the starts of segments 3 ... G - 1 (the last segment's end state and
// transfer are never needed), and the last launch walks segments 2 ... G - 1 in full.
// Segment lengths of a split walk over NC chunks: segments 0 and 1 take c0 and c1 chunks,
// the others segc each (the last one what remains).  From G = 4 on, segment 0's full walk
// shares a launch with end-state walks and segment 1's with transfer walks, which take
// about 0.79 and 0.65 of a full walk's time per chunk (2.96 and 2.43 against 3.75 us per
// chunk at B1 H16 T128K), so segments 0 and 1 get 51/64 and 42/64 of segc and the
// workgroups of each launch end together.
static void split_lengths(int NC, int G, int& segc, int& c0, int& c1) {
  if (G <= 3) {
    segc = c0 = c1 = (NC + G - 1) / G;
    return;
  }
  segc = max(1, (int)((long)NC * 64 / ((long)(G - 2) * 64 + 51 + 42)));
  for (;; ++segc) {
    c0 = segc * 51 / 64;
    c1 = segc * 42 / 64;
    if (c0 + c1 + (long)(G - 2) * segc >= NC) break;
  }
}

template <bool G2, bool CPX>
static hipError_t launch_walk_split(const ChunkArgs& a, const void* ws, int G) {
  const int BH = a.B * a.H, NC = (a.T + C - 1) / C, tv = a.dv / 64;
  int segc, c0, c1;
  split_lengths(NC, G, segc, c0, c1);
  const size_t rec = (size_t)BH * NC * WalkRecord<128>::BYTES;
  float* Bst = (float*)((char*)ws + rec);
  float* P = Bst + (size_t)BH * G * 128 * a.dv;
  float* Sst = P + (size_t)BH * G * 128 * 128;
  const hipStream_t st = (hipStream_t)a.stream;
  const int nfirst = BH * tv, nmid = G > 3 ? G - 3 : 0;  // segments 2 ... G - 2
  // segment 0 in full; the end states of segments 2 ... G - 2 from a zero start
  hipLaunchKernelGGL((chunk_walk_pair_kernel<G2, CPX, kWalkState>), dim3(nfirst + BH * nmid * tv),
                     dim3(WCfg<128, 64>::NT), 0, st, (const char*)ws, a.q, a.k, a.alpha, a.erase, a.v, a.write, a.s0,
                     a.o, Sst, Bst, a.T, a.H, a.dv, a.dv, BH, G, segc, c0, c1, nfirst, 0, kSegNoOut, nmid, 2);
  if (G > 2) {
    // segment 1 in full; the transfers of segments 2 ... G - 2: the identity walked with
    // v = 0 (the write gate is then irrelevant)
    hipLaunchKernelGGL((chunk_walk_pair_kernel<G2, CPX, kWalkTransfer>), dim3(nfirst + BH * nmid * 2),
                       dim3(WCfg<128, 64>::NT), 0, st, (const char*)ws, a.q, a.k, a.alpha, a.erase, a.v, a.write, Sst,
                       a.o, Sst, P, a.T, a.H, a.dv, 128, BH, G, segc, c0, c1, nfirst, 1,
                       kSegNoOut | kSegZeroV | kSegIdentity, nmid, 2);
  }
  if (nmid > 0)
    hipLaunchKernelGGL(seg_scan_kernel<128>, dim3(BH * (a.dv / 16)), dim3(kScanThreads), 0, st, a.s0, P, Bst, Sst, G,
                       a.dv, 2);
  // segments 2 ... G - 1 from their start states (the last one writes the final state);
  // with G = 2, segment 1
  const int lo = G > 2 ? 2 : 1;
  walk_launch<128, 64, G2, CPX>(a, ws, BH * (G - lo) * tv, BH, a.dv, Sst, a.sT, G, segc, kSegLastOnly, G - lo, lo,
                                c0, c1);
  return hipGetLastError();
}

// KDA_STATE_SEG=0 keeps the single walk per chain, =G forces G segments (tuning aid)
static int state_seg_override() {
  static const int v = [] {
    const char* e = getenv("KDA_STATE_SEG");
    return e ? atoi(e) : -1;
  }();
  return v;
}

// The split costs three launches of G - 2 segments' walks of NC / G chunks at 64 columns
// per workgroup against one walk of NC chunks on narrower tiles (with half the compute
// units idle or fewer): G - 2 segments fill the compute units once per launch; the split
// is taken from G = 8 segments of at least 16 chunks.
int state_segments(int B, int T, int H, int dk, int dv, bool bf16) {
  if (!bf16 || dk != 128 || (dv != 64 && dv != 128)) return 1;
  const int NC = (T + C - 1) / C, o = state_seg_override();
  if (o >= 0) {
    const int G = min(o, NC / 16);
    return G >= 2 ? G : 1;
  }
  const long tiles = (long)B * H * (dv / 64);  // 64-column tiles of one walk per chain
  if (tiles <= 0 || tiles >= 256) return 1;
  const int G = min((int)((256 + tiles - 1) / tiles) + 2, NC / 16);  // at least 16 chunks per segment
  return G >= 8 ? G : 1;
}

size_t state_split_bytes(int B, int T, int H, int dk, int dv, bool bf16) {
  const int G = state_segments(B, T, H, dk, dv, bf16);
  if (G < 2) return 0;
  return (size_t)B * H * G * dk * (2 * (size_t)dv + dk) * sizeof(float);
}

// KDA_STATE_VT=16|32|64 pins the walk's value-tile width (tuning aid)
static int state_vt_override() {
  static const int v = [] {
    const char* e = getenv("KDA_STATE_VT");
    return e ? atoi(e) : 0;
  }();
  return v;
}

// Value-tile width: each workgroup walks the whole chunk chain of one (b, h, tile), so
// with few (b, h) pairs narrower tiles put more compute units on the chains (each tile
// rebuilds the same operands; the repeated reads hit in L2).
static int pick_walk_vt(const ChunkArgs& a) {
  const int o = state_vt_override();
  int vt;
  if (o == 16 || o == 32 || o == 64) {
    vt = o <= a.dv ? o : a.dv;
  } else {
    const long bh = (long)(a.cu ? a.n_seqs : a.B) * a.H;
    vt = bh * (a.dv / 64) >= 256 ? 64 : bh * (a.dv / 32) >= 256 ? 32 : 16;
  }
  return vt < 64 ? vt : 64;
}

template <int DK, bool G2, bool CPX>
static hipError_t launch_walk_vt(const ChunkArgs& a, const void* ws) {
  switch (pick_walk_vt(a)) {
    case 16: return launch_walk_t<DK, 16, G2, CPX>(a, ws);
    case 32: return launch_walk_t<DK, 32, G2, CPX>(a, ws);
    default: return launch_walk_t<DK, 64, G2, CPX>(a, ws);
  }
}

template <bool G2, bool CPX>
static hipError_t launch_walk_g(const ChunkArgs& a, const void* ws) {
  if (!a.cu) {
    const int G = state_segments(a.B, a.T, a.H, a.dk, a.dv, true);
    if (G >= 2) return launch_walk_split<G2, CPX>(a, ws, G);
  }
  return a.dk == 64 ? launch_walk_vt<64, G2, CPX>(a, ws) : launch_walk_vt<128, G2, CPX>(a, ws);
}

// bf16 walk over the records of kda_records.hip (d_k in {64, 128})
hipError_t launch_walk(const ChunkArgs& a, const void* ws) {
  if ((a.cu ? a.n_seqs : a.B) * a.H == 0) return hipSuccess;
  if (!a.bf16 || (a.dk != 64 && a.dk != 128) || (a.cpx && a.write)) return hipErrorInvalidValue;
  if ((long)C * a.H * a.dk * 2 >= (1L << 32)) return hipErrorInvalidValue;  // 32-bit row offsets
  if (a.cpx) return launch_walk_g<false, true>(a, ws);
  return a.write ? launch_walk_g<true, false>(a, ws) : launch_walk_g<false, false>(a, ws);
}

}  // namespace kda
