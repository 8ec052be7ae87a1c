// kda_walk.hip -- second pass of the two-pass chunk forward for bf16 inputs: the walk of
// the state along the chunks of each (b, h, value tile).
//
// Per chunk, with the fp32 state S [d_k x VT] in registers (matrix-core accumulator
// layout), the chunk's record (A, M~ = (I + T)^-1 diag(beta), the gate block products) and
// the chunk's q, k, alpha, v:
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
// producer waves.  The producers move the chunk's record (A, M~ hi, M~ lo) and v tile
// global -> LDS with 16-byte DMA (two buffers: the next chunk streams in while the
// current one computes), and rebuild the chunk's operands Q o gamma, -(K o gamma) and
// (K o rho)^T from q, k, alpha and the record's block products (one gate item = 16 rows x
// one channel pair per lane, loaded one chunk ahead).
#include <stdlib.h>

#include "kda_common.h"
#include "kda_internal.h"
#include "kda_record.h"
#include "kda_tile.h"

namespace kda {

namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

// 16 bytes per lane from global memory straight into LDS: lane l of the wave writes
// lds_wave_base + 16 l (the LDS base is wave-uniform).  Completion is tracked by the
// vector-memory counter; the data is visible to the workgroup after a vmcnt(0) wait
// and a barrier.
__device__ __forceinline__ void dma16(const void* g, void* lds_wave_base) {
#ifndef KDA_HOST_PASS
  __builtin_amdgcn_global_load_lds((global_void*)g, (lds_void*)lds_wave_base, 16, 0, 0);
#endif
}

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
  static constexpr int GRP = DK / 2;  // gate items per 16-row block
  static constexpr int NITEM = NB * GRP;
  static_assert(NITEM <= NP * 64, "one gate item per producer lane");
  static_assert(N_DMA_V * 64 == C * UPR, "v tile split");
  static_assert(2 * (OPS + RL::DMA + V_BYTES) <= 160 * 1024, "LDS budget");
  // byte offset of the 16-byte unit u of (K o rho)^T row c: the unit index is XORed with
  // bits 1..3 of the row, so the sixteen rows a matrix-core fragment load touches (and
  // the two rows a gate item writes) spread over all LDS banks without row padding
  __device__ static constexpr int kt_unit(int c, int u) { return c * RS_KT + 16 * (u ^ ((c >> 1) & 7)); }
};

// flags of a split walk (launch_walk_split): no output stores; v read as zero; start from
// the identity; only the last segment writes the end state, indexed by (b, h)
enum : int { kSegNoOut = 1, kSegZeroV = 2, kSegIdentity = 4, kSegLastOnly = 8 };

__device__ __forceinline__ void fence_sched() {
#ifndef KDA_HOST_PASS
  __builtin_amdgcn_sched_barrier(0);
#endif
}

// One chunk of the walk for compute wave `wave` (value columns 16 wave + n of the tile):
// operands in `ops`, record (A, MH, ML) in `rec`, v tile in `vv` (rows nv.. of the chunk lie
// past the end of the sequence and read as zero); S advances one chunk and the outputs are
// staged over this wave's own (consumed) columns of `vv`.
template <int DK, int VT, bool G2, bool CPX>
__device__ __forceinline__ void walk_chunk(const char* ops, const char* rec, char* vv, const float (&wf)[16],
                                           bool zero_v, int nv, f32x4_t (&S)[DK / 16], int wave, int g, int n) {
  using K = WCfg<DK, VT>;
  using RL = typename K::RL;
  constexpr int KS = K::KS;
  const char* OQ = ops + K::OFF_Q;
  const char* OK = ops + K::OFF_K;
  const char* OKT = ops + K::OFF_KT;
  const float* OG = (const float*)(ops + K::OFF_G);
  const int col = 16 * wave + n;

  // R = V - (K o gamma) (S_hi + S_lo)  (the operand tile holds -(K o gamma)); O = (Q o gamma) S_hi
  // (one base address, rows at immediate offsets; the tile is read whole and the rows past
  // the end masked, so no per-row address or branch)
  char* const vb = vv + 4 * g * K::RS_V + col * 2;
  const int nvl = zero_v ? 0 : nv - 4 * g;  // rows 16 I + e of this lane that exist: 16 I + e < nvl
  f32x4_t Rr[NB], O[NB];
#pragma unroll
  for (int I = 0; I < NB; ++I) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x = bf16_to_f32(*(const uint16_t*)(vb + (16 * I + e) * K::RS_V));
      if constexpr (G2) x *= wf[4 * I + e];
      Rr[I][e] = 16 * I + e < nvl ? x : 0.f;
    }
    O[I] = zero4();
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    // S as hi / lo B fragments (k-slots: rows 32 ks + 4g + e and 32 ks + 16 + 4g + e)
    Frag<bf16_t> bsh, bsl;
    split_acc(S[2 * ks], S[2 * ks + 1], bsh, bsl);
    const int c0 = 32 * ks + 4 * g;
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      Frag<bf16_t> fk, fq;
      const char* krow = OK + (16 * I + n) * K::RS_Q;
      const char* qrow = OQ + (16 * I + n) * K::RS_Q;
      fk.load4x2(krow + c0 * 2, krow + (c0 + 16) * 2);
      fq.load4x2(qrow + c0 * 2, qrow + (c0 + 16) * 2);
      mma(Rr[I], fk, bsh);
      mma(Rr[I], fk, bsl);
      mma(O[I], fq, bsh);
    }
  }

  // Delta = M~ R over the lower blocks (I, s2) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1):
  // M~_hi R_hi + M~_hi R_lo + M~_lo R_hi
  Frag<bf16_t> brh[2], brl[2];
  split_acc(Rr[0], Rr[1], brh[0], brl[0]);
  split_acc(Rr[2], Rr[3], brh[1], brl[1]);
  f32x4_t D[NB];
#pragma unroll
  for (int I = 0; I < NB; ++I) D[I] = zero4();
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    const int I = j < 2 ? j : 2 + (j - 2) / 2, s2 = j < 2 ? 0 : (j - 2) % 2;
    const int o1 = RL::at(16 * I + n, 32 * s2 + 4 * g), o2 = RL::at(16 * I + n, 32 * s2 + 16 + 4 * g);
    Frag<bf16_t> fh, fl;
    fh.load4x2(rec + RL::MH + o1, rec + RL::MH + o2);
    fl.load4x2(rec + RL::ML + o1, rec + RL::ML + o2);
    mma(D[I], fh, brh[s2]);
    mma(D[I], fh, brl[s2]);
    mma(D[I], fl, brh[s2]);
  }

  // O += A Delta_hi
  Frag<bf16_t> bdh[2], bdl[2];
  split_acc(D[0], D[1], bdh[0], bdl[0]);
  split_acc(D[2], D[3], bdh[1], bdl[1]);
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    const int I = j < 2 ? j : 2 + (j - 2) / 2, s2 = j < 2 ? 0 : (j - 2) % 2;
    const int o1 = RL::at(16 * I + n, 32 * s2 + 4 * g), o2 = RL::at(16 * I + n, 32 * s2 + 16 + 4 * g);
    Frag<bf16_t> fa;
    fa.load4x2(rec + RL::A + o1, rec + RL::A + o2);
    mma(O[I], fa, bdh[s2]);
  }

  // S <- diag(gamma_last) S + (K o rho)^T (Delta_hi + Delta_lo)
#pragma unroll
  for (int r = 0; r < DK / 16; ++r) {
    const float4 c = *(const float4*)(OG + 16 * r + 4 * g);
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
    const int kc = 16 * r + n;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      // positions 32 s2 + 4g .. +3 and 32 s2 + 16 + 4g .. +3: units 4 s2 + g / 2 and + 2, half g & 1
      const int u = 4 * s2 + (g >> 1), h8 = 8 * (g & 1);
      Frag<bf16_t> fk;
      fk.load4x2(OKT + K::kt_unit(kc, u) + h8, OKT + K::kt_unit(kc, u + 2) + h8);
      mma(S[r], fk, bdh[s2]);
      mma(S[r], fk, bdl[s2]);
    }
  }

  // O over this wave's own (already consumed) v columns
#pragma unroll
  for (int I = 0; I < NB; ++I)
#pragma unroll
    for (int e = 0; e < 4; ++e) *(uint16_t*)(vb + (16 * I + e) * K::RS_V) = f32_to_bf16(O[I][e]);
}

}  // namespace

template <int DK, int VT, bool G2, bool CPX>
__global__ __launch_bounds__((VT / 16 + 4) * 64) void chunk_walk_kernel(
    const char* __restrict__ ws, const void* __restrict__ gq, const void* __restrict__ gk,
    const void* __restrict__ galpha, const void* __restrict__ gerase, const void* __restrict__ gv,
    const void* __restrict__ gw, const float* s0, void* __restrict__ go, float* sT, int Tlen, int H, int DV,
    int BH, const int* __restrict__ cu, const int* __restrict__ cbase, int gmax, int nseg, int segc, int flags) {
  using K = WCfg<DK, VT>;
  using RL = typename K::RL;
  using R = Raw<bf16_t>;
  using G = Gp2<CPX>;
  constexpr int NW = K::NW;
  constexpr int NP = K::NP;
  constexpr int NT = K::NT;
  constexpr int GRP = K::GRP;
  // separate LDS objects per buffer, so that reads of one buffer are not ordered
  // behind the DMA (or the operand stores) still filling the other
  __shared__ __align__(16) char ops_a[K::OPS];
  __shared__ __align__(16) char ops_b[K::OPS];
  __shared__ __align__(16) char rec_a[RL::DMA];
  __shared__ __align__(16) char rec_b[RL::DMA];
  __shared__ __align__(16) char v_a[K::V_BYTES];
  __shared__ __align__(16) char v_b[K::V_BYTES];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool producer = wave >= NW;
  const int pw = wave - NW;  // producer index
  const int g = lane >> 4;
  const int n = lane & 15;
  const int NVT = DV / VT;
  // chains: (b, h) pairs, times nseg segments of segc chunks each when the walk is split;
  // the value tiles of one chain (or segment) read the same records and share an XCD
  const int BHs = BH * nseg;
  int bhs, vt;
  {
    const int bid = blockIdx.x;
    if (NVT > 1 && (BHs & 7) == 0) {
      const int r = bid >> 3;
      vt = r % NVT;
      bhs = (r / NVT) * 8 + (bid & 7);
    } else {
      bhs = bid / NVT;
      vt = bid % NVT;
    }
  }
  const int bh = bhs / nseg, seg = bhs - bh * nseg;
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
  if (nseg > 1) {  // this workgroup's segment: chunks [seg segc, (seg + 1) segc)
    const int cb = seg * segc;
    rec0 += (size_t)cb * RL::BYTES;
    sbase += (size_t)cb * C;
    slen = max(0, min(slen - cb * C, segc * C));
  }
  const int nchunks = (slen + C - 1) / C;
  const size_t sidx = (size_t)bhs;  // start / end state index: (b, h), or (b, h, segment)
  const bool zero_v = (flags & kSegZeroV) != 0, no_out = (flags & kSegNoOut) != 0;

  f32x4_t S[DK / 16];
#pragma unroll
  for (int r = 0; r < DK / 16; ++r) S[r] = zero4();
  if ((flags & kSegIdentity) && !producer) {  // S = I (the walk then yields the transfer P)
#pragma unroll
    for (int r = 0; r < DK / 16; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[r][e] = 16 * r + 4 * g + e == v0 + 16 * wave + n ? 1.f : 0.f;
  } else if (s0 && !producer) {
#pragma unroll
    for (int r = 0; r < DK / 16; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[r][e] = s0[(sidx * DK + 16 * r + 4 * g + e) * DV + v0 + 16 * wave + n];
  }

  // ---- producer side: gate item of lane pt = (block iI, channel pair icp)
  const int pt = tid - NW * 64;
  const bool has_item = producer && pt < K::NITEM;
  // (producer wave pw) the outputs of chunk c staged in `vv` -> o, for the 1 KiB units of
  // the v tile this wave fills by DMA; then chunk c + 2's record matrices and v tile into
  // the same buffers.  Each wave reads out exactly the LDS bytes it overwrites next, so no
  // workgroup barrier sits between the two.
  auto store_o = [&](int c, const char* vv) __attribute__((always_inline)) {
    const int t0 = c * C;
    const int nv = min(C, slen - t0);
    for (int x = pw; x < K::N_DMA_V; x += NP) {
      const int sl = x * 64 + lane;
      const int row = sl / K::UPR, u = sl % K::UPR;
      if (row < nv)
        *(uint4*)((char*)go + ((sbase + t0 + row) * H + h) * DV * 2 + (size_t)v0 * 2 + (size_t)u * 16) =
            *(const uint4*)(vv + sl * 16);
    }
  };
  auto issue_dma = [&](int c, char* rec_dst, char* v_dst) __attribute__((always_inline)) {
    const char* rc = rec0 + (size_t)c * RL::BYTES;
    const int t0 = c * C;
    if (!zero_v) {
#pragma nounroll
      for (int x = pw; x < K::N_DMA_V; x += NP) {
        const int sl = x * 64 + lane;
        const int row = sl / K::UPR, u = sl % K::UPR;
        const size_t gr = (sbase + min(t0 + row, slen - 1)) * H + h;
        const size_t off = (gr * DV + v0) * 2 + (size_t)u * 16;
        dma16((const char*)gv + off, v_dst + x * 1024);
      }
    }
#pragma nounroll
    for (int x = pw; x < K::N_DMA_REC; x += NP) dma16(rc + x * 1024 + lane * 16, rec_dst + x * 1024);
  };
  // one chunk ahead: the item's 16 rows of q, k, alpha (and the erase gate) and its block's
  // gate products, raw.  Rows past the end are clamped to the last row (unconditional
  // loads) and given gate 1 when used.
  // (native vectors, not arrays: arrays captured by the lambdas stay in scratch memory)
  typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
  typedef float f32x2v __attribute__((ext_vector_type(2)));
  u32x16 pq, pk, pa, pe;
  f32x2v pgp = {1.f, CPX ? 0.f : 1.f}, prp = pgp, pgl = pgp;
  int plim = 0;  // rows of the loaded chunk that exist in this item's block
  auto issue_in = [&](int c) __attribute__((always_inline)) {
    // the item's first row and column byte from an opaque copy of the thread index: the
    // row offsets are then recomputed per chunk instead of hoisted out of the loop and
    // spilled (a reload would wait for every load in flight)
    int t = threadIdx.x - NW * 64;
    asm volatile("" : "+v"(t));
    const int blk = t / GRP, cp = t % GRP;
    const int t0 = c * C;
    const size_t base = ((sbase + t0) * H + h) * DK * 2;
    const uint32_t rs = (uint32_t)H * DK * 2;
    const int last = slen - 1 - t0;
    plim = slen - t0 - SUB * blk;
#pragma unroll
    for (int m = 0; m < SUB; ++m) {
      const uint32_t off = (uint32_t)min(SUB * blk + m, last) * rs + 4 * cp;
      pq[m] = *(const uint32_t*)((const char*)gq + base + off);
      pk[m] = *(const uint32_t*)((const char*)gk + base + off);
      pa[m] = *(const uint32_t*)((const char*)galpha + base + off);
      if constexpr (G2) pe[m] = *(const uint32_t*)((const char*)gerase + base + off);
    }
    const char* rc = rec0 + (size_t)c * RL::BYTES;
    if (blk > 0) pgp = *(const f32x2v*)(rc + RL::GP + ((blk - 1) * DK + 2 * cp) * 4);
    if (blk < NB - 1) prp = *(const f32x2v*)(rc + RL::RP + (blk * DK + 2 * cp) * 4);
    if (blk == 0) pgl = *(const f32x2v*)(rc + RL::G63 + 8 * cp);
  };
  // the operands of the loaded chunk into `ops`, bf16: Q o gamma and -(E o gamma) rows (E:
  // k, or b o k for Gated DeltaNet-2), (K o rho)^T columns, gamma_last
  auto form = [&](char* ops) __attribute__((always_inline)) {
    int t = threadIdx.x - NW * 64;
    asm volatile("" : "+v"(t));
    const int blk = t / GRP, cp = t % GRP;
    constexpr uint32_t kOne = CPX ? 0x00003F80u : R::kOneWord;
    G al[SUB];
#pragma unroll
    for (int m = 0; m < SUB; ++m) R::unpack(m < plim ? pa[m] : kOne, al[m].x, al[m].y);
    char* oq = ops + K::OFF_Q + (SUB * blk) * K::RS_Q + 4 * cp;
    char* ok = ops + K::OFF_K + (SUB * blk) * K::RS_Q + 4 * cp;
    G f{pgp[0], pgp[1]};
#pragma unroll
    for (int m = 0; m < SUB; ++m) {
      f *= al[m];
      float q0, q1, e0, e1, r0, r1;
      R::unpack(pq[m], q0, q1);
      R::unpack(pk[m], e0, e1);
      if constexpr (G2) {
        float b0, b1;
        R::unpack(pe[m], b0, b1);
        e0 *= b0;
        e1 *= b1;
      }
      f.row(q0, q1, r0, r1);
      *(uint32_t*)(oq + m * K::RS_Q) = pack_bf16x2(r0, r1);
      f.row(e0, e1, r0, r1);
      *(uint32_t*)(ok + m * K::RS_Q) = pack_bf16x2(-r0, -r1);
    }
    G bb{prp[0], prp[1]};
    typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
    u32x8 w0, w1;
#pragma unroll
    for (int m = SUB - 1; m >= 0; m -= 2) {
      float k0, k1, a0, a1, c0, c1;
      R::unpack(pk[m], k0, k1);
      bb.col(k0, k1, a0, a1);
      bb *= al[m];
      R::unpack(pk[m - 1], k0, k1);
      bb.col(k0, k1, c0, c1);
      bb *= al[m - 1];
      w0[m / 2] = pack_bf16x2(c0, a0);
      w1[m / 2] = pack_bf16x2(c1, a1);
    }
    char* kt = ops + K::OFF_KT;
    *(uint4*)(kt + K::kt_unit(2 * cp, 2 * blk)) = make_uint4(w0[0], w0[1], w0[2], w0[3]);
    *(uint4*)(kt + K::kt_unit(2 * cp, 2 * blk + 1)) = make_uint4(w0[4], w0[5], w0[6], w0[7]);
    *(uint4*)(kt + K::kt_unit(2 * cp + 1, 2 * blk)) = make_uint4(w1[0], w1[1], w1[2], w1[3]);
    *(uint4*)(kt + K::kt_unit(2 * cp + 1, 2 * blk + 1)) = make_uint4(w1[4], w1[5], w1[6], w1[7]);
    if (blk == 0) *(f32x2v*)(ops + K::OFF_G + 8 * cp) = pgl;
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

  if (nchunks > 0) {
    if (producer) issue_dma(0, rec_a, v_a);
    if (has_item) {
      issue_in(0);
      form(ops_a);
      if (nchunks > 1) issue_in(1);
    }
    if (G2 && !zero_v && !producer) load_w(0);
  }
  // Step c: the compute waves walk chunk c from buffers P (operands, record, v tile); the
  // producers store chunk c - 1's outputs out of buffers Q, stream chunk c + 1's record and v
  // tile into Q and build its operands there, and load chunk c + 2's inputs.  One barrier.
  auto step = [&](int c, const char* opsP, const char* recP, char* vP, char* opsQ, char* recQ, char* vQ) __attribute__((always_inline)) {
    full_barrier();  // chunk c landed and its operands are in place; chunk c - 1 finished
    if (producer) {
      if (c > 0 && !no_out) {
        store_o(c - 1, vQ);
#ifndef KDA_HOST_PASS
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the outputs are read out of vQ
#endif
      }
      if (c + 1 < nchunks) {
        issue_dma(c + 1, recQ, vQ);
        if (has_item) {
          form(opsQ);
          if (c + 2 < nchunks) issue_in(c + 2);
        }
      }
    } else {
      walk_chunk<DK, VT, G2, CPX>(opsP, recP, vP, wf, zero_v, slen - c * C, S, wave, g, n);
      if (G2 && !zero_v && c + 1 < nchunks) load_w(c + 1);
    }
  };
  for (int chunk = 0; chunk < nchunks; chunk += 2) {
    step(chunk, ops_a, rec_a, v_a, ops_b, rec_b, v_b);
    if (chunk + 1 >= nchunks) break;
    step(chunk + 1, ops_b, rec_b, v_b, ops_a, rec_a, v_a);
  }
  if (nchunks > 0) {
    full_barrier();
    if (producer && !no_out) store_o(nchunks - 1, ((nchunks - 1) & 1) ? v_b : v_a);
  }

  const bool last_only = (flags & kSegLastOnly) != 0;
  if (sT && !producer && (!last_only || seg == nseg - 1)) {
    const size_t oi = last_only ? (size_t)bh : sidx;
#pragma unroll
    for (int r = 0; r < DK / 16; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) sT[(oi * DK + 16 * r + 4 * g + e) * DV + v0 + 16 * wave + n] = S[r][e];
  }
}

// Start states of the segments of a split walk: Sst[b, h, 0] = S_0 (or zero) and
// Sst[b, h, g + 1] = P_g Sst[b, h, g] + B_g, where B_g is segment g's end state from a zero
// start and P_g (d_k x d_k) its end state from the identity with v = 0 -- the affine
// transfer of a block of the SFDA page ("Principales Contribuciones", item 3), applied
// segment by segment.  One workgroup per (b, h, 16 state columns), fp32.
template <int DK>
__global__ __launch_bounds__(256) void seg_scan_kernel(const float* __restrict__ s0, const float* __restrict__ P,
                                                     const float* __restrict__ Bst, float* __restrict__ Sst, int G,
                                                     int DV) {
  __shared__ float sS[DK][17];
  const int nsl = DV / 16, bh = blockIdx.x / nsl, c0 = (blockIdx.x % nsl) * 16;
  const int tid = threadIdx.x, c = tid & 15, r0 = tid >> 4;  // rows r0 + 16 j
  constexpr int RJ = DK / 16;
  const size_t SS = (size_t)DK * DV;
  float* out0 = Sst + (size_t)bh * G * SS;
#pragma unroll
  for (int j = 0; j < RJ; ++j) {
    const int r = r0 + 16 * j;
    const float x = s0 ? s0[((size_t)bh * DK + r) * DV + c0 + c] : 0.f;
    sS[r][c] = x;
    out0[(size_t)r * DV + c0 + c] = x;
  }
  for (int gi = 0; gi + 1 < G; ++gi) {
    __syncthreads();
    const float* Pg = P + ((size_t)bh * G + gi) * DK * DK;
    const float* Bg = Bst + ((size_t)bh * G + gi) * SS;
    float acc[RJ];
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
      const int r = r0 + 16 * j;
      float a = Bg[(size_t)r * DV + c0 + c];
      const float4* prow = (const float4*)(Pg + (size_t)r * DK);
#pragma unroll 4
      for (int k4 = 0; k4 < DK / 4; ++k4) {
        const float4 p = prow[k4];
        a += p.x * sS[4 * k4][c] + p.y * sS[4 * k4 + 1][c] + p.z * sS[4 * k4 + 2][c] + p.w * sS[4 * k4 + 3][c];
      }
      acc[j] = a;
    }
    __syncthreads();
    float* outg = Sst + ((size_t)bh * G + gi + 1) * SS;
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
      const int r = r0 + 16 * j;
      sS[r][c] = acc[j];
      outg[(size_t)r * DV + c0 + c] = acc[j];
    }
  }
}

template <int DK, int VT, bool G2, bool CPX>
static void walk_launch(const ChunkArgs& a, const void* ws, int nblocks, int BH, int DV, const float* s0, float* sT,
                        int nseg, int segc, int flags) {
  using K = WCfg<DK, VT>;
  hipLaunchKernelGGL((chunk_walk_kernel<DK, VT, G2, CPX>), dim3(nblocks), dim3(K::NT), 0, (hipStream_t)a.stream,
                     (const char*)ws, a.q, a.k, a.alpha, a.erase, a.v, a.write, s0, a.o, sT, a.T, a.H, DV, BH, a.cu,
                     a.ctab_base, a.gmax, nseg, segc, flags);
}

template <int DK, int VT, bool G2, bool CPX>
static hipError_t launch_walk_t(const ChunkArgs& a, const void* ws) {
  // varlen: one chain per (sequence, head): BH = n_seqs * H
  const int BHc = a.cu ? a.n_seqs * a.H : a.B * a.H;
  walk_launch<DK, VT, G2, CPX>(a, ws, BHc * (a.dv / VT), BHc, a.dv, a.s0, a.sT, 1, 0, 0);
  return hipGetLastError();
}

// The split walk (fixed-length batches at d_k = 128, few (b, h) chains): four launches
// over G segments per chain, 64 value columns per workgroup, scratch after the records:
// B [BH G][d_k][d_v], P [BH G][d_k][d_k], segment start states [BH G][d_k][d_v].
template <bool G2, bool CPX>
static hipError_t launch_walk_split(const ChunkArgs& a, const void* ws, int G) {
  const int BH = a.B * a.H, NC = (a.T + C - 1) / C, segc = (NC + G - 1) / G;
  const size_t rec = (size_t)BH * NC * WalkRecord<128>::BYTES;
  float* Bst = (float*)((char*)ws + rec);
  float* P = Bst + (size_t)BH * G * 128 * a.dv;
  float* Sst = P + (size_t)BH * G * 128 * 128;
  // the end states from a zero start (outputs not stored)
  walk_launch<128, 64, G2, CPX>(a, ws, BH * G * (a.dv / 64), BH, a.dv, nullptr, Bst, G, segc, kSegNoOut);
  // the transfers: the identity walked with v = 0 (the write gate is then irrelevant)
  walk_launch<128, 64, G2, CPX>(a, ws, BH * G * 2, BH, 128, nullptr, P, G, segc,
                                kSegNoOut | kSegZeroV | kSegIdentity);
  hipLaunchKernelGGL(seg_scan_kernel<128>, dim3(BH * (a.dv / 16)), dim3(256), 0, (hipStream_t)a.stream, a.s0, P,
                     Bst, Sst, G, a.dv);
  walk_launch<128, 64, G2, CPX>(a, ws, BH * G * (a.dv / 64), BH, a.dv, Sst, a.sT, G, segc, kSegLastOnly);
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

// The split costs three walks of NC / G chunks at 64 columns per workgroup against one
// walk of NC chunks on narrower tiles (with half the compute units idle or fewer): it is
// taken from G = 8 segments of at least 16 chunks.
int state_segments(int B, int T, int H, int dk, int dv, bool bf16) {
  if (!bf16 || dk != 128 || (dv != 64 && dv != 128)) return 1;
  const int NC = (T + C - 1) / C, o = state_seg_override();
  if (o >= 0) {
    const int G = min(o, NC / 16);
    return G >= 2 ? G : 1;
  }
  const long tiles = (long)B * H * (dv / 64);  // 64-column tiles of one walk per chain
  if (tiles <= 0 || tiles >= 256) return 1;
  const int G = min((int)((256 + tiles - 1) / tiles), NC / 16);  // at least 16 chunks per segment
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
