// kda_state.hip -- second pass of the two-pass chunk forward for fp32 inputs (d_k = d_v = 64):
// inter-chunk state propagation over the fp32 records of the fused kernel's first half.
// (bf16 inputs take the walk of kda_walk.hip.)
//
// For every (b, h, value tile) the workgroup walks the chunks in order, carrying the
// fp32 state S [d_k x VT] in registers (matrix-core accumulator layout), and applies
// the chunk's exact affine transfer (SFDA page, "Principales Contribuciones" item 3)
// from the record the first pass wrote:
//   U     = M~ V                       (M~ = (I + T)^-1 diag(beta))
//   Delta = U - W S
//   O     = (Q o gamma) S + A Delta
//   S    <- diag(gamma_last) S + (K o rho)^T Delta
// Records and v tiles move from global memory straight into LDS (16-byte DMA per lane);
// with two LDS buffers the next chunk streams in while the current one computes.
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

// NW compute waves (16 value columns each) and NP producer waves that only move each
// chunk's record and v tile global -> LDS with 16-byte DMA.  A wave stalled issuing
// DMA cannot issue matrix work, and one wave's DMA issue rate is well below a CU's
// share of HBM bandwidth, hence several producers beside the compute waves.
// G2: Gated DeltaNet-2 -- U = M (w o v); each compute wave loads the write gate of its own
// rows and columns into registers one chunk ahead, so the LDS holds only v tiles and the
// value tiles can be as wide as KDA's.
template <typename T, int DK, int VT, bool G2 = false>
struct SCfg {
  using RL = RecordLayout<T, DK>;
  static constexpr int ES = Elem<T>::kBytes;
  static constexpr int NW = VT / 16;
  static constexpr int NP = 4;
  static constexpr int NT = (NW + NP) * 64;
  static constexpr int KS = DK / 32;
  static constexpr int RS_V = VT * ES;        // v tile rows (dense: filled by DMA), reused for O
  static constexpr int UPR = RS_V / 16;        // 16-byte units per v row
  static constexpr int N_DMA_REC = (RL::IMG + 1023) / 1024;  // wave-wide DMA steps per record
  static constexpr int N_DMA_V = C * UPR / 64;
  static constexpr int V_BYTES = C * RS_V;
  static constexpr int NTILE = 1;            // v tiles per buffer
  // two record and v buffers when they fit: the next chunk streams in during this one
  static constexpr int NBUF = 2 * (RL::IMG + NTILE * V_BYTES) <= 160 * 1024 ? 2 : 1;
  static_assert(N_DMA_V * 64 == C * UPR, "v tile split");
  static_assert(NBUF * (RL::IMG + NTILE * V_BYTES) <= 160 * 1024, "LDS budget");
};

// flags of a split walk (launch_state_split): no output stores; v read as zero; start from
// the identity; only the last segment writes the end state, indexed by (b, h)
enum : int { kSegNoOut = 1, kSegZeroV = 2, kSegIdentity = 4, kSegLastOnly = 8 };

}  // namespace

// Keeps the compiler's scheduler from moving instructions across this point: the
// fragment loads issued before it stay ahead of the matrix-core work after it.
__device__ __forceinline__ void fence_sched() {
#ifndef KDA_HOST_PASS
  __builtin_amdgcn_sched_barrier(0);
#endif
}

// One chunk of the state pass: record `rec` and v tile `vv` are in LDS; S advances one
// chunk and the chunk's outputs are staged into this wave's own columns of `vv`.
//   U = M~ V ;  Delta = U - W S ;  O = (Q o gamma) S + A Delta ;
//   S <- diag(gamma_last) S + (K o rho)^T Delta
// With one compute wave per SIMD little else hides LDS latency, so the operand
// fragments of each group of products are loaded one group ahead (software pipelining).
// CPX: SFDA complex gates -- gamma_last holds (Re, Im) per key-channel pair and turns the
// state's row pairs (rows 2p, 2p+1 = one complex coordinate, same lane) by that product.
template <typename T, int DK, int VT, bool G2 = false, bool CPX = false>
__device__ __forceinline__ void state_chunk(const char* rec, char* vv, const Frag<T>* wf, f32x4_t (&S)[DK / 16],
                                            int wave, int g, int n) {
  using K = SCfg<T, DK, VT, G2>;
  using RL = typename K::RL;
  constexpr int ES = K::ES;
  constexpr int KS = K::KS;
  const char* WW = rec + RL::WW;
  const char* QG = rec + RL::QG;
  const char* KRT = rec + RL::KRT;
  const char* AT = rec + RL::AT;
  const char* MT = rec + RL::MT;
  const float* GC = (const float*)(rec + RL::GC);

  // -W and Q o gamma rows of block I, key steps ks: A fragments (slots 4g.. and 16 + 4g..)
  auto load_wq = [&](Frag<T> (&fw)[KS], Frag<T> (&fq)[KS], int I) {
    const char* wrow = WW + (16 * I + n) * RL::RS_DK;
    const char* qrow = QG + (16 * I + n) * RL::RS_DK;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c0 = 32 * ks + 4 * g;
      fw[ks].load4x2(wrow + c0 * ES, wrow + (c0 + 16) * ES);
      fq[ks].load4x2(qrow + c0 * ES, qrow + (c0 + 16) * ES);
    }
  };

  // group 0 operands: M~ (lower blocks only), the v tile columns of this wave, block 0 of W, Q
  Frag<T> fm[6], bv[2];
  Frag<T> fw[2][KS], fq[2][KS];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) bv[ks].load_col8(vv + (32 * ks + 8 * g) * K::RS_V + (16 * wave + n) * ES, K::RS_V);
  if constexpr (G2) {  // the write side: z = w o v, rounded once to the operand type
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float z[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) z[e] = bv[ks].get(e) * wf[ks].get(e);
#pragma unroll
      for (int e = 0; e < 8; ++e) bv[ks].set(e, z[e]);
    }
  }
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    const int I = j < 2 ? j : 2 + (j - 2) / 2, ks = j < 2 ? 0 : (j - 2) % 2;
    fm[j].load8(MT + (16 * I + n) * RL::RS_C + (32 * ks + 8 * g) * ES);
  }
  load_wq(fw[0], fq[0], 0);
  Frag<T> bs[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) bs[ks].from_acc(S[2 * ks], S[2 * ks + 1]);
  fence_sched();

  // U = M~ V, then per block I: Delta_I = U_I - W_I S, O_I = Q_I S (operands of I + 1 in flight)
  f32x4_t Dl[NB], Ot[NB];
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    const int I = j < 2 ? j : 2 + (j - 2) / 2, ks = j < 2 ? 0 : (j - 2) % 2;
    if (ks == 0) Dl[I] = zero4();
    mma(Dl[I], fm[j], bv[ks]);
  }
#pragma unroll
  for (int I = 0; I < NB; ++I) {
    if (I + 1 < NB) load_wq(fw[(I + 1) & 1], fq[(I + 1) & 1], I + 1);
    fence_sched();
    Ot[I] = zero4();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      mma(Dl[I], fw[I & 1][ks], bs[ks]);
      mma(Ot[I], fq[I & 1][ks], bs[ks]);
    }
    fence_sched();
  }

  // A Delta (A lower blocks) and the first half of (K o rho)^T, loaded while the
  // last products retire
  Frag<T> fa[6];
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    const int I = j < 2 ? j : 2 + (j - 2) / 2, s2 = j < 2 ? 0 : (j - 2) % 2;
    const char* arow = AT + (16 * I + n) * RL::RS_C;
    const int p0 = 32 * s2 + 4 * g;
    fa[j].load4x2(arow + p0 * ES, arow + (p0 + 16) * ES);
  }
  constexpr int RH = DK / 32;  // S row blocks per half
  Frag<T> fk[2][RH][2];
  float4 gc[2][RH];
  auto load_k = [&](int half) {
#pragma unroll
    for (int rr = 0; rr < RH; ++rr) {
      const int r = half * RH + rr;
      const char* krow = KRT + (16 * r + n) * RL::RS_C;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int p0 = 32 * s2 + 4 * g;
        fk[half][rr][s2].load4x2(krow + p0 * ES, krow + (p0 + 16) * ES);
      }
      gc[half][rr] = *(const float4*)(GC + 16 * r + 4 * g);
    }
  };
  load_k(0);
  fence_sched();
  Frag<T> bd[2];
  bd[0].from_acc(Dl[0], Dl[1]);
  bd[1].from_acc(Dl[2], Dl[3]);
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    const int I = j < 2 ? j : 2 + (j - 2) / 2, s2 = j < 2 ? 0 : (j - 2) % 2;
    mma(Ot[I], fa[j], bd[s2]);
  }
  load_k(1);
  fence_sched();
  // S <- diag(gamma_last) S + (K o rho)^T Delta
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int rr = 0; rr < RH; ++rr) {
      const int r = half * RH + rr;
      if constexpr (CPX) {
        const float4 c = gc[half][rr];
        const float s0 = S[r][0], s1 = S[r][1], s2 = S[r][2], s3 = S[r][3];
        S[r][0] = c.x * s0 - c.y * s1;
        S[r][1] = c.y * s0 + c.x * s1;
        S[r][2] = c.z * s2 - c.w * s3;
        S[r][3] = c.w * s2 + c.z * s3;
      } else {
        S[r][0] *= gc[half][rr].x;
        S[r][1] *= gc[half][rr].y;
        S[r][2] *= gc[half][rr].z;
        S[r][3] *= gc[half][rr].w;
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) mma(S[r], fk[half][rr][s2], bd[s2]);
    }
  // O over this wave's own (already consumed) v columns
#pragma unroll
  for (int I = 0; I < NB; ++I)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      char* p = vv + (16 * I + 4 * g + e) * K::RS_V + (16 * wave + n) * ES;
      if (ES == 2)
        *(uint16_t*)p = f32_to_bf16(Ot[I][e]);
      else
        *(float*)p = Ot[I][e];
    }
}

template <typename T, int DK, int VT, bool G2, bool CPX = false>
__global__ __launch_bounds__((VT / 16 + 4) * 64) void chunk_state_kernel(const char* __restrict__ ws,
                                                                         const void* __restrict__ gv,
                                                                         const float* s0, void* __restrict__ go,
                                                                         float* sT, int Tlen, int H, int DV, int BH,
                                                                         const void* __restrict__ gw,
                                                                         const int* __restrict__ cu,
                                                                         const int* __restrict__ cbase, int gmax,
                                                                         int nseg, int segc, int flags) {
  using K = SCfg<T, DK, VT, G2>;
  constexpr int NP = K::NP;
  using RL = typename K::RL;
  constexpr int ES = K::ES;
  constexpr int NT = K::NT;
  constexpr int NW = K::NW;
  // separate LDS objects per buffer, so that reads of one buffer are not ordered
  // behind the DMA still filling the other
  __shared__ __align__(16) char rec_a[RL::IMG];
  __shared__ __align__(16) char v_a[K::V_BYTES];
  __shared__ __align__(16) char rec_b[K::NBUF == 2 ? RL::IMG : 16];
  __shared__ __align__(16) char v_b[K::NBUF == 2 ? K::V_BYTES : 16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool producer = wave >= NW;  // move the data; the other waves only compute
  const int pw = wave - NW;          // producer index
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
  const bool zero_v = (flags & kSegZeroV) != 0, no_out = (flags & kSegNoOut) != 0;

  // (producer waves) chunk c's record and v tile -> LDS; v rows past the end are clamped
  // to the last row here and zeroed once they have landed
  auto issue = [&](int c, char* rec_dst, char* v_dst) {
    const char* rec = rec0 + (size_t)c * RL::BYTES;
    const int t0 = c * C;
#pragma nounroll
    for (int x = zero_v ? K::N_DMA_V : pw; x < K::N_DMA_V; x += NP) {
      const int sl = x * 64 + lane;
      const int row = sl / K::UPR, u = sl % K::UPR;
      const size_t gr = (sbase + min(t0 + row, slen - 1)) * H + h;
      const size_t off = (gr * DV + v0) * ES + (size_t)u * 16;
      dma16((const char*)gv + off, v_dst + x * 1024);
    }
#pragma nounroll
    for (int x = pw; x < K::N_DMA_REC; x += NP) {
      const int off = x * 1024 + lane * 16;
      if (off < RL::IMG) dma16(rec + off, rec_dst + x * 1024);
    }
  };
  // the staged outputs of chunk c (in the consumed v tile `vv`) -> o
  auto store_o = [&](int c, const char* vv) {
    if (no_out) return;
    const int t0 = c * C;
    const int nv = min(C, slen - t0);
    for (int j = tid; j < C * K::UPR; j += NT) {
      const int row = j / K::UPR, u = j % K::UPR;
      if (row < nv)
        *(uint4*)((char*)go + ((sbase + t0 + row) * H + h) * DV * ES + (size_t)v0 * ES + (size_t)u * 16) =
            *(const uint4*)(vv + row * K::RS_V + u * 16);
    }
  };
  // v rows past the end of the sequence read as zero
  auto pad_rows = [&](int c, char* vv) {
    const int nv = zero_v ? 0 : slen - c * C;
    if (nv < C) {
      for (int j = nv * K::UPR + tid; j < C * K::UPR; j += NT) *(uint4*)(vv + j * 16) = make_uint4(0, 0, 0, 0);
      lds_barrier();
    }
  };

  // (compute waves, G2) the write gate of this lane's rows 32 ks + 8 g + e and column of
  // chunk c, rows past the end clamped to the last row (their v rows are zero)
  Frag<T> wf[G2 ? 2 : 1];
#pragma unroll
  for (int ks = 0; ks < (G2 ? 2 : 1); ++ks) wf[ks].zero();  // stays zero where v reads as zero
  auto load_w = [&](int c) {
    const int t0 = c * C, col = v0 + 16 * wave + n;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const size_t row = sbase + min(t0 + 32 * ks + 8 * g + e, slen - 1);
        wf[ks].set(e, Elem<T>::load(gw, (row * H + h) * DV + col));
      }
  };
  if (G2 && !zero_v && nchunks > 0 && !producer) load_w(0);
  if (nchunks > 0 && producer) issue(0, rec_a, v_a);
  if constexpr (K::NBUF == 2) {
    // chunk c computes from buffers P while the producer streams chunk c + 1 into
    // buffers Q; the outputs of chunk c - 1, staged in Q's v tile, are stored first
    auto step = [&](int c, const char* recP, char* vP, char* recQ, char* vQ) {
      full_barrier();  // chunk c landed; chunk c - 1 finished everywhere
      if (c > 0) {
        store_o(c - 1, vQ);
        lds_barrier();  // vQ read out before the next v tile lands there
      }
      pad_rows(c, vP);
      if (producer) {
        if (c + 1 < nchunks) issue(c + 1, recQ, vQ);
      } else {
        state_chunk<T, DK, VT, G2, CPX>(recP, vP, wf, S, wave, g, n);
        if (G2 && !zero_v && c + 1 < nchunks) load_w(c + 1);
      }
    };
    for (int chunk = 0; chunk < nchunks; chunk += 2) {
      step(chunk, rec_a, v_a, rec_b, v_b);
      if (chunk + 1 >= nchunks) break;
      step(chunk + 1, rec_b, v_b, rec_a, v_a);
    }
    if (nchunks > 0) {
      lds_barrier();
      store_o(nchunks - 1, ((nchunks - 1) & 1) ? v_b : v_a);
    }
  } else {
    for (int chunk = 0; chunk < nchunks; ++chunk) {
      full_barrier();
      pad_rows(chunk, v_a);
      if (!producer) {
        state_chunk<T, DK, VT, G2, CPX>(rec_a, v_a, wf, S, wave, g, n);
        if (G2 && !zero_v && chunk + 1 < nchunks) load_w(chunk + 1);
      }
      lds_barrier();
      store_o(chunk, v_a);
      if (chunk + 1 < nchunks) {
        lds_barrier();  // every output read out of v_a before the next chunk lands there
        if (producer) issue(chunk + 1, rec_a, v_a);
      }
    }
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

template <typename T, int DK, int VT, bool G2, bool CPX>
static hipError_t launch_state_t(const ChunkArgs& a, const void* ws) {
  using K = SCfg<T, DK, VT, G2>;
  const int BH = a.B * a.H;
  auto kern = chunk_state_kernel<T, DK, VT, G2, CPX>;
  // varlen: one chain per (sequence, head): BH = n_seqs * H
  const int BHc = a.cu ? a.n_seqs * a.H : BH;
  hipLaunchKernelGGL(kern, dim3(BHc * (a.dv / VT)), dim3(K::NT), 0, (hipStream_t)a.stream, (const char*)ws, a.v,
                     a.s0, a.o, a.sT, a.T, a.H, a.dv, BHc, a.write, a.cu, a.ctab_base, a.gmax, 1, 0, 0);
  return hipGetLastError();
}

// KDA_STATE_VT=16|32|64 pins the state pass's value-tile width (tuning aid)
static int state_vt_override() {
  static const int v = [] {
    const char* e = getenv("KDA_STATE_VT");
    return e ? atoi(e) : 0;
  }();
  return v;
}

// Value-tile width of the state pass: each workgroup walks the whole chunk chain of one
// (b, h, tile), so with few (b, h) pairs narrower tiles put more compute units on the
// chains (every tile reads the whole record; the extra reads hit in L2).  The Gated
// DeltaNet-2 write gate rides in registers, so every gate family takes the same widths.
static int pick_state_vt(const ChunkArgs& a) {
  const int cap = 64;
  const int o = state_vt_override();
  int vt;
  if (o == 16 || o == 32 || o == 64) {
    vt = o <= a.dv ? o : a.dv;
  } else {
    const long bh = (long)(a.cu ? a.n_seqs : a.B) * a.H;
    vt = bh * (a.dv / 64) >= 256 ? 64 : bh * (a.dv / 32) >= 256 ? 32 : 16;
  }
  return vt < cap ? vt : cap;
}

template <typename T, int DK, bool G2, bool CPX>
static hipError_t launch_state_vt(const ChunkArgs& a, const void* ws) {
  switch (pick_state_vt(a)) {
    case 16: return launch_state_t<T, DK, 16, G2, CPX>(a, ws);
    case 32: return launch_state_t<T, DK, 32, G2, CPX>(a, ws);
    default: return launch_state_t<T, DK, 64, G2, CPX>(a, ws);
  }
}

template <bool G2>
static hipError_t launch_state_g(const ChunkArgs& a, const void* ws) {
  return a.dk == 64 && a.dv == 64 ? launch_state_vt<float, 64, G2, false>(a, ws) : hipErrorInvalidValue;
}

// fp32 records (RecordLayout) are walked here; bf16 ones by launch_walk (kda_walk.hip)
hipError_t launch_state(const ChunkArgs& a, const void* ws) {
  if ((a.cu ? a.n_seqs : a.B) * a.H == 0) return hipSuccess;
  if (a.bf16) return launch_walk(a, ws);
  if (a.cpx) return hipErrorInvalidValue;
  return a.write ? launch_state_g<true>(a, ws) : launch_state_g<false>(a, ws);
}

}  // namespace kda
