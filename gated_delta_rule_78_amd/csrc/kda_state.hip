// kda_state.hip -- second pass of the two-pass chunk forward: inter-chunk state propagation.
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
#include "kda_common.h"
#include "kda_internal.h"
#include "kda_record.h"

namespace kda {

namespace {

constexpr int C = 64;
constexpr int NB = 4;

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

__device__ __forceinline__ void wait_vmem() {
#ifndef KDA_HOST_PASS
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt left at their maxima
#endif
}

template <typename T, int DK, int VT>
struct SCfg {
  using RL = RecordLayout<T, DK>;
  static constexpr int ES = Elem<T>::kBytes;
  static constexpr int NW = VT / 16;
  static constexpr int NT = NW * 64;
  static constexpr int KS = DK / 32;
  static constexpr int RS_V = VT * ES;        // v tile rows (dense: filled by DMA), reused for O
  static constexpr int UPR = RS_V / 16;        // 16-byte units per v row
  static constexpr int N_DMA_REC = (RL::IMG + 1023) / 1024;  // wave-wide DMA steps per record
  static constexpr int N_DMA_V = C * UPR / 64;
  static constexpr int V_BYTES = C * RS_V;
  // two record and v buffers when they fit: the next chunk streams in during this one
  static constexpr int NBUF = 2 * (RL::IMG + V_BYTES) <= 160 * 1024 ? 2 : 1;
  static_assert(N_DMA_V * 64 == C * UPR, "v tile split");
  static_assert(NBUF * (RL::IMG + V_BYTES) <= 160 * 1024, "LDS budget");
};

}  // namespace

// One chunk of the state pass: record `rec` and v tile `vv` are in LDS; S advances one
// chunk and the chunk's outputs are staged into this wave's own columns of `vv`.
template <typename T, int DK, int VT>
__device__ __forceinline__ void state_chunk(const char* rec, char* vv, f32x4_t (&S)[DK / 16], int wave, int g,
                                            int n) {
  using K = SCfg<T, DK, VT>;
  using RL = typename K::RL;
  constexpr int ES = K::ES;
  const char* WW = rec + RL::WW;
  const char* QG = rec + RL::QG;
  const char* KRT = rec + RL::KRT;
  const char* AT = rec + RL::AT;
  const char* MT = rec + RL::MT;
  const float* GC = (const float*)(rec + RL::GC);

  // U = M~ V for this wave's 16 value columns
  f32x4_t Dl[NB];
  {
    Frag<T> bv[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) bv[ks].load_col8(vv + (32 * ks + 8 * g) * K::RS_V + (16 * wave + n) * ES, K::RS_V);
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      Dl[I] = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks == 0 || I >= 2) {
          Frag<T> fa;
          fa.load8(MT + (16 * I + n) * RL::RS_C + (32 * ks + 8 * g) * ES);
          mma(Dl[I], fa, bv[ks]);
        }
      }
    }
  }
  // Delta = U - W S ; O = (Q o gamma) S + A Delta ; S <- diag(gamma_last) S + (K o rho)^T Delta
  Frag<T> bs[K::KS];
#pragma unroll
  for (int ks = 0; ks < K::KS; ++ks) bs[ks].from_acc(S[2 * ks], S[2 * ks + 1]);
  f32x4_t Ot[NB];
#pragma unroll
  for (int I = 0; I < NB; ++I) {
    Ot[I] = zero4();
    const char* wrow = WW + (16 * I + n) * RL::RS_DK;
    const char* qrow = QG + (16 * I + n) * RL::RS_DK;
    Frag<T> fw[K::KS], fq[K::KS];
#pragma unroll
    for (int ks = 0; ks < K::KS; ++ks) {
      const int c0 = 32 * ks + 4 * g;
      fw[ks].load4x2(wrow + c0 * ES, wrow + (c0 + 16) * ES);
      fq[ks].load4x2(qrow + c0 * ES, qrow + (c0 + 16) * ES);
    }
#pragma unroll
    for (int ks = 0; ks < K::KS; ++ks) {
      mma(Dl[I], fw[ks], bs[ks]);
      mma(Ot[I], fq[ks], bs[ks]);
    }
  }
  Frag<T> bd[2];
  bd[0].from_acc(Dl[0], Dl[1]);
  bd[1].from_acc(Dl[2], Dl[3]);
#pragma unroll
  for (int I = 0; I < NB; ++I) {
    const char* arow = AT + (16 * I + n) * RL::RS_C;
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
    const char* krow = KRT + (16 * r + n) * RL::RS_C;
    Frag<T> fa[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int p0 = 32 * s2 + 4 * g;
      fa[s2].load4x2(krow + p0 * ES, krow + (p0 + 16) * ES);
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) mma(S[r], fa[s2], bd[s2]);
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

template <typename T, int DK, int VT>
__global__ __launch_bounds__((VT / 16) * 64) void chunk_state_kernel(const char* __restrict__ ws,
                                                                     const void* __restrict__ gv, const float* s0,
                                                                     void* __restrict__ go, float* sT, int Tlen, int H,
                                                                     int DV, int BH) {
  using K = SCfg<T, DK, VT>;
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
  const int g = lane >> 4;
  const int n = lane & 15;
  const int NVT = DV / VT;
  int bh, vt;
  {
    const int bid = blockIdx.x;
    if (NVT > 1 && (BH & 7) == 0) {
      const int r = bid >> 3;
      vt = r % NVT;
      bh = (r / NVT) * 8 + (bid & 7);
    } else {
      bh = bid / NVT;
      vt = bid % NVT;
    }
  }
  const int b = bh / H, h = bh % H;
  const int v0 = vt * VT;
  const int nchunks = (Tlen + C - 1) / C;
  const char* rec0 = ws + (size_t)bh * nchunks * RL::BYTES;

  f32x4_t S[DK / 16];
#pragma unroll
  for (int r = 0; r < DK / 16; ++r) S[r] = zero4();
  if (s0) {
#pragma unroll
    for (int r = 0; r < DK / 16; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) S[r][e] = s0[((size_t)bh * DK + 16 * r + 4 * g + e) * DV + v0 + 16 * wave + n];
  }

  // chunk c's record and v tile (rows past the end clamped to the last row) -> LDS
  auto issue = [&](int c, char* rec_dst, char* v_dst) {
    const char* rec = rec0 + (size_t)c * RL::BYTES;
    for (int x = wave; x < K::N_DMA_REC; x += NW) {
      const int off = x * 1024 + lane * 16;
      if (off < RL::IMG) dma16(rec + off, rec_dst + x * 1024);
    }
    const int t0 = c * C;
    for (int x = wave; x < K::N_DMA_V; x += NW) {
      const int sl = x * 64 + lane;
      const int row = sl / K::UPR, u = sl % K::UPR;
      const size_t gr = ((size_t)b * Tlen + min(t0 + row, Tlen - 1)) * H + h;
      dma16((const char*)gv + (gr * DV + v0) * ES + (size_t)u * 16, v_dst + x * 1024);
    }
  };
  // after the wait: zero the v rows past the end, then store the staged outputs
  auto finish = [&](int c, char* vv) {
    const int t0 = c * C;
    const int nv = min(C, Tlen - t0);
    __syncthreads();
    for (int j = tid; j < C * K::UPR; j += NT) {
      const int row = j / K::UPR, u = j % K::UPR;
      if (row < nv)
        *(uint4*)((char*)go + (((size_t)b * Tlen + t0 + row) * H + h) * DV * ES + (size_t)v0 * ES + (size_t)u * 16) =
            *(const uint4*)(vv + row * K::RS_V + u * 16);
    }
  };
  auto pad_rows = [&](int c, char* vv) {
    const int nv = Tlen - c * C;
    if (nv < C) {
      for (int j = nv * K::UPR + tid; j < C * K::UPR; j += NT) *(uint4*)(vv + j * 16) = make_uint4(0, 0, 0, 0);
      __syncthreads();
    }
  };

  if (nchunks > 0) issue(0, rec_a, v_a);
  if constexpr (K::NBUF == 2) {
    for (int chunk = 0; chunk < nchunks; chunk += 2) {
      wait_vmem();
      __syncthreads();
      pad_rows(chunk, v_a);
      if (chunk + 1 < nchunks) issue(chunk + 1, rec_b, v_b);
      state_chunk<T, DK, VT>(rec_a, v_a, S, wave, g, n);
      finish(chunk, v_a);
      if (chunk + 1 >= nchunks) break;
      wait_vmem();
      __syncthreads();
      pad_rows(chunk + 1, v_b);
      if (chunk + 2 < nchunks) issue(chunk + 2, rec_a, v_a);
      state_chunk<T, DK, VT>(rec_b, v_b, S, wave, g, n);
      finish(chunk + 1, v_b);
    }
  } else {
    for (int chunk = 0; chunk < nchunks; ++chunk) {
      wait_vmem();
      __syncthreads();
      pad_rows(chunk, v_a);
      state_chunk<T, DK, VT>(rec_a, v_a, S, wave, g, n);
      finish(chunk, v_a);
      if (chunk + 1 < nchunks) {
        __syncthreads();  // every output read out of v_a before the next chunk lands there
        issue(chunk + 1, rec_a, v_a);
      }
    }
  }

  if (sT) {
#pragma unroll
    for (int r = 0; r < DK / 16; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sT[((size_t)bh * DK + 16 * r + 4 * g + e) * DV + v0 + 16 * wave + n] = S[r][e];
  }
}

template <typename T, int DK, int VT>
static hipError_t launch_state_t(const ChunkArgs& a, const void* ws) {
  using K = SCfg<T, DK, VT>;
  const int BH = a.B * a.H;
  auto kern = chunk_state_kernel<T, DK, VT>;
  hipLaunchKernelGGL(kern, dim3(BH * (a.dv / VT)), dim3(K::NT), 0, (hipStream_t)a.stream,
                     (const char*)ws, a.v, a.s0, a.o, a.sT, a.T, a.H, a.dv, BH);
  return hipGetLastError();
}

hipError_t launch_state(const ChunkArgs& a, const void* ws) {
  if (a.B * a.H == 0) return hipSuccess;
  if (!a.bf16) return a.dk == 64 && a.dv == 64 ? launch_state_t<float, 64, 64>(a, ws) : hipErrorInvalidValue;
  return a.dk == 64 ? launch_state_t<bf16_t, 64, 64>(a, ws) : launch_state_t<bf16_t, 128, 64>(a, ws);
}

}  // namespace kda
