// kda_decode.hip -- one recurrent KDA / CKDA token per (batch, head), state in place.
//
//   S' = Diag(alpha) S ;  u = S'^T k ;  p = S'^T q ;  delta = beta (v - u)
//   S  <- S' + k delta^T ;  o = S^T q = p + (q . k) delta
//
// This is one step of the recurrence on the SFDA page ("Arquitectura
// Central", phases zero) in its constant-memory inference use ("Complex KDA"
// summary, practical implications: O(1) inference memory).
//
// Bandwidth bound: every step streams the fp32 d_k x d_v state from HBM once
// and back once.  One workgroup of 512 threads owns one (b, h) tile; a thread
// keeps DK / (512 * 4 / DV) rows x 4 columns of the tile in registers (one
// 16-byte load and one 16-byte store per row), so the tile is read and written
// exactly once (few registers per thread: many waves in flight per CU).  The two
// column reductions over d_k (u and p) go through lane shuffles inside a wave
// and a small LDS exchange across the eight waves.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

// G2: Gated DeltaNet-2 step -- the read goes through the erase gate, u = S'^T (b o k),
// the write through the write gate, delta = w o v - u (no beta).
// CPX: SFDA step -- S' = Lambda S with complex gates (SFDA page, "Arquitectura
// Central"): alpha holds (Re, Im) of the gate of each key-channel pair, and rows 2p, 2p+1
// of every state column (one complex coordinate) are multiplied by that gate.
template <typename T, int DK, int DV, bool G2, bool CPX = false>
__global__ __launch_bounds__(512) void decode_kernel(const void* __restrict__ q,
                                                     const void* __restrict__ k,
                                                     const void* __restrict__ v,
                                                     const void* __restrict__ alpha,
                                                     const void* __restrict__ beta,
                                                     float* __restrict__ state,
                                                     void* __restrict__ o,
                                                     const void* __restrict__ erase,
                                                     const void* __restrict__ write, int ntok, int H) {
  constexpr int NT = 512;
  constexpr int NWV = NT / 64;
  constexpr int TPR = DV / 4;      // threads covering one state row (4 columns each)
  constexpr int RG = NT / TPR;     // row groups
  constexpr int RPT = DK / RG;     // rows per thread
  static_assert(RPT * RG == DK && TPR * 4 == DV, "tile split");
  static_assert(!CPX || RPT % 2 == 0, "complex gates: a thread holds whole row pairs");

  // token inputs are staged NTK tokens at a time, so that the token loop waits on no
  // global load; the column sums of u, p and q . k alternate between two buffers, so
  // that each token needs one barrier
  constexpr int NTK = 8;
  __shared__ float s_q[NTK][DK], s_k[NTK][DK], s_a[NTK][DK], s_v[NTK][DV], s_bt[NTK];
  __shared__ float s_e[G2 ? NTK : 1][G2 ? DK : 1];  // read-side key b o k (G2)
  __shared__ float s_red[2][NWV][2][DV];
  __shared__ float s_qk[2][NWV];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const size_t bh = blockIdx.x;
  const size_t b = bh / H, h = bh % H;
  const int cq = tid % TPR;        // column quad
  const int rg = tid / TPR;        // row group
  // the thread's i-th state row: rows rg + RG i; with complex gates, the row pairs
  // (2p, 2p+1) for p = rg + RG (i / 2), so that both rows of a coordinate sit in one thread
  auto row_of = [&](int i) { return CPX ? 2 * (rg + RG * (i >> 1)) + (i & 1) : rg + RG * i; };

  // the state streams through once per call: nontemporal loads and stores keep it from
  // displacing cached lines it will not reuse
  f32x4_t* S = reinterpret_cast<f32x4_t*>(state + bh * (size_t)DK * DV);
  float4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const f32x4_t t = __builtin_nontemporal_load(&S[(size_t)row_of(i) * TPR + cq]);
    s[i] = make_float4(t[0], t[1], t[2], t[3]);
  }

  // tokens in order, the state staying in registers ([B, ntok, H, .] inputs and outputs;
  // ntok = 1 is the single decode step)
  for (int t0 = 0; t0 < ntok; t0 += NTK) {
    const int nb = min(NTK, ntok - t0);
    if (t0 > 0) __syncthreads();  // the previous batch's staged inputs are consumed
    for (int x = tid; x < nb * DK; x += NT) {
      const int j = x / DK, c = x % DK;
      const size_t row = (b * ntok + t0 + j) * H + h;
      const float kk = Elem<T>::load(k, row * DK + c);
      s_q[j][c] = Elem<T>::load(q, row * DK + c);
      s_k[j][c] = kk;
      s_a[j][c] = Elem<T>::load(alpha, row * DK + c);
      if constexpr (G2) s_e[j][c] = Elem<T>::load(erase, row * DK + c) * kk;
    }
    // the write value: v (KDA, beta applied below) or w o v (G2)
    for (int x = tid; x < nb * DV; x += NT) {
      const int j = x / DV, c = x % DV;
      const size_t row = (b * ntok + t0 + j) * H + h;
      s_v[j][c] = G2 ? Elem<T>::load(write, row * DV + c) * Elem<T>::load(v, row * DV + c)
                     : Elem<T>::load(v, row * DV + c);
    }
    if (tid < nb) s_bt[tid] = G2 ? 1.f : Elem<T>::load(beta, (b * ntok + t0 + tid) * H + h);
    __syncthreads();

    for (int j = 0; j < nb; ++j) {
      const int par = (t0 + j) & 1;
      float u[4] = {0.f, 0.f, 0.f, 0.f}, p[4] = {0.f, 0.f, 0.f, 0.f};
      float qk = 0.f;  // q . k over this thread's rows, counted once per row (column quad 0)
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int r = row_of(i);
        const float kk = G2 ? s_e[j][r] : s_k[j][r], qq = s_q[j][r];
        if constexpr (CPX) {
          // rows 2p (i even) and 2p+1 (i odd) of this thread: z <- lambda z with
          // row 2p <- Re s_2p - Im s_2p+1, row 2p+1 <- Im s_2p + Re s_2p+1
          if ((i & 1) == 0) {
            const float lr = s_a[j][r], li = s_a[j][r + 1];
            const float4 x = s[i], y = s[i + 1];
            s[i] = make_float4(lr * x.x - li * y.x, lr * x.y - li * y.y, lr * x.z - li * y.z, lr * x.w - li * y.w);
            s[i + 1] = make_float4(li * x.x + lr * y.x, li * x.y + lr * y.y, li * x.z + lr * y.z, li * x.w + lr * y.w);
          }
        } else {
          const float a = s_a[j][r];
          s[i].x *= a; s[i].y *= a; s[i].z *= a; s[i].w *= a;
        }
        u[0] += kk * s[i].x; u[1] += kk * s[i].y; u[2] += kk * s[i].z; u[3] += kk * s[i].w;
        p[0] += qq * s[i].x; p[1] += qq * s[i].y; p[2] += qq * s[i].z; p[3] += qq * s[i].w;
        if (cq == 0) qk += qq * s_k[j][r];
      }
      // reduce the row groups that share a wave
#pragma unroll
      for (int off = TPR; off < 64; off <<= 1) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          u[jj] += __shfl_xor(u[jj], off);
          p[jj] += __shfl_xor(p[jj], off);
        }
        qk += __shfl_xor(qk, off);
      }
      if (lane < TPR) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          s_red[par][wave][0][4 * cq + jj] = u[jj];
          s_red[par][wave][1][4 * cq + jj] = p[jj];
        }
      }
      if (lane == 0) s_qk[par][wave] = qk;
      __syncthreads();
      float d[4];
      float qkt = 0.f;
#pragma unroll
      for (int w = 0; w < NWV; ++w) qkt += s_qk[par][w];
      const float bt = s_bt[j];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int c = 4 * cq + jj;
        float uu = 0.f, pp = 0.f;
#pragma unroll
        for (int w = 0; w < NWV; ++w) {
          uu += s_red[par][w][0][c];
          pp += s_red[par][w][1][c];
        }
        d[jj] = bt * (s_v[j][c] - uu);
        p[jj] = pp;
      }
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float kk = s_k[j][row_of(i)];
        s[i].x += kk * d[0]; s[i].y += kk * d[1]; s[i].z += kk * d[2]; s[i].w += kk * d[3];
      }
      if (rg == 0) {
        const size_t row = (b * ntok + t0 + j) * H + h;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) Elem<T>::store(o, row * DV + 4 * cq + jj, p[jj] + qkt * d[jj]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const f32x4_t t = {s[i].x, s[i].y, s[i].z, s[i].w};
    __builtin_nontemporal_store(t, &S[(size_t)row_of(i) * TPR + cq]);
  }
}

template <typename T, int DK, int DV, bool G2, bool CPX>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  hipLaunchKernelGGL((decode_kernel<T, DK, DV, G2, CPX>), dim3(a.BH), dim3(512), 0, (hipStream_t)a.stream,
                     a.q, a.k, a.v, a.alpha, a.beta, a.state, a.o, a.erase, a.write, a.ntok, a.H);
  return hipGetLastError();
}

template <typename T, bool G2, bool CPX = false>
static hipError_t launch_decode_d(const DecodeArgs& a) {
  if (a.dk == 64 && a.dv == 64) return launch_decode_t<T, 64, 64, G2, CPX>(a);
  if (a.dk == 64 && a.dv == 128) return launch_decode_t<T, 64, 128, G2, CPX>(a);
  if (a.dk == 128 && a.dv == 64) return launch_decode_t<T, 128, 64, G2, CPX>(a);
  return launch_decode_t<T, 128, 128, G2, CPX>(a);
}

hipError_t launch_decode(const DecodeArgs& a) {
  if (a.BH == 0) return hipSuccess;
  if (a.cpx) {
    if (a.erase) return hipErrorInvalidValue;
    return a.bf16 ? launch_decode_d<bf16_t, false, true>(a) : launch_decode_d<float, false, true>(a);
  }
  if (a.erase) return a.bf16 ? launch_decode_d<bf16_t, true>(a) : launch_decode_d<float, true>(a);
  return a.bf16 ? launch_decode_d<bf16_t, false>(a) : launch_decode_d<float, false>(a);
}

}  // namespace kda
