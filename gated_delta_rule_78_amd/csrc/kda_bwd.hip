// kda_bwd.hip -- gradients of the chunkwise KDA / CKDA forward (gfx950 only).
//
// The gradients of L = sum_t <dO_t, o_t> + <dS_T, S_T> with respect to q, k, v, alpha, beta
// and S_0, taken through the chunk form of the recurrence: the chunk-WY product form of the
// SFDA page ("El Teorema de Chunk-WY Constructivo") with the decay absorbed into the keys
// and queries as on the Gated DeltaNet-2 page (section 3, efficient chunkwise parallel
// training, whose gate-aware backward item asks for exactly this: the per-channel gates
// kept inside the gradients of the intra-chunk matrices).  Per chunk of C = 64 rows, with
// r_ij = prod_{l=j+1..i} alpha_l per key channel, gamma_i = r_(i,-1), rho_j = r_(C-1,j):
//   A = [sum_c q_ic k_jc r_ijc] (j <= i),  D = [sum_c k_ic k_jc r_ijc] (j < i),
//   M = (I + diag(beta) D)^-1,  Mt = M diag(beta),  W = Mt (K o gamma),
//   Delta = Mt V - W S,  O = (Q o gamma) S + A Delta,  S' = gamma_L o S + (K o rho)^T Delta.
// The adjoint of these steps, per chunk:
//   dDelta = (K o rho) dS' + A^T dO,   dS = gamma_L o dS' + (Q o gamma)^T dO - W^T dDelta,
//   d(Q o gamma) = dO S^T,  dA = (dO Delta^T) o low,  d(K o rho) = Delta dS'^T,
//   dW = -dDelta S^T,  dV = Mt^T dDelta,  dMt = (dDelta V^T + dW (K o gamma)^T) o low,
//   d(K o gamma) = Mt^T dW,  dbeta = colsum(dMt o M) + rowsum(dT o D),
//   dT = -(M^T dMt Mt^T) o strict-low,  dD = diag(beta) dT,
// then the decayed products (Zq_i = sum_j dA_ij k_j r_ij and its kin) and the gate gradient.
//
// Four kernels, everything in fp32 (inputs widened from bf16 or fp32; products on the fp32
// matrix cores, 16x16x4 steps):
//   bwd_records_kernel   per chunk: gate products, A, D, M, W
//   bwd_state_kernel     per (b, h, value tile), forward: chunk-start states S_n, Delta_n
//   bwd_adjoint_kernel   per (b, h, value tile), reverse: end-state adjoints dS'_n,
//                        dDelta_n and dS_0
//   bwd_grads_kernel     per chunk: dq, dk, dv, dalpha, dbeta
// The gate gradient never divides by a gate: d alpha_m is the sum over the pairs
// j < m <= i of the weight of r_ij times r_ij with alpha_m left out of the product
// (r_(i,m) r_(m-1,j)).  Inside each 16-row block that sum is a recursion over m; the
// pairs that reach outside the block enter through matrix products anchored at the block
// edges (every factor a product of gates, so bounded by one), which keeps exact zero gates
// exact.
#include "kda_common.h"
#include "kda_internal.h"
#include "kda_tile.h"

namespace kda {

namespace {

constexpr int NT = 256;   // threads per workgroup of the walks
constexpr int NTW = 512;  // threads per workgroup of the state walk (two waves per 16 columns)
constexpr int NTG = 512;  // threads per workgroup of the gradient kernel and, at d_k = 128, of the
                          // records kernel (two waves per SIMD)

// ---------------------------------------------------------------------------------------
// One 16x16 fp32 tile: acc[i][j] = sum_k fa(i, k) fb(k, j), K a multiple of 16.  Lane
// (n = lane & 15, g = lane >> 4) feeds A[n][k0 + g] and B[k0 + g][n]; the result holds
// element (4 g + r, n) in acc[r].  The operands of the next 16 k are loaded while the
// current four steps run.
template <class FA, class FB>
__device__ __forceinline__ f32x4_t tile_mm(int K, FA fa, FB fb) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float a0[4], b0[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    a0[t] = fa(n, 4 * t + g);
    b0[t] = fb(4 * t + g, n);
  }
#pragma unroll 1
  for (int k0 = 0; k0 < K; k0 += 16) {
    float a1[4], b1[4];
    if (k0 + 16 < K) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a1[t] = fa(n, k0 + 16 + 4 * t + g);
        b1[t] = fb(k0 + 16 + 4 * t + g, n);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#ifndef KDA_HOST_PASS
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[t], b0[t], acc, 0, 0, 0);
#endif
      a0[t] = a1[t];
      b0[t] = b1[t];
    }
  }
  return acc;
}

struct ChunkGeom {
  int b, h, n, t0, len;
};

// Chunk n of a chain (fixed-length batch: chain = b H + h; packed batch: chain =
// sequence H + h) and the index of its workspace block (fixed: chain NC + n; packed:
// h gmax + the sequence's first global chunk + n).
__device__ __forceinline__ ChunkGeom chain_chunk(const BwdArgs& a, int NC, int chain, int n, size_t* ws) {
  ChunkGeom q;
  q.n = n;
  q.h = chain % a.H;
  if (!a.ctab) {
    q.b = chain / a.H;
    q.t0 = n * C;
    q.len = min(C, a.T - q.t0);
    *ws = (size_t)chain * NC + n;
  } else {
    const int s = chain / a.H;
    q.b = 0;
    q.t0 = a.cs[s] + n * C;
    q.len = min(C, a.cs[s + 1] - q.t0);
    *ws = (size_t)q.h * a.gmax + a.cbase[s] + n;
  }
  return q;
}

// chunks in a chain
__device__ __forceinline__ int chain_chunks(const BwdArgs& a, int NC, int chain) {
  if (!a.ctab) return NC;
  const int s = chain / a.H;
  return (a.cs[s + 1] - a.cs[s] + C - 1) / C;
}

// the chunk of a per-chunk workgroup (fixed: blockIdx = chain NC + n; packed: blockIdx =
// h gmax + global chunk); false for a packed batch's workgroups past the last chunk
__device__ __forceinline__ bool block_chunk(const BwdArgs& a, int NC, ChunkGeom* q, size_t* ws,
                                            int blk = blockIdx.x) {
  if (!a.ctab) {
    *q = chain_chunk(a, NC, blk / NC, blk % NC, ws);
    return true;
  }
  const int gc = blk % a.gmax, h = blk / a.gmax;
  if (gc >= *a.ctotal) return false;
  *q = chain_chunk(a, NC, a.ctab[2 * gc] * a.H + h, a.ctab[2 * gc + 1], ws);
  return true;
}

// element offset of (b, t0, h, 0) in a [B, T, H, d] tensor
__device__ __forceinline__ size_t row0(const ChunkGeom& q, int T, int H, int d) {
  return (((size_t)q.b * T + q.t0) * H + q.h) * (size_t)d;
}

}  // namespace

namespace {

constexpr int VTW = 64;  // value columns per walk workgroup, 16 per wave

// four consecutive elements (i % 4 == 0) of an input tensor, widened
template <typename T>
__device__ __forceinline__ float4 ld4(const void* p, size_t i);
template <>
__device__ __forceinline__ float4 ld4<bf16_t>(const void* p, size_t i) {
  const uint2 w = *(const uint2*)((const uint16_t*)p + i);
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                     __uint_as_float(w.y & 0xFFFF0000u));
}
template <>
__device__ __forceinline__ float4 ld4<float>(const void* p, size_t i) {
  return *(const float4*)((const float*)p + i);
}

__device__ __forceinline__ f32x4_t zero4f() {
  f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  return z;
}
// Raw input words held in registers between a load and its use one step later: widening
// bf16 at the load would make the load's wait come at once, ahead of the matrix work.
template <typename T>
struct RawIn;
template <>
struct RawIn<bf16_t> {
  using v4 = uint2;
  using s1 = uint32_t;
  static __device__ __forceinline__ v4 load4(const void* p, size_t i) { return *(const uint2*)((const uint16_t*)p + i); }
  static __device__ __forceinline__ s1 load1(const void* p, size_t i) { return ((const uint16_t*)p)[i]; }
  static __device__ __forceinline__ f32x4_t widen(v4 w) {
    f32x4_t r = {__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u), __uint_as_float(w.y << 16),
                 __uint_as_float(w.y & 0xFFFF0000u)};
    return r;
  }
  static __device__ __forceinline__ float widen(s1 b) { return __uint_as_float(b << 16); }
};
template <>
struct RawIn<float> {
  using v4 = f32x4_t;
  using s1 = float;
  static __device__ __forceinline__ v4 load4(const void* p, size_t i) { return *(const f32x4_t*)((const float*)p + i); }
  static __device__ __forceinline__ s1 load1(const void* p, size_t i) { return ((const float*)p)[i]; }
  static __device__ __forceinline__ f32x4_t widen(v4 w) { return w; }
  static __device__ __forceinline__ float widen(s1 b) { return b; }
};

// Keeps the scheduler from moving instructions across this point: LDS reads issued before it
// stay ahead of the matrix-core work after it.
__device__ __forceinline__ void sched_fence() {
#ifndef KDA_HOST_PASS
  __builtin_amdgcn_sched_barrier(0);
#endif
}
// acc += sum_t A[4 slots] B[4 slots] over one 16-wide slice of the contraction
__device__ __forceinline__ void mfma4v(f32x4_t& acc, const f32x4_t& av, const float* bv) {
#ifndef KDA_HOST_PASS
#pragma unroll
  for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[t], bv[t], acc, 0, 0, 0);
#endif
}
__device__ __forceinline__ void mfma4v(f32x4_t& acc, const f32x4_t& av, const f32x4_t& bv) {
#ifndef KDA_HOST_PASS
#pragma unroll
  for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[t], bv[t], acc, 0, 0, 0);
#endif
}


// acc += sgn * A[row][k0 .. k0 + 15] B[k0 .. k0 + 15][n], this lane's A row in LDS at `arow`,
// fb(t) = B[k0 + 4 g + t][n]
template <class FB>
__device__ __forceinline__ void mm16(f32x4_t& acc, const float* arow, int k0, FB fb, float sgn = 1.f) {
  const int g = (threadIdx.x & 63) >> 4;
  const float4 a4 = *(const float4*)(arow + k0 + 4 * g);
  const float av[4] = {sgn * a4.x, sgn * a4.y, sgn * a4.z, sgn * a4.w};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#ifndef KDA_HOST_PASS
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[t], fb(t), acc, 0, 0, 0);
#endif
  }
  (void)av;
}

}  // namespace

namespace {
__device__ __forceinline__ float f4c(const float4& v, int t) {
  return t == 0 ? v.x : (t == 1 ? v.y : (t == 2 ? v.z : v.w));
}
__device__ __forceinline__ float4 mul4(const float4& a, const float4& b) {
  return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
}
__device__ __forceinline__ void mfma4(f32x4_t& acc, const float (&av)[4], const float (&bv)[4]) {
#ifndef KDA_HOST_PASS
#pragma unroll
  for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[t], bv[t], acc, 0, 0, 0);
#endif
}

// SFDA complex gates: key channels 2p, 2p+1 hold one complex coordinate (x = channel 2p,
// y = channel 2p+1); the gate of coordinate p multiplies it.  A real dot product over the
// channels is sum_p Re(conj(a_p) b_p), so the anchored operands of a decayed product carry
// conj() of the factor on the row side.
struct cf {
  float x, y;
};
__device__ __forceinline__ cf cmul(cf a, cf b) { return {a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x}; }
__device__ __forceinline__ cf cmulc(cf a, cf b) { return {a.x * b.x + a.y * b.y, a.y * b.x - a.x * b.y}; }  // a conj(b)
__device__ __forceinline__ cf cadd(cf a, cf b) { return {a.x + b.x, a.y + b.y}; }
__device__ __forceinline__ cf cscale(cf a, float s) { return {a.x * s, a.y * s}; }
__device__ __forceinline__ cf cconj(cf a) { return {a.x, -a.y}; }
__device__ __forceinline__ float comp(cf a, int e) { return e ? a.y : a.x; }
// the complex number of the pair holding channel c, from a per-channel array
__device__ __forceinline__ cf cpair(const float* p, int c) { return {p[c & ~1], p[c | 1]}; }
}  // namespace

// ---------------------------------------------------------------------------------------
// (d) of the records kernels: M = (I + diag(beta) D)^-1, diagonal blocks by substitution,
// then block rows I = 1..3: M_IJ = -M_II sum_{J <= K < I} (beta D)_IK M_KJ
template <int NTR>
__device__ __forceinline__ void records_inverse(const float* sD, float* sM, const float* sB, float (*sY)[16][17]) {
  constexpr int LC = C + 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, g = lane >> 4;
  if (tid < 4 * SUB) {  // (the thread's column stays in registers until it is complete)
    const int s = (tid / SUB) * SUB, col = tid % SUB;
    float x[SUB];
#pragma unroll
    for (int r = 0; r < SUB; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < r; ++j) acc += sD[(s + r) * LC + s + j] * x[j];
      x[r] = (r == col ? 1.f : 0.f) - sB[s + r] * acc;
    }
#pragma unroll
    for (int r = 0; r < SUB; ++r) sM[(s + r) * LC + s + col] = x[r];
  }
  __syncthreads();
  for (int I = 1; I < NB; ++I) {
    const int si = I * SUB;
    for (int J = wave; J < I; J += NTR / 64) {
      const int sj = J * SUB;
      const f32x4_t y = tile_mm(
          si - sj, [&](int r, int kk) { return sB[si + r] * sD[(si + r) * LC + sj + kk]; },
          [&](int kk, int col) { return sM[(sj + kk) * LC + sj + col]; });
#pragma unroll
      for (int r = 0; r < 4; ++r) sY[J][4 * g + r][n] = y[r];
    }
    __syncthreads();
    for (int J = wave; J < I; J += NTR / 64) {
      const int sj = J * SUB;
      const f32x4_t m = tile_mm(
          SUB, [&](int r, int kk) { return sM[(si + r) * LC + si + kk]; }, [&](int kk, int col) { return sY[J][kk][col]; });
#pragma unroll
      for (int r = 0; r < 4; ++r) sM[(si + 4 * g + r) * LC + sj + n] = -m[r];
    }
    __syncthreads();
  }
}

// (e) of the records kernels, after K o gamma (its complex form for SFDA) is staged in R0:
// W = M diag(beta) R0, then A, D, M to the workspace
template <int DK, int NTR>
__device__ __forceinline__ void records_w_out(float* ch, const BwdLayout& L, const float* R0, const float* sA,
                                              const float* sD, const float* sM, const float* sB) {
  constexpr int LK = DK + 4, LC = C + 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, g = lane >> 4;
  for (int job = wave; job < 4 * (DK / 16); job += NTR / 64) {
    const int I = job / (DK / 16), ct = job % (DK / 16), c = 16 * ct + n;
    f32x4_t acc = zero4f();
#pragma unroll
    for (int k0 = 0; k0 < C; k0 += 16) {
      float av[4], bv[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int j = k0 + 4 * g + t;
        av[t] = sM[(16 * I + n) * LC + j] * sB[j];
        bv[t] = R0[j * LK + c];
      }
      mfma4(acc, av, bv);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) ch[L.W + (16 * I + 4 * g + r) * DK + c] = acc[r];
  }
  for (int x = tid; x < C * C; x += NTR) {
    const int i = x / C, j = x % C;
    ch[L.A + x] = sA[i * LC + j];
    ch[L.D + x] = sD[i * LC + j];
    ch[L.M + x] = sM[i * LC + j];
  }
}

// ---------------------------------------------------------------------------------------
// bwd_records_kernel: one workgroup per (b, h, chunk).  A (channel, block) item keeps the
// 16 rows of alpha, q, k of its channel and block in registers throughout.
//   (a) gate products: pi (from the block start, inclusive), sigma (to the block end,
//       exclusive), block totals, gamma (from the chunk start), rho (to the chunk end,
//       exclusive);
//   (b) the six off-diagonal 16x16 tiles (I > J) of A and D, anchored at row s_I - 1:
//       r_ij = pi_i * sigma_j * (the whole blocks between J and I);
//   (c) the diagonal tiles, one matrix-core product per level lam = 8, 4, 2, 1: a pair
//       (i, j) of one block whose local indices differ first in bit lam has
//       r_ij = F_i B_j, F the product from the start of i's lam-half through i, B the
//       product after j through the end of j's lam-half; level 0 gives A's diagonal;
//   (d) M = (I + diag(beta) D)^-1 by blocks; (e) W = M diag(beta) (K o gamma).
template <typename T, int DK, bool G2>
__global__ __launch_bounds__(DK == 128 ? NTG : NT) void bwd_records_kernel(BwdArgs a, int NC) {
  constexpr int NTR = DK == 128 ? NTG : NT;  // one (channel, block) item per thread
  constexpr int LK = DK + 4, LC = C + 1, NI = DK * NB / NTR;  // items per thread
  static_assert(NI >= 1 && DK * NB % NTR == 0, "items");
  __shared__ float sR[3 * C * LK];  // operand staging, reused by (b), (c), (e)
  __shared__ float sA[C * LC], sD[C * LC], sM[C * LC];
  __shared__ float sPib[NB * DK], sB[C], sY[3][16][17];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, g = lane >> 4;
  const BwdLayout L(DK, a.Dv);
  ChunkGeom cg;
  size_t wsi;
  if (!block_chunk(a, NC, &cg, &wsi)) return;
  const int len = cg.len;
  float* ch = a.ws + wsi * L.total;
  const size_t kb = row0(cg, a.T, a.H, DK), ks = (size_t)a.H * DK;
  const size_t bb = ((size_t)cg.b * a.T + cg.t0) * a.H + cg.h;
  float *R0 = sR, *R1 = sR + C * LK, *R2 = sR + 2 * C * LK;

  // ---- (a) items (c, I): load, block products
  // xv: the row operand of T and of W: k (KDA, beta applied in the inverse) or the
  // Gated DeltaNet-2 erase vector b o k
  float al[NI][SUB], qv[NI][SUB], kv[NI][SUB], xv[NI][SUB], pi[NI][SUB], sg[NI][SUB];
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int item = tid + it * NTR, c = item % DK, I = item / DK;
#pragma unroll
    for (int r = 0; r < SUB; ++r) {
      const int i = I * SUB + r;
      const bool in = i < len;
      al[it][r] = in ? Elem<T>::load(a.alpha, kb + i * ks + c) : 1.f;
      qv[it][r] = in ? Elem<T>::load(a.q, kb + i * ks + c) : 0.f;
      kv[it][r] = in ? Elem<T>::load(a.k, kb + i * ks + c) : 0.f;
      xv[it][r] = G2 ? (in ? Elem<T>::load(a.erase, kb + i * ks + c) : 0.f) * kv[it][r] : kv[it][r];
    }
  }
  for (int i = tid; i < C; i += NTR) sB[i] = G2 ? 1.f : (i < len ? Elem<T>::load(a.beta, bb + (size_t)i * a.H) : 0.f);
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int item = tid + it * NTR, c = item % DK, I = item / DK;
    float p = 1.f;
#pragma unroll
    for (int r = 0; r < SUB; ++r) {
      p *= al[it][r];
      pi[it][r] = p;
    }
    sPib[I * DK + c] = p;
    ch[L.pib + I * DK + c] = p;
    float sf = 1.f;
#pragma unroll
    for (int r = SUB - 1; r >= 0; --r) {
      sg[it][r] = sf;
      sf *= al[it][r];
    }
#pragma unroll
    for (int r = 0; r < SUB; ++r) {
      ch[L.pin + (I * SUB + r) * DK + c] = pi[it][r];
      ch[L.sig + (I * SUB + r) * DK + c] = sg[it][r];
    }
  }
  for (int x = tid; x < C * C; x += NTR) {
    const int i = x / C, j = x % C;
    if (j / SUB > i / SUB) sA[i * LC + j] = sD[i * LC + j] = sM[i * LC + j] = 0.f;
  }
  __syncthreads();
  // gamma, rho; the anchored operands of (b): q o pi, k o pi, k o sigma
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int item = tid + it * NTR, c = item % DK, I = item / DK;
    float before = 1.f, after = 1.f;
#pragma unroll
    for (int J = 0; J < NB; ++J) {
      if (J < I) before *= sPib[J * DK + c];
      if (J > I) after *= sPib[J * DK + c];
    }
#pragma unroll
    for (int r = 0; r < SUB; ++r) {
      const int i = I * SUB + r;
      ch[L.gam + i * DK + c] = before * pi[it][r];
      ch[L.rho + i * DK + c] = after * sg[it][r];
      ch[L.KR + i * DK + c] = kv[it][r] * (after * sg[it][r]);
      ch[L.QG + i * DK + c] = qv[it][r] * (before * pi[it][r]);
      R0[i * LK + c] = qv[it][r] * pi[it][r];
      R1[i * LK + c] = xv[it][r] * pi[it][r];
      R2[i * LK + c] = kv[it][r] * sg[it][r];
    }
  }
  __syncthreads();

  // ---- (b) off-diagonal tiles: A[I, J] = (q o pi)_I ((k o sigma) btw)_J^T, D likewise
  for (int job = wave; job < 12; job += NTR / 64) {
    // tiles (I, J) = (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
    const int mat = job / 6, p = job % 6, I = p < 1 ? 1 : (p < 3 ? 2 : 3), J = p - I * (I - 1) / 2;
    const float* xrow = (mat ? R1 : R0) + (16 * I + n) * LK;
    const float* yrow = R2 + (16 * J + n) * LK;
    f32x4_t acc = zero4f();
#pragma unroll
    for (int k0 = 0; k0 < DK; k0 += 16) {
      const float4 y4 = *(const float4*)(yrow + k0 + 4 * g);
      float w[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        w[t] = 1.f;
        for (int x = J + 1; x < I; ++x) w[t] *= sPib[x * DK + k0 + 4 * g + t];
      }
      mm16(acc, xrow, k0, [&](int t) { return f4c(y4, t) * w[t]; });
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) (mat ? sD : sA)[(16 * I + 4 * g + r) * LC + 16 * J + n] = acc[r];
  }

  // ---- (c) diagonal tiles by levels lam = 8, 4, 2, 1, then 0 (A's diagonal)
  for (int lam = 8; lam >= 0; lam = lam > 1 ? lam / 2 : lam - 1) {
    __syncthreads();  // the previous readers of the staging region are done
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int item = tid + it * NTR, c = item % DK, I = item / DK;
      float Fv[SUB], Bv[SUB];
      if (lam > 0) {
        float p = 1.f;
#pragma unroll
        for (int r = 0; r < SUB; ++r) {
          if ((r & (lam - 1)) == 0) p = 1.f;
          p *= al[it][r];
          Fv[r] = p;
        }
        p = 1.f;
#pragma unroll
        for (int r = SUB - 1; r >= 0; --r) {
          if (((r + 1) & (lam - 1)) == 0) p = 1.f;
          Bv[r] = p;
          p *= al[it][r];
        }
      } else {
#pragma unroll
        for (int r = 0; r < SUB; ++r) Fv[r] = Bv[r] = 1.f;
      }
#pragma unroll
      for (int r = 0; r < SUB; ++r) {
        const int i = I * SUB + r;
        R0[i * LK + c] = qv[it][r] * Fv[r];
        R1[i * LK + c] = xv[it][r] * Fv[r];
        R2[i * LK + c] = kv[it][r] * Bv[r];
      }
    }
    __syncthreads();
    for (int job = wave; job < 8; job += NTR / 64) {  // level 0 also clears D's diagonal and upper part
      const int I = job % NB, mat = job / NB, si = 16 * I;
      const float* xrow = (mat ? R1 : R0) + (si + n) * LK;
      const float* yrow = R2 + (si + n) * LK;
      f32x4_t acc = zero4f();
#pragma unroll
      for (int k0 = 0; k0 < DK; k0 += 16) {
        const float4 y4 = *(const float4*)(yrow + k0 + 4 * g);
        mm16(acc, xrow, k0, [&](int t) { return f4c(y4, t); });
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int il = 4 * g + r, jl = n;  // local row, column
        bool keep;
        if (lam > 0)
          keep = (il & lam) && !(jl & lam) && ((il & ~(2 * lam - 1)) == (jl & ~(2 * lam - 1)));
        else
          keep = il == jl && !mat;
        if (keep) (mat ? sD : sA)[(si + il) * LC + si + jl] = acc[r];
        else if (lam == 0 && jl >= il) (mat ? sD : sA)[(si + il) * LC + si + jl] = 0.f;
      }
    }
  }
  __syncthreads();

  records_inverse<NTR>(sD, sM, sB, sY);

  // ---- (e) K o gamma into the staging region; W = M diag(beta) (K o gamma); A, D, M out
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int item = tid + it * NTR, c = item % DK, I = item / DK;
    float before = 1.f;
#pragma unroll
    for (int J = 0; J < NB; ++J)
      if (J < I) before *= sPib[J * DK + c];
#pragma unroll
    for (int r = 0; r < SUB; ++r) R0[(I * SUB + r) * LK + c] = xv[it][r] * pi[it][r] * before;
  }
  __syncthreads();
  records_w_out<DK, NTR>(ch, L, R0, sA, sD, sM, sB);
}

// ---------------------------------------------------------------------------------------
// bwd_records_cpx_kernel: the records for SFDA complex gates (SFDA page, "Arquitectura
// Central").  Same items, anchors and levels as bwd_records_kernel, with every gate product
// complex per key-channel pair: a thread keeps its pair's gate, q and k (both channels,
// so the two threads of a pair do the same complex arithmetic) and writes its own channel's
// component.  For i in block I and j in block J < I, r_ij = pi_i (blocks between) sigma_j,
// and A_ij = sum_p Re(conj(q_ip) r_ijp k_jp) = sum over channels of (q conj(pi))_i times
// ((blocks between) sigma k)_j; gamma, rho, pi, sigma and the block totals are stored as
// (Re, Im) in the pair's channels; Q o gamma becomes q conj(gamma), K o gamma k conj(gamma)
// and K o rho rho k.
template <typename T, int DK>
__global__ __launch_bounds__(DK == 128 ? NTG : NT) void bwd_records_cpx_kernel(BwdArgs a, int NC) {
  constexpr int NTR = DK == 128 ? NTG : NT;
  constexpr int LK = DK + 4, LC = C + 1, NI = DK * NB / NTR;
  static_assert(NI >= 1 && DK * NB % NTR == 0, "items");
  __shared__ float sR[3 * C * LK];
  __shared__ float sA[C * LC], sD[C * LC], sM[C * LC];
  __shared__ float sPib[NB * DK], sB[C], sY[3][16][17];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, g = lane >> 4;
  const BwdLayout L(DK, a.Dv);
  ChunkGeom cg;
  size_t wsi;
  if (!block_chunk(a, NC, &cg, &wsi)) return;
  const int len = cg.len;
  float* ch = a.ws + wsi * L.total;
  const size_t kb = row0(cg, a.T, a.H, DK), ks = (size_t)a.H * DK;
  const size_t bb = ((size_t)cg.b * a.T + cg.t0) * a.H + cg.h;
  float *R0 = sR, *R1 = sR + C * LK, *R2 = sR + 2 * C * LK;

  // ---- (a) items (c, I): the pair's gate, q, k; pi, sigma and the block total
  cf al[NI][SUB], qv[NI][SUB], kv[NI][SUB];
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int item = tid + it * NTR, c0 = (item % DK) & ~1, I = item / DK;
#pragma unroll
    for (int r = 0; r < SUB; ++r) {
      const int i = I * SUB + r;
      const bool in = i < len;
      const size_t o = kb + i * ks + c0;
      al[it][r] = in ? cf{Elem<T>::load(a.alpha, o), Elem<T>::load(a.alpha, o + 1)} : cf{1.f, 0.f};
      qv[it][r] = in ? cf{Elem<T>::load(a.q, o), Elem<T>::load(a.q, o + 1)} : cf{0.f, 0.f};
      kv[it][r] = in ? cf{Elem<T>::load(a.k, o), Elem<T>::load(a.k, o + 1)} : cf{0.f, 0.f};
    }
  }
  for (int i = tid; i < C; i += NTR) sB[i] = i < len ? Elem<T>::load(a.beta, bb + (size_t)i * a.H) : 0.f;
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int item = tid + it * NTR, c = item % DK, I = item / DK, e = c & 1;
    cf p = {1.f, 0.f};
#pragma unroll
    for (int r = 0; r < SUB; ++r) {
      p = cmul(p, al[it][r]);
      ch[L.pin + (I * SUB + r) * DK + c] = comp(p, e);
    }
    sPib[I * DK + c] = comp(p, e);
    ch[L.pib + I * DK + c] = comp(p, e);
    cf sf = {1.f, 0.f};
#pragma unroll
    for (int r = SUB - 1; r >= 0; --r) {
      ch[L.sig + (I * SUB + r) * DK + c] = comp(sf, e);
      sf = cmul(sf, al[it][r]);
    }
  }
  for (int x = tid; x < C * C; x += NTR) {
    const int i = x / C, j = x % C;
    if (j / SUB > i / SUB) sA[i * LC + j] = sD[i * LC + j] = sM[i * LC + j] = 0.f;
  }
  __syncthreads();
  // gamma, rho, Q o gamma, K o rho; the anchored operands of (b): q conj(pi), k conj(pi), sigma k
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int item = tid + it * NTR, c = item % DK, I = item / DK, e = c & 1;
    cf before = {1.f, 0.f}, after = {1.f, 0.f};
#pragma unroll
    for (int J = 0; J < NB; ++J) {
      if (J < I) before = cmul(before, cpair(sPib + J * DK, c));
      if (J > I) after = cmul(after, cpair(sPib + J * DK, c));
    }
    cf sgl[SUB];
    cf sf = {1.f, 0.f};
#pragma unroll
    for (int r = SUB - 1; r >= 0; --r) {
      sgl[r] = sf;
      sf = cmul(sf, al[it][r]);
    }
    cf p = {1.f, 0.f};
#pragma unroll
    for (int r = 0; r < SUB; ++r) {
      const int i = I * SUB + r;
      p = cmul(p, al[it][r]);
      const cf gam = cmul(before, p), rho = cmul(after, sgl[r]);
      ch[L.gam + i * DK + c] = comp(gam, e);
      ch[L.rho + i * DK + c] = comp(rho, e);
      ch[L.KR + i * DK + c] = comp(cmul(rho, kv[it][r]), e);
      ch[L.QG + i * DK + c] = comp(cmulc(qv[it][r], gam), e);
      R0[i * LK + c] = comp(cmulc(qv[it][r], p), e);
      R1[i * LK + c] = comp(cmulc(kv[it][r], p), e);
      R2[i * LK + c] = comp(cmul(sgl[r], kv[it][r]), e);
    }
  }
  __syncthreads();

  // ---- (b) off-diagonal tiles; the blocks between J and I multiply the column operand's pairs
  for (int job = wave; job < 12; job += NTR / 64) {
    const int mat = job / 6, p = job % 6, I = p < 1 ? 1 : (p < 3 ? 2 : 3), J = p - I * (I - 1) / 2;
    const float* xrow = (mat ? R1 : R0) + (16 * I + n) * LK;
    const float* yrow = R2 + (16 * J + n) * LK;
    f32x4_t acc = zero4f();
#pragma unroll
    for (int k0 = 0; k0 < DK; k0 += 16) {
      const float4 y4 = *(const float4*)(yrow + k0 + 4 * g);
      const int cb = k0 + 4 * g;  // channels cb .. cb + 3: pairs (cb, cb + 1), (cb + 2, cb + 3)
      cf w0 = {1.f, 0.f}, w1 = {1.f, 0.f};
      for (int x = J + 1; x < I; ++x) {
        w0 = cmul(w0, cpair(sPib + x * DK, cb));
        w1 = cmul(w1, cpair(sPib + x * DK, cb + 2));
      }
      const cf y0 = cmul(cf{y4.x, y4.y}, w0), y1 = cmul(cf{y4.z, y4.w}, w1);
      const float yv[4] = {y0.x, y0.y, y1.x, y1.y};
      mm16(acc, xrow, k0, [&](int t) { return yv[t]; });
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) (mat ? sD : sA)[(16 * I + 4 * g + r) * LC + 16 * J + n] = acc[r];
  }

  // ---- (c) diagonal tiles by levels lam = 8, 4, 2, 1, then 0 (A's diagonal)
  for (int lam = 8; lam >= 0; lam = lam > 1 ? lam / 2 : lam - 1) {
    __syncthreads();
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int item = tid + it * NTR, c = item % DK, I = item / DK, e = c & 1;
      cf Fv[SUB], Bv[SUB];
      if (lam > 0) {
        cf p = {1.f, 0.f};
#pragma unroll
        for (int r = 0; r < SUB; ++r) {
          if ((r & (lam - 1)) == 0) p = cf{1.f, 0.f};
          p = cmul(p, al[it][r]);
          Fv[r] = p;
        }
        p = cf{1.f, 0.f};
#pragma unroll
        for (int r = SUB - 1; r >= 0; --r) {
          if (((r + 1) & (lam - 1)) == 0) p = cf{1.f, 0.f};
          Bv[r] = p;
          p = cmul(p, al[it][r]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < SUB; ++r) Fv[r] = Bv[r] = cf{1.f, 0.f};
      }
#pragma unroll
      for (int r = 0; r < SUB; ++r) {
        const int i = I * SUB + r;
        R0[i * LK + c] = comp(cmulc(qv[it][r], Fv[r]), e);
        R1[i * LK + c] = comp(cmulc(kv[it][r], Fv[r]), e);
        R2[i * LK + c] = comp(cmul(Bv[r], kv[it][r]), e);
      }
    }
    __syncthreads();
    for (int job = wave; job < 8; job += NTR / 64) {
      const int I = job % NB, mat = job / NB, si = 16 * I;
      const float* xrow = (mat ? R1 : R0) + (si + n) * LK;
      const float* yrow = R2 + (si + n) * LK;
      f32x4_t acc = zero4f();
#pragma unroll
      for (int k0 = 0; k0 < DK; k0 += 16) {
        const float4 y4 = *(const float4*)(yrow + k0 + 4 * g);
        mm16(acc, xrow, k0, [&](int t) { return f4c(y4, t); });
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int il = 4 * g + r, jl = n;
        bool keep;
        if (lam > 0)
          keep = (il & lam) && !(jl & lam) && ((il & ~(2 * lam - 1)) == (jl & ~(2 * lam - 1)));
        else
          keep = il == jl && !mat;
        if (keep) (mat ? sD : sA)[(si + il) * LC + si + jl] = acc[r];
        else if (lam == 0 && jl >= il) (mat ? sD : sA)[(si + il) * LC + si + jl] = 0.f;
      }
    }
  }
  __syncthreads();

  records_inverse<NTR>(sD, sM, sB, sY);

  // ---- (e) k conj(gamma) into the staging region; W = M diag(beta) (K o gamma); A, D, M out
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int item = tid + it * NTR, c = item % DK, I = item / DK, e = c & 1;
    cf before = {1.f, 0.f};
#pragma unroll
    for (int J = 0; J < NB; ++J)
      if (J < I) before = cmul(before, cpair(sPib + J * DK, c));
    cf p = {1.f, 0.f};
#pragma unroll
    for (int r = 0; r < SUB; ++r) {
      p = cmul(p, al[it][r]);
      R0[(I * SUB + r) * LK + c] = comp(cmulc(kv[it][r], cmul(before, p)), e);
    }
  }
  __syncthreads();
  records_w_out<DK, NTR>(ch, L, R0, sA, sD, sM, sB);
}

// ---------------------------------------------------------------------------------------
// The two walks.  One workgroup per (b, h, 64 value columns); wave w owns the 16 columns
// v0 + 16 w .. v0 + 16 w + 15 (the value columns of the state evolve independently) and
// keeps them in matrix-core accumulators for the whole walk: DK / 16 tiles, element
// (16 I + 4 g + r, n) in register r of tile I.  The four steps of each 16-wide slice of a
// product take k-slot k0 + 4 g + t at step t, so an accumulator tile is itself the B
// operand of a product over its rows: neither the state nor Delta leaves the registers.
// Only the chunk's shared operands are staged in LDS (row strides padded by four floats),
// with vector loads issued together.

// A split walk (few chains over long sequences): each chain is cut into nseg segments of
// segc chunks that are walked in parallel -- from a zero start with the real inputs (end
// states B_g), from the identity with the inputs read as zero (the d_k x d_k transfers
// P_g, cols = d_k), then, after a scan of the segment start states, from those start
// states with the per-chunk writes.  nseg = 1 is the plain walk.
// A launch covers segments seg_lo ... seg_lo + nsub - 1.  Segment lengths: c0, c1, then
// segc each (the last one what remains), counted from the sequence's start, or (mirror)
// from its end, so that the two short segments are the last two.
struct WalkSplit {
  int nseg = 1, segc = 0, cols = 0, flags = 0;
  const float* start = nullptr;  // [chains nseg][d_k][cols], NULL: zero (nseg > 1)
  float* end = nullptr;          // [chains nseg][d_k][cols], or NULL
  int nsub = 1, seg_lo = 0, c0 = 0, c1 = 0, mirror = 0;
};
// no per-chunk writes; inputs read as zero; start from the identity; start from the
// chain's own start (S_0, or dS_T for the adjoint walk) instead of `start`; end state
// written as the start of the next (kWEndNext) or previous (kWEndPrev) segment
enum : int { kWNoWrite = 1, kWZeroIn = 2, kWIdentity = 4, kWHead = 8, kWEndNext = 16, kWEndPrev = 32 };

// the descriptor of this workgroup's walk, picked field by field (a select of the whole
// struct is kept in scratch memory)
__device__ __forceinline__ WalkSplit pick_split(const WalkSplit& x, const WalkSplit& y, bool second) {
  WalkSplit w;
  w.nseg = second ? y.nseg : x.nseg;
  w.segc = second ? y.segc : x.segc;
  w.cols = second ? y.cols : x.cols;
  w.flags = second ? y.flags : x.flags;
  w.start = second ? y.start : x.start;
  w.end = second ? y.end : x.end;
  w.nsub = second ? y.nsub : x.nsub;
  w.seg_lo = second ? y.seg_lo : x.seg_lo;
  w.c0 = second ? y.c0 : x.c0;
  w.c1 = second ? y.c1 : x.c1;
  w.mirror = second ? y.mirror : x.mirror;
  return w;
}

// chunks [c0, c0 + nch) of segment `seg` of a chain of nall chunks
__device__ __forceinline__ void walk_seg_range(const WalkSplit& sp, int seg, int nall, int& c0, int& nch) {
  const int g = sp.mirror ? sp.nseg - 1 - seg : seg;
  const int st = g == 0 ? 0 : g == 1 ? sp.c0 : sp.c0 + sp.c1 + (g - 2) * sp.segc;
  const int ln = g == 0 ? sp.c0 : g == 1 ? sp.c1 : sp.segc;
  if (!sp.mirror) {
    c0 = st;
    nch = max(0, min(ln, nall - st));
  } else {
    const int hi = max(0, nall - st), lo = max(0, nall - st - ln);
    c0 = lo;
    nch = hi - lo;
  }
}

// bwd_state_kernel: chunks in order; writes the chunk-start state S_n and Delta_n.  The
// next chunk's operands are loaded into registers while the current one computes.
// CPX: SFDA complex gates -- gamma_L multiplies the state's row pairs (2p, 2p+1), which
// are registers r, r + 1 (r even) of one lane.
template <typename T, int DK, bool G2, bool CPX, int WMODE = 0>
__global__ __launch_bounds__(NTW) void bwd_state_kernel(BwdArgs a, int NC, WalkSplit sp0, WalkSplit sp1,
                                                        int nfirst) {
  // WMODE 0: one walk per chain (the descriptors are ignored, none of the split logic is
  // compiled); 1: one segment walk per workgroup (sp0); 2: a paired launch, workgroups from
  // nfirst on run the second walk (sp1).  The plain walk keeps its registers.
  const bool second = WMODE == 2 && (int)blockIdx.x >= nfirst;
  const WalkSplit sp = WMODE == 2 ? pick_split(sp0, sp1, second) : WMODE == 1 ? sp0 : WalkSplit{};
  const int bid = second ? (int)blockIdx.x - nfirst : (int)blockIdx.x;
  constexpr int LM = C + 4, LW = DK + 4, LV = VTW + 4;
  constexpr int NM = C * C / 4 / NTW, NW = C * DK / 4 / NTW, NV = C * VTW / 4 / NTW;
  constexpr int NH = DK / 32;  // state row blocks per wave: two waves share 16 columns
  __shared__ __attribute__((aligned(16))) float sM[C * LM], sW[C * LW], sKrT[DK * LM], sV[C * LV], sGl[DK];
  __shared__ __attribute__((aligned(16))) f32x4_t sX[8 * 4 * 64];  // partial Delta of each wave
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, g = lane >> 4;
  const int cw = wave & 3, hh = wave >> 2;  // column slice; half of the state rows (blocks hh NH ..)
  const bool split = sp.nseg > 1;
  const int dv = a.Dv, cols = split ? sp.cols : dv, ntile = cols / VTW;
  const int cl = bid / ntile, v0 = (bid % ntile) * VTW;  // cl: chain (and segment) of this launch
  const int bh = cl / sp.nsub, seg = sp.seg_lo + cl % sp.nsub;  // bh: the chain (b H + h, or sequence H + h)
  const int cs = bh * sp.nseg + seg;  // index of the segment's start and end states
  const int nall = chain_chunks(a, NC, bh);
  int c0 = 0, nch = nall;
  if (split) walk_seg_range(sp, seg, nall, c0, nch);
  const bool zero_in = sp.flags & kWZeroIn, no_write = sp.flags & kWNoWrite;
  const int col = v0 + 16 * cw + n;  // this lane's state column
  const BwdLayout L(DK, dv);
  f32x4_t S[NH];  // rows of blocks hh NH + I
#pragma unroll
  for (int I = 0; I < NH; ++I)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * (hh * NH + I) + 4 * g + r;
      if (sp.flags & kWIdentity)
        S[I][r] = row == col ? 1.f : 0.f;
      else if (split && !(sp.flags & kWHead))
        S[I][r] = sp.start ? sp.start[((size_t)cs * DK + row) * cols + col] : 0.f;
      else
        S[I][r] = a.s0 ? a.s0[((size_t)bh * DK + row) * dv + col] : 0.f;
    }
#ifndef KDA_HOST_PASS
  // the start values are in registers before the walk: otherwise the compiler keeps their
  // loads pending into the loop and waits on every outstanding load at the first store
  __builtin_amdgcn_s_waitcnt(0);
#endif
  // one chunk's operands in registers: M; W; K o rho; V and beta (or, Gated DeltaNet-2,
  // the write gate w: M (w o V)); gamma_last.  Step st
  // moves chunk st - 1 from registers to LDS, issues the loads of chunk st, then computes
  // chunk st - 1 while they are in flight.
  using RI = RawIn<T>;
  f32x4_t pm[NM], pw[NW], pk[NW];
  typename RI::v4 pv[NV], pwg[G2 ? NV : 1];
  typename RI::s1 pb[NV];
  float pg = 0.f;
  int plen = 0;  // rows of the loaded v tile that are inside the chunk (0: v read as zero)
  size_t wnext = 0;  // workspace slot of the chunk loaded last (chunk tables are read once)
  for (int st = 0; st <= nch; ++st) {
    const size_t wcur = wnext;
    if (st > 0) {
      __syncthreads();  // the previous chunk's LDS reads are done
#pragma unroll
      for (int it = 0; it < NM; ++it) {
        const int x = tid + it * NTW, i = x / (C / 4), j = 4 * (x % (C / 4));
        *(f32x4_t*)(sM + i * LM + j) = pm[it];
      }
#pragma unroll
      for (int it = 0; it < NW; ++it) {
        const int x = tid + it * NTW, i = x / (DK / 4), c = 4 * (x % (DK / 4));
        const int ti = x % C, tc = 4 * (x / C);  // transposed tiles: a wave's lanes take consecutive rows
        *(f32x4_t*)(sW + i * LW + c) = pw[it];
        sKrT[(tc + 0) * LM + ti] = pk[it].x;
        sKrT[(tc + 1) * LM + ti] = pk[it].y;
        sKrT[(tc + 2) * LM + ti] = pk[it].z;
        sKrT[(tc + 3) * LM + ti] = pk[it].w;
      }
#pragma unroll
      for (int it = 0; it < NV; ++it) {
        const int x = tid + it * NTW, j = x / (VTW / 4), c = 4 * (x % (VTW / 4));
        const bool in = j < plen;
        if (G2) {
          *(f32x4_t*)(sV + j * LV + c) = in ? RI::widen(pv[it]) * RI::widen(pwg[G2 ? it : 0]) : zero4f();
        } else {
          const float b = RI::widen(pb[it]);
          *(f32x4_t*)(sV + j * LV + c) = in ? RI::widen(pv[it]) * b : zero4f();
        }
      }
      if (tid < DK) sGl[tid] = pg;
      __syncthreads();
    }
    if (st < nch) {
      size_t wsl;
      const ChunkGeom cg = chain_chunk(a, NC, bh, c0 + st, &wsl);
      wnext = wsl;
      const float* cl = a.ws + wsl * L.total;
      const size_t vb = row0(cg, a.T, a.H, dv), vs = (size_t)a.H * dv;
      const size_t bb = ((size_t)cg.b * a.T + cg.t0) * a.H + cg.h;
      // loads are unconditional (rows past the chunk clamped to its last row, masked when
      // staged), so that no wait on them is forced before the chunk's products
      plen = zero_in ? 0 : cg.len;  // the transfer walk reads v as zero
      const int lastr = max(cg.len - 1, 0);
#pragma unroll
      for (int it = 0; it < NM; ++it) {
        const int x = tid + it * NTW, i = x / (C / 4), j = 4 * (x % (C / 4));
        pm[it] = *(const f32x4_t*)(cl + L.M + i * C + j);
      }
#pragma unroll
      for (int it = 0; it < NW; ++it) {
        const int x = tid + it * NTW, i = x / (DK / 4), c = 4 * (x % (DK / 4));
        const int ti = x % C, tc = 4 * (x / C);
        pw[it] = *(const f32x4_t*)(cl + L.W + i * DK + c);
        pk[it] = *(const f32x4_t*)(cl + L.KR + ti * DK + tc);
      }
#pragma unroll
      for (int it = 0; it < NV; ++it) {
        const int x = tid + it * NTW, j = x / (VTW / 4), c = 4 * (x % (VTW / 4));
        const int jr = min(j, lastr);
        pv[it] = RI::load4(a.v, vb + jr * vs + v0 + c);
        if (G2)
          pwg[G2 ? it : 0] = RI::load4(a.write, vb + jr * vs + v0 + c);
        else
          pb[it] = RI::load1(a.beta, bb + (size_t)jr * a.H);
      }
      pg = cl[L.gam + (C - 1) * DK + min(tid, DK - 1)];  // unconditional: no branch around the load
    }
    if (st == 0) continue;
    const int nc = st - 1;
    float* ch = a.ws + wcur * L.total;
    if (!no_write) {
#pragma unroll
      for (int I = 0; I < NH; ++I)
#pragma unroll
        for (int r = 0; r < 4; ++r) ch[L.S + (16 * (hh * NH + I) + 4 * g + r) * dv + col] = S[I][r];
    }
    // Delta = M (beta o V) - W S, then S' = gamma_L o S + (K o rho)^T Delta.  The two waves
    // of a column slice each hold half of the state rows: each forms the part of Delta
    // over its rows (and half of M (beta o V)), the parts meet through LDS, and each
    // advances its own rows.  The A operands of the next row block are read from LDS while
    // the current one multiplies.
    float bvv[2][4];  // B operands shared by every row block: this wave's columns of beta o V
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int t = 0; t < 4; ++t) bvv[q][t] = sV[(16 * (2 * hh + q) + 4 * g + t) * LV + 16 * cw + n];
    f32x4_t am[2][2], aw[2][NH], ak[2][4], agl[2];
    auto load_d = [&](int b, int I) {
      const float* mrow = sM + (16 * I + n) * LM + 4 * g + 32 * hh;
      const float* wrow = sW + (16 * I + n) * LW + 4 * g + 16 * NH * hh;
#pragma unroll
      for (int q = 0; q < 2; ++q) am[b][q] = *(const f32x4_t*)(mrow + 16 * q);
#pragma unroll
      for (int kt = 0; kt < NH; ++kt) aw[b][kt] = *(const f32x4_t*)(wrow + 16 * kt);
    };
    auto load_s = [&](int b, int I) {  // I: this wave's row block (global block hh NH + I)
      const float* krow = sKrT + (16 * (hh * NH + I) + n) * LM + 4 * g;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) ak[b][kt] = *(const f32x4_t*)(krow + 16 * kt);
      agl[b] = *(const f32x4_t*)(sGl + 16 * (hh * NH + I) + 4 * g);
    };
    load_d(0, 0);
    sched_fence();
    f32x4_t Dl[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      if (I + 1 < 4)
        load_d((I + 1) & 1, I + 1);
      else
        load_s(0, 0);
      sched_fence();
      f32x4_t acc = zero4f(), accw = zero4f();
#pragma unroll
      for (int q = 0; q < 2; ++q) mfma4v(acc, am[I & 1][q], bvv[q]);
#pragma unroll
      for (int kt = 0; kt < NH; ++kt) mfma4v(accw, aw[I & 1][kt], S[kt]);
      Dl[I] = acc - accw;
      sX[(wave * 4 + I) * 64 + lane] = Dl[I];
      sched_fence();
    }
    __syncthreads();  // both halves' parts of Delta are in LDS
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      const f32x4_t o = sX[((wave ^ 4) * 4 + I) * 64 + lane];
      Dl[I] = hh == 0 ? Dl[I] + o : o + Dl[I];  // the same sum, in the same order, in both halves
    }
    if (!no_write) {
#pragma unroll
      for (int I = 0; I < 4; ++I)
        if ((I >> 1) == hh) {
#pragma unroll
          for (int r = 0; r < 4; ++r) ch[L.DL + (16 * I + 4 * g + r) * dv + col] = Dl[I][r];
        }
    }
    if (nc + 1 < nch || sp.end) {
#pragma unroll
      for (int I = 0; I < NH; ++I) {
        if (I + 1 < NH) load_s((I + 1) & 1, I + 1);
        sched_fence();
        f32x4_t acc = zero4f();
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) mfma4v(acc, ak[I & 1][kt], Dl[kt]);
        const f32x4_t gl = agl[I & 1];
        if constexpr (CPX) {
#pragma unroll
          for (int r = 0; r < 4; r += 2) {
            const cf z = cmul(cf{gl[r], gl[r + 1]}, cf{S[I][r], S[I][r + 1]});
            S[I][r] = z.x + acc[r];
            S[I][r + 1] = z.y + acc[r + 1];
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) S[I][r] = gl[r] * S[I][r] + acc[r];
        }
        sched_fence();
      }
    }
  }
  if (sp.end) {
    const int ce = cs + ((sp.flags & kWEndNext) ? 1 : (sp.flags & kWEndPrev) ? -1 : 0);
#pragma unroll
    for (int I = 0; I < NH; ++I)
#pragma unroll
      for (int r = 0; r < 4; ++r) sp.end[((size_t)ce * DK + 16 * (hh * NH + I) + 4 * g + r) * cols + col] = S[I][r];
  }
}

// bwd_adjoint_kernel: chunks in reverse; writes the end-state adjoint dS'_n and dDelta_n
// of every chunk, and dS_0.  The next chunk's operands are loaded into registers while
// the current one computes.
// CPX: SFDA complex gates -- the transpose of the chunk-end rotation-decay is conj(gamma_L)
// on the row pairs.
template <typename T, int DK, bool CPX, int WMODE = 0>
__global__ __launch_bounds__(NT) void bwd_adjoint_kernel(BwdArgs a, int NC, WalkSplit sp0, WalkSplit sp1,
                                                         int nfirst) {
  // WMODE as in bwd_state_kernel: 0 one walk per chain, 1 one segment walk per workgroup,
  // 2 a paired launch (workgroups from nfirst on run the second walk)
  const bool second = WMODE == 2 && (int)blockIdx.x >= nfirst;
  const WalkSplit sp = WMODE == 2 ? pick_split(sp0, sp1, second) : WMODE == 1 ? sp0 : WalkSplit{};
  const int bid = second ? (int)blockIdx.x - nfirst : (int)blockIdx.x;
  constexpr int LK = DK + 4, LM = C + 4, LV = VTW + 4;
  constexpr int NM = C * C / 4 / NT, NW = C * DK / 4 / NT, NV = C * VTW / 4 / NT;
  __shared__ __attribute__((aligned(16))) float sKr[C * LK], sAT[C * LM], sQgT[DK * LM], sWT[DK * LM], sO[C * LV], sGl[DK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, g = lane >> 4;
  const bool split = sp.nseg > 1;
  const int dv = a.Dv, cols = split ? sp.cols : dv, ntile = cols / VTW;
  const int cl = bid / ntile, v0 = (bid % ntile) * VTW;  // cl: chain (and segment) of this launch
  const int bh = cl / sp.nsub, seg = sp.seg_lo + cl % sp.nsub;  // bh: the chain (b H + h, or sequence H + h)
  const int cs = bh * sp.nseg + seg;  // index of the segment's start and end adjoints
  const int nall = chain_chunks(a, NC, bh);
  int c0 = 0, nch = nall;  // chunks c0 .. c0 + nch - 1, in reverse
  if (split) walk_seg_range(sp, seg, nall, c0, nch);
  const bool zero_in = sp.flags & kWZeroIn, no_write = sp.flags & kWNoWrite;
  const int col = v0 + 16 * wave + n;
  const BwdLayout L(DK, dv);
  f32x4_t dS[DK / 16];
#pragma unroll
  for (int I = 0; I < DK / 16; ++I)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * I + 4 * g + r;
      if (sp.flags & kWIdentity)
        dS[I][r] = row == col ? 1.f : 0.f;
      else if (split && !(sp.flags & kWHead))
        dS[I][r] = sp.start ? sp.start[((size_t)cs * DK + row) * cols + col] : 0.f;
      else
        dS[I][r] = a.dsT ? a.dsT[((size_t)bh * DK + row) * dv + col] : 0.f;
    }
#ifndef KDA_HOST_PASS
  // the start values are in registers before the walk: otherwise the compiler keeps their
  // loads pending into the loop and waits on every outstanding load at the first store
  __builtin_amdgcn_s_waitcnt(0);
#endif
  // one chunk's operands in registers: K o rho; Q o gamma; W; A; dO; gamma_last.  Step st
  // moves chunk nch - st from registers to LDS, issues the loads of chunk nch - 1 - st,
  // then computes chunk nch - st while they are in flight.
  using RI = RawIn<T>;
  f32x4_t pk[NW], pq[NW], pw[NW], pa[NM];
  typename RI::v4 po[NV];
  float pg = 0.f;
  int plen = 0;  // rows of the loaded dO tile that are inside the chunk (0: dO read as zero)
  size_t wnext = 0;  // workspace slot of the chunk loaded last (chunk tables are read once)
  for (int st = 0; st <= nch; ++st) {
    const size_t wcur = wnext;
    if (st > 0) {
      __syncthreads();
#pragma unroll
      for (int it = 0; it < NW; ++it) {
        const int x = tid + it * NT, i = x / (DK / 4), c = 4 * (x % (DK / 4));
        const int ti = x % C, tc = 4 * (x / C);  // transposed tiles: a wave's lanes take consecutive rows
        *(f32x4_t*)(sKr + i * LK + c) = pk[it];
        sQgT[(tc + 0) * LM + ti] = pq[it].x;
        sQgT[(tc + 1) * LM + ti] = pq[it].y;
        sQgT[(tc + 2) * LM + ti] = pq[it].z;
        sQgT[(tc + 3) * LM + ti] = pq[it].w;
        sWT[(tc + 0) * LM + ti] = pw[it].x;
        sWT[(tc + 1) * LM + ti] = pw[it].y;
        sWT[(tc + 2) * LM + ti] = pw[it].z;
        sWT[(tc + 3) * LM + ti] = pw[it].w;
      }
#pragma unroll
      for (int it = 0; it < NM; ++it) {
        const int x = tid + it * NT, j = x % C, i = 4 * (x / C);  // consecutive rows j per wave
        sAT[(i + 0) * LM + j] = pa[it].x;
        sAT[(i + 1) * LM + j] = pa[it].y;
        sAT[(i + 2) * LM + j] = pa[it].z;
        sAT[(i + 3) * LM + j] = pa[it].w;
      }
#pragma unroll
      for (int it = 0; it < NV; ++it) {
        const int x = tid + it * NT, i = x / (VTW / 4), c = 4 * (x % (VTW / 4));
        *(f32x4_t*)(sO + i * LV + c) = i < plen ? RI::widen(po[it]) : zero4f();
      }
      if (tid < DK) sGl[tid] = pg;
      __syncthreads();
    }
    if (st < nch) {
      const int ld = c0 + nch - 1 - st;
      size_t wsl;
      const ChunkGeom cg = chain_chunk(a, NC, bh, ld, &wsl);
      wnext = wsl;
      const float* cl = a.ws + wsl * L.total;
      const size_t vb = row0(cg, a.T, a.H, dv), vs = (size_t)a.H * dv;
      plen = zero_in ? 0 : cg.len;  // unconditional loads, rows past the chunk clamped and masked when staged
      const int lastr = max(cg.len - 1, 0);
#pragma unroll
      for (int it = 0; it < NW; ++it) {
        const int x = tid + it * NT, i = x / (DK / 4), c = 4 * (x % (DK / 4));
        const int ti = x % C, tc = 4 * (x / C);
        pk[it] = *(const f32x4_t*)(cl + L.KR + i * DK + c);
        pq[it] = *(const f32x4_t*)(cl + L.QG + ti * DK + tc);
        pw[it] = *(const f32x4_t*)(cl + L.W + ti * DK + tc);
      }
#pragma unroll
      for (int it = 0; it < NM; ++it) {
        const int x = tid + it * NT, j = x % C, i = 4 * (x / C);
        pa[it] = *(const f32x4_t*)(cl + L.A + j * C + i);
      }
#pragma unroll
      for (int it = 0; it < NV; ++it) {
        const int x = tid + it * NT, i = x / (VTW / 4), c = 4 * (x % (VTW / 4));
        po[it] = RI::load4(a.dO, vb + min(i, lastr) * vs + v0 + c);
      }
      pg = cl[L.gam + (C - 1) * DK + min(tid, DK - 1)];  // unconditional: no branch around the load
    }
    if (st == 0) continue;
    float* ch = a.ws + wcur * L.total;  // chunk c0 + nch - st
    if (!no_write) {
#pragma unroll
      for (int I = 0; I < DK / 16; ++I)
#pragma unroll
        for (int r = 0; r < 4; ++r) ch[L.DS + (16 * I + 4 * g + r) * dv + col] = dS[I][r];
    }
    // dDelta = (K o rho) dS' + A^T dO, then dS = gamma_L o dS' + (Q o gamma)^T dO - W^T dDelta,
    // one row block at a time, the A operands of the next block read while the current
    // one multiplies (one wave per SIMD: nothing else hides the LDS latency).
    float bo[4][4];  // B operands shared by every row block: this wave's columns of dO
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int t = 0; t < 4; ++t) bo[q][t] = sO[(16 * q + 4 * g + t) * LV + 16 * wave + n];
    f32x4_t akr[2][DK / 16], aat[2][4], aq[2][4], awt[2][4], agl[2];
    auto load_a = [&](int b, int I) {
      const float* krow = sKr + (16 * I + n) * LK + 4 * g;
      const float* arow = sAT + (16 * I + n) * LM + 4 * g;
#pragma unroll
      for (int kt = 0; kt < DK / 16; ++kt) akr[b][kt] = *(const f32x4_t*)(krow + 16 * kt);
#pragma unroll
      for (int q = 0; q < 4; ++q) aat[b][q] = *(const f32x4_t*)(arow + 16 * q);
    };
    auto load_b = [&](int b, int I) {
      const float* qrow = sQgT + (16 * I + n) * LM + 4 * g;
      const float* wrow = sWT + (16 * I + n) * LM + 4 * g;
#pragma unroll
      for (int q = 0; q < 4; ++q) aq[b][q] = *(const f32x4_t*)(qrow + 16 * q);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) awt[b][kt] = *(const f32x4_t*)(wrow + 16 * kt);
      agl[b] = *(const f32x4_t*)(sGl + 16 * I + 4 * g);
    };
    load_a(0, 0);
    sched_fence();
    f32x4_t dD[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      if (I + 1 < 4)
        load_a((I + 1) & 1, I + 1);
      else
        load_b(0, 0);
      sched_fence();
      f32x4_t acc = zero4f();
#pragma unroll
      for (int kt = 0; kt < DK / 16; ++kt) mfma4v(acc, akr[I & 1][kt], dS[kt]);
#pragma unroll
      for (int q = 0; q < 4; ++q) mfma4v(acc, aat[I & 1][q], bo[q]);
      dD[I] = acc;
      sched_fence();
      if (!no_write) {
#pragma unroll
        for (int r = 0; r < 4; ++r) ch[L.DDL + (16 * I + 4 * g + r) * dv + col] = acc[r];
      }
    }
#pragma unroll
    for (int I = 0; I < DK / 16; ++I) {
      if (I + 1 < DK / 16) load_b((I + 1) & 1, I + 1);
      sched_fence();
      f32x4_t acc = zero4f(), accw = zero4f();
#pragma unroll
      for (int q = 0; q < 4; ++q) mfma4v(acc, aq[I & 1][q], bo[q]);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) mfma4v(accw, awt[I & 1][kt], dD[kt]);
      acc -= accw;
      const f32x4_t gl = agl[I & 1];
      if constexpr (CPX) {
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const cf z = cmulc(cf{dS[I][r], dS[I][r + 1]}, cf{gl[r], gl[r + 1]});
          dS[I][r] = z.x + acc[r];
          dS[I][r + 1] = z.y + acc[r + 1];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) dS[I][r] = gl[r] * dS[I][r] + acc[r];
      }
      sched_fence();
    }
  }
  if (sp.end) {
    const int ce = cs + ((sp.flags & kWEndNext) ? 1 : (sp.flags & kWEndPrev) ? -1 : 0);
#pragma unroll
    for (int I = 0; I < DK / 16; ++I)
#pragma unroll
      for (int r = 0; r < 4; ++r) sp.end[((size_t)ce * DK + 16 * I + 4 * g + r) * cols + col] = dS[I][r];
  } else if (a.ds0 && seg == 0) {  // the chain's first segment ends at S_0
#pragma unroll
    for (int I = 0; I < DK / 16; ++I)
#pragma unroll
      for (int r = 0; r < 4; ++r) a.ds0[((size_t)bh * DK + 16 * I + 4 * g + r) * dv + col] = dS[I][r];
  }
}

// Segment start states of a split walk, fp32, one workgroup per (chain, 16 columns):
// forward (the state walk) X_0 = init, X_(g+1) = P_g X_g + B_g; reverse (the adjoint walk,
// whose segments run backwards) X_(G-1) = init, X_(g-1) = P_g X_g + B_g.  init may be NULL.
// g_first >= 0: the scan starts from X_(g_first), already written (by the full walk of the
// segment before it).
template <int DK>
__global__ __launch_bounds__(256) void walk_scan_kernel(const float* __restrict__ init, const float* __restrict__ P,
                                                      const float* __restrict__ Bst, float* __restrict__ X, int G,
                                                      int dv, int reverse, int g_first) {
  __shared__ float sX[DK][17];
  const int nsl = dv / 16, ch = blockIdx.x / nsl, c0 = (blockIdx.x % nsl) * 16;
  const int tid = threadIdx.x, c = tid & 15, r0 = tid >> 4;
  constexpr int RJ = DK / 16;
  const size_t SS = (size_t)DK * dv;
  const int g0 = g_first >= 0 ? g_first : reverse ? G - 1 : 0;
#pragma unroll
  for (int j = 0; j < RJ; ++j) {
    const int r = r0 + 16 * j;
    float* xg = X + ((size_t)ch * G + g0) * SS + (size_t)r * dv + c0 + c;
    if (g_first >= 0) {
      sX[r][c] = *xg;
    } else {
      const float x = init ? init[((size_t)ch * DK + r) * dv + c0 + c] : 0.f;
      sX[r][c] = x;
      *xg = x;
    }
  }
  const int nsteps = reverse ? g0 : G - 1 - g0;
  for (int step = 0; step < nsteps; ++step) {
    const int gi = reverse ? g0 - step : g0 + step, gn = reverse ? gi - 1 : gi + 1;
    __syncthreads();
    const float* Pg = P + ((size_t)ch * G + gi) * DK * DK;
    const float* Bg = Bst + ((size_t)ch * G + gi) * SS;
    float acc[RJ];
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
      const int r = r0 + 16 * j;
      float s = Bg[(size_t)r * dv + c0 + c];
      const float4* prow = (const float4*)(Pg + (size_t)r * DK);
#pragma unroll 4
      for (int k4 = 0; k4 < DK / 4; ++k4) {
        const float4 p = prow[k4];
        s += p.x * sX[4 * k4][c] + p.y * sX[4 * k4 + 1][c] + p.z * sX[4 * k4 + 2][c] + p.w * sX[4 * k4 + 3][c];
      }
      acc[j] = s;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
      const int r = r0 + 16 * j;
      sX[r][c] = acc[j];
      X[((size_t)ch * G + gn) * SS + (size_t)r * dv + c0 + c] = acc[j];
    }
  }
}

// ---------------------------------------------------------------------------------------
// Scratch slots of the gradient kernel: n slots of GradScratch (n a multiple of 8), then
// the lock words (zero: free; cleared before every launch), [8][GradScratch::lock_row(n)]
// so that each XCD's words fill cache lines of their own.  Slot s belongs to XCD s % 8: a
// workgroup takes a free slot of the XCD it runs on and frees it at its end, so a slot's
// lines only ever sit in that XCD's L2 and the lock needs no cache maintenance (the
// workgroup's own accesses to the slot have completed when it frees it).  An XCD holds
// fewer resident workgroups than its n / 8 slots, or waits for one of its own workgroups
// to free one; a holder never waits for anything before it frees its slot.
__device__ inline int* grad_slot_lock(float* base, int n, int slot_floats, int s) {
  return (int*)(base + (size_t)n * slot_floats) + (s & 7) * GradScratch::lock_row(n) + (s >> 3);
}
__device__ inline int xcc_id() {
  int x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  return x & 7;
}
__device__ inline int grad_slot_acquire(float* base, int n, int slot_floats) {
  const int per = n / 8, x = xcc_id();
  int j = (int)(blockIdx.x / 8) % per;
  while (atomicCAS(grad_slot_lock(base, n, slot_floats, x + 8 * j), 0, 1) != 0) j = j + 1 == per ? 0 : j + 1;
  return x + 8 * j;
}
__device__ inline void grad_slot_release(float* base, int n, int slot_floats, int s) {
  atomicExch(grad_slot_lock(base, n, slot_floats, s), 0);
}
__global__ void clear_words_kernel(int* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

// ---------------------------------------------------------------------------------------
// bwd_grads_kernel: per (b, h, chunk), in five phases:
//   A  products over the value dimension, by key-channel tile: a wave holds its 16
//      channels' rows of S and dS' as B fragments in registers and runs d(Q o gamma),
//      dW and d(K o rho) against dO, dDelta and Delta staged in LDS, then
//      d(K o gamma) = Mt^T dW with its dW tiles as B operands; dgamma_L comes from the
//      same registers;
//   B  dA, dV, dMt from LDS (dW staged where dO and Delta were);
//   C  dbeta, X = dMt Mt^T, dT and dD in LDS;
//   D  the block-anchored products PA, PD, F with their B operands staged in LDS;
//   E  per (channel, block): the in-block decayed sums, dq and dk, the gate gradient.

//   CPX (SFDA complex gates): the per-channel products of A become complex products of a
//   lane's pair with its neighbour lane's (the pair's other channel, lane ^ 1); D forms
//   the anchored operands with complex factors; E takes one (pair, block) item per
//   thread, in complex arithmetic.
template <typename T, int DK, int DV, bool G2, bool CPX>
__global__ __launch_bounds__(NTG) void bwd_grads_kernel(BwdArgs a, int NC) {
  constexpr int LV = DV + 4, LK = DK + 4, LC = C + 1;
  constexpr int RSZ = (3 * C * LV > 3 * C * LK) ? 3 * C * LV : 3 * C * LK;
  static_assert(LK <= 2 * LV, "dW must fit where dO and Delta were");
  __shared__ float sR[RSZ];  // staging region, reused by every phase
  __shared__ float sM[C * LC], sdA[C * LC], sdT[C * LC];  // sdT: dMt, then dT, then dD
  __shared__ float sB[C], sdB[C], sGl[DK], sPib[NB * DK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, g = lane >> 4;
  const BwdLayout L(DK, DV);
  ChunkGeom cg;
  size_t wsi;
  if (!block_chunk(a, NC, &cg, &wsi)) return;
  const int len = cg.len;
  float* ch = a.ws + wsi * L.total;
  const size_t kb = row0(cg, a.T, a.H, DK), ks = (size_t)a.H * DK;
  const size_t vb = row0(cg, a.T, a.H, DV), vs = (size_t)a.H * DV;
  const size_t bb = ((size_t)cg.b * a.T + cg.t0) * a.H + cg.h;
  const float *GAM = ch + L.gam, *RHO = ch + L.rho, *PIN = ch + L.pin, *SIG = ch + L.sig;
  const float *S = ch + L.S, *DS = ch + L.DS;
  // this workgroup's scratch slot, held until the kernel's last use of it
  __shared__ int sSlot;
  const GradScratch GS(DK);
  if (tid == 0) sSlot = grad_slot_acquire(a.gscr, a.gslots, GS.total);
  __syncthreads();
  float* gs = a.gscr + (size_t)sSlot * GS.total;
  float *AV = gs + GS.AV, *BV = gs + GS.BV, *DWg = gs + GS.DW, *F = gs + GS.F, *PA = gs + GS.PA, *PD = gs + GS.PD;
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  auto in4 = [&](const void* p, int i, int c) { return i < len ? ld4<T>(p, kb + i * ks + c) : z4; };
  auto in1 = [&](const void* p, int i, int c) { return i < len ? Elem<T>::load(p, kb + i * ks + c) : 0.f; };
  auto between = [&](int J, int I, int c) {
    float w = 1.f;
    for (int x = J + 1; x < I; ++x) w *= sPib[x * DK + c];
    return w;
  };

  // ---- stage dO, Delta, dDelta; M, beta, the block totals
  float *RO = sR, *RL = sR + C * LV, *RD = sR + 2 * C * LV;
#pragma unroll
  for (int it = 0; it < C * DV / 4 / NTG; ++it) {
    const int x = tid + it * NTG, i = x / (DV / 4), v = 4 * (x % (DV / 4));
    *(float4*)(RO + i * LV + v) = i < len ? ld4<T>(a.dO, vb + i * vs + v) : z4;
    *(float4*)(RL + i * LV + v) = *(const float4*)(ch + L.DL + i * DV + v);
    *(float4*)(RD + i * LV + v) = *(const float4*)(ch + L.DDL + i * DV + v);
  }
#pragma unroll
  for (int it = 0; it < C * C / 4 / NTG; ++it) {
    const int x = tid + it * NTG, i = x / (C / 4), j = 4 * (x % (C / 4));
    const float4 m = *(const float4*)(ch + L.M + i * C + j);
    sM[i * LC + j] = m.x;
    sM[i * LC + j + 1] = m.y;
    sM[i * LC + j + 2] = m.z;
    sM[i * LC + j + 3] = m.w;
  }
  for (int i = tid; i < C; i += NTG) sB[i] = G2 ? 1.f : (i < len ? Elem<T>::load(a.beta, bb + (size_t)i * a.H) : 0.f);
  for (int x = tid; x < NB * DK; x += NTG) sPib[x] = ch[L.pib + x];
  __syncthreads();

  // ---- A: d(Q o gamma) = dO S^T, dW = -dDelta S^T, d(K o rho) = Delta dS'^T, dgamma_L
  for (int ct = wave; ct < DK / 16; ct += NTG / 64) {
    const int c = 16 * ct + n;
    float4 sf[DV / 16], df[DV / 16];
#pragma unroll
    for (int u = 0; u < DV / 16; ++u) {
      sf[u] = *(const float4*)(S + c * DV + 16 * u + 4 * g);
      df[u] = *(const float4*)(DS + c * DV + 16 * u + 4 * g);
    }
    float gm[4][4], rh[4][4], qq[4][4], kk[4][4], eb[4][4];  // eb: erase gate (GDN-2)
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * g + r;
        gm[I][r] = GAM[i * DK + c];
        rh[I][r] = RHO[i * DK + c];
        qq[I][r] = in1(a.q, i, c);
        kk[I][r] = in1(a.k, i, c);
        eb[I][r] = G2 ? in1(a.erase, i, c) : 0.f;
      }
    float part = 0.f;
#pragma unroll
    for (int u = 0; u < DV / 16; ++u)
      part += sf[u].x * df[u].x + sf[u].y * df[u].y + sf[u].z * df[u].z + sf[u].w * df[u].w;
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    if constexpr (CPX) {
      // dgl_p = sum_j conj(dS'_pj) S_pj: Re = sum (d0 s0 + d1 s1), Im = sum (d0 s1 - d1 s0);
      // cross = sum_j s_c d_(c^1), from the neighbour lane's dS' row
      float cross = 0.f;
#pragma unroll
      for (int u = 0; u < DV / 16; ++u)
        cross += sf[u].x * __shfl_xor(df[u].x, 1) + sf[u].y * __shfl_xor(df[u].y, 1) +
                 sf[u].z * __shfl_xor(df[u].z, 1) + sf[u].w * __shfl_xor(df[u].w, 1);
      cross += __shfl_xor(cross, 16);
      cross += __shfl_xor(cross, 32);
      const float part_o = __shfl_xor(part, 1), cross_o = __shfl_xor(cross, 1);
      if (g == 0) sGl[c] = (c & 1) ? cross - cross_o : part + part_o;
    } else {
      if (g == 0) sGl[c] = part;
    }
    f32x4_t aq[4], aw[4], ar[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      aq[I] = aw[I] = ar[I] = zero4f();
      const float *ro = RO + (16 * I + n) * LV, *rd = RD + (16 * I + n) * LV, *rl = RL + (16 * I + n) * LV;
#pragma unroll
      for (int u = 0; u < DV / 16; ++u) {
        mm16(aq[I], ro, 16 * u, [&](int t) { return f4c(sf[u], t); });
        mm16(aw[I], rd, 16 * u, [&](int t) { return f4c(sf[u], t); }, -1.f);
        mm16(ar[I], rl, 16 * u, [&](int t) { return f4c(df[u], t); });
      }
    }
    // d(K o gamma) = Mt^T dW for this channel tile: the dW tiles are the B operands
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      f32x4_t kg = zero4f();
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        float av[4], bv[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          av[t] = sM[(16 * kt + 4 * g + t) * LC + 16 * J + n] * sB[16 * J + n];
          bv[t] = aw[kt][t];
        }
        mfma4(kg, av, bv);
      }
      if constexpr (CPX) {
        // complex pairs in channel order (this lane's channel and its neighbour's):
        // av = d(Q~) conj(q) + d(K~g) conj(k), bv = conj(d(K~r)) k, dq = d(Q~) gamma,
        // dk = d(K~g) gamma + d(K~r) conj(rho)
        const int e = c & 1;
        auto pr = [&](float own) {
          const float oth = __shfl_xor(own, 1);
          return e ? cf{oth, own} : cf{own, oth};
        };
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * J + 4 * g + r;
          const cf dq_ = pr(aq[J][r]), dkg = pr(kg[r]), dkr = pr(ar[J][r]);
          const cf qc = pr(qq[J][r]), kc = pr(kk[J][r]), gc = pr(gm[J][r]), rc = pr(rh[J][r]);
          AV[i * DK + c] = comp(cadd(cmulc(dq_, qc), cmulc(dkg, kc)), e);
          BV[i * DK + c] = comp(cmulc(kc, dkr), e);
          DWg[i * DK + c] = aw[J][r];
          if (i < len) {
            a.dq[kb + i * ks + c] = comp(cmul(dq_, gc), e);
            a.dk[kb + i * ks + c] = comp(cadd(cmul(dkg, gc), cmulc(dkr, rc)), e);
          }
        }
        continue;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * J + 4 * g + r;
        // KDA: kg = d(K o gamma) (beta inside Mt); GDN-2: kg = d(E o gamma), e = b o k
        const float xk = G2 ? eb[J][r] * kk[J][r] : kk[J][r];
        AV[i * DK + c] = aq[J][r] * qq[J][r] + kg[r] * xk;
        BV[i * DK + c] = ar[J][r] * kk[J][r];
        DWg[i * DK + c] = aw[J][r];
        if (i < len) {
          a.dq[kb + i * ks + c] = aq[J][r] * gm[J][r];
          if (G2) {
            const float de = kg[r] * gm[J][r];
            a.dk[kb + i * ks + c] = ar[J][r] * rh[J][r] + eb[J][r] * de;
            a.derase[kb + i * ks + c] = kk[J][r] * de;
          } else {
            a.dk[kb + i * ks + c] = ar[J][r] * rh[J][r] + kg[r] * gm[J][r];
          }
        }
      }
    }
  }

  // ---- B: dA = (dO Delta^T) o low;  dV = Mt^T dDelta
  for (int job = wave; job < 16 + 4 * (DV / 16); job += NTG / 64) {
    if (job < 16) {
      const int I = job / 4, J = job % 4;
      f32x4_t acc = zero4f();
      if (J <= I) {
        const float *ro = RO + (16 * I + n) * LV, *rl = RL + (16 * J + n) * LV;
#pragma unroll
        for (int u = 0; u < DV / 16; ++u) mm16(acc, ro, 16 * u, [&](int t) { return rl[16 * u + 4 * g + t]; });
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * g + r, j = 16 * J + n;
        sdA[i * LC + j] = j <= i ? acc[r] : 0.f;
      }
    } else {
      const int jj = job - 16, J = jj / (DV / 16), vt = jj % (DV / 16);
      f32x4_t acc = zero4f();
#pragma unroll
      for (int k0 = 0; k0 < C; k0 += 16) {
        float av[4], bv[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int i = k0 + 4 * g + t;
          av[t] = sM[i * LC + 16 * J + n] * sB[16 * J + n];
          bv[t] = RD[i * LV + 16 * vt + n];
        }
        mfma4(acc, av, bv);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * J + 4 * g + r;
        if (j < len) {
          const size_t o = vb + j * vs + 16 * vt + n;
          if (G2) {  // acc = d(w o V)
            a.dv[o] = acc[r] * Elem<T>::load(a.write, o);
            a.dwrite[o] = acc[r] * Elem<T>::load(a.v, o);
          } else {
            a.dv[o] = acc[r];
          }
        }
      }
    }
  }
  __syncthreads();
  float* RW = sR;  // dW [C][LK], where dO and Delta were
#pragma unroll
  for (int it = 0; it < C * DK / 4 / NTG; ++it) {
    const int x = tid + it * NTG, i = x / (DK / 4), c = 4 * (x % (DK / 4));
    *(float4*)(RW + i * LK + c) = *(const float4*)(DWg + i * DK + c);
  }
  __syncthreads();
  // dMt = (dDelta V^T + dW (K o gamma)^T) o low
  for (int job = wave; job < 16; job += NTG / 64) {
    {
      const int I = job / 4, J = job % 4, j = 16 * J + n;
      f32x4_t acc = zero4f();
      if (J <= I) {
        float4 vv[DV / 16], kg[DK / 16];
#pragma unroll
        for (int u = 0; u < DV / 16; ++u) {
          vv[u] = j < len ? ld4<T>(a.v, vb + j * vs + 16 * u + 4 * g) : z4;
          if (G2) vv[u] = mul4(vv[u], j < len ? ld4<T>(a.write, vb + j * vs + 16 * u + 4 * g) : z4);
        }
#pragma unroll
        for (int u = 0; u < DK / 16; ++u) {
          const float4 k4 = in4(a.k, j, 16 * u + 4 * g), g4 = *(const float4*)(GAM + j * DK + 16 * u + 4 * g);
          if constexpr (CPX) {  // k conj(gamma) on the two pairs of the four channels
            const cf z0 = cmulc(cf{k4.x, k4.y}, cf{g4.x, g4.y}), z1 = cmulc(cf{k4.z, k4.w}, cf{g4.z, g4.w});
            kg[u] = make_float4(z0.x, z0.y, z1.x, z1.y);
          } else {
            kg[u] = mul4(k4, g4);
          }
          if (G2) kg[u] = mul4(kg[u], in4(a.erase, j, 16 * u + 4 * g));
        }
        const float *rd = RD + (16 * I + n) * LV, *rw = RW + (16 * I + n) * LK;
#pragma unroll
        for (int u = 0; u < DV / 16; ++u) mm16(acc, rd, 16 * u, [&](int t) { return f4c(vv[u], t); });
#pragma unroll
        for (int u = 0; u < DK / 16; ++u) mm16(acc, rw, 16 * u, [&](int t) { return f4c(kg[u], t); });
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * g + r;
        sdT[i * LC + j] = j <= i ? acc[r] : 0.f;
      }
    }
  }
  __syncthreads();

  // ---- C: dbeta = colsum(dMt o M) + rowsum(dT o D);  X = dMt Mt^T;  dT = -(M^T X) o strict-low
  if (!G2) {  // (eight threads per column, rows interleaved, the sum by lane exchanges)
    static_assert(NTG == 8 * C, "eight threads per column");
    const int j = tid >> 3;
    float s = 0.f;
    for (int i = j + (tid & 7); i < C; i += 8) s += sdT[i * LC + j] * sM[i * LC + j];
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    if ((tid & 7) == 0) sdB[j] = s;
  }
  float* RX = sR;  // X [C][LC]
  for (int job = wave; job < 16; job += NTG / 64) {
    const int I = job / 4, J = job % 4;
    f32x4_t acc = zero4f();
#pragma unroll
    for (int k0 = 0; k0 < C; k0 += 16) {
      float av[4], bv[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int kx = k0 + 4 * g + t;
        av[t] = sdT[(16 * I + n) * LC + kx];
        bv[t] = sM[(16 * J + n) * LC + kx] * sB[kx];
      }
      mfma4(acc, av, bv);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) RX[(16 * I + 4 * g + r) * LC + 16 * J + n] = acc[r];
  }
  __syncthreads();
  for (int job = wave; job < 16; job += NTG / 64) {
    const int I = job / 4, J = job % 4;
    f32x4_t acc = zero4f();
    if (J <= I) {
#pragma unroll
      for (int k0 = 0; k0 < C; k0 += 16) {
        float av[4], bv[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int kx = k0 + 4 * g + t;
          av[t] = sM[kx * LC + 16 * I + n];
          bv[t] = RX[kx * LC + 16 * J + n];
        }
        mfma4(acc, av, bv);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * I + 4 * g + r, j = 16 * J + n;
      sdT[i * LC + j] = j < i ? -acc[r] : 0.f;
    }
  }
  __syncthreads();
  if (!G2) {
    // dbeta_i = sdB_i + sum_{j < i} dT_ij D_ij, then dT <- diag(beta) dT: eight threads per
    // row, eight columns each (D's row read as two 16-byte vectors, all rows at once), the
    // row sum by lane exchanges
    static_assert(NTG == 8 * C, "eight threads per row");
    const int i = tid >> 3, j0 = 8 * (tid & 7);
    const float4 d0 = *(const float4*)(ch + L.D + i * C + j0), d1 = *(const float4*)(ch + L.D + i * C + j0 + 4);
    const float dv8[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (j0 + e < i) s += sdT[i * LC + j0 + e] * dv8[e];
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    if ((tid & 7) == 0 && i < len) a.dbeta[bb + (size_t)i * a.H] = sdB[i] + s;
    const float bi = sB[i];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (j0 + e < i) sdT[i * LC + j0 + e] *= bi;
  }
  __syncthreads();
  const float* sdD = sdT;

  // ---- D: PA^M = dA[>= s_M, < s_M] Khat^M, PD^M likewise with dD (M = 1..3), with
  // Khat^M_j = k_j sigma_j (blocks between); F^M_j = sum_{i > e_M} (dA_ij q_i + dD_ij k_i)
  // r(i, e_M), r(i, e_M) = pi_i (blocks between) (M = 0..2)
  float *RKS = sR, *RQP = sR + C * LK, *RKP = sR + 2 * C * LK;
#pragma unroll
  for (int it = 0; it < C * DK / 4 / NTG; ++it) {
    const int x = tid + it * NTG, i = x / (DK / 4), c = 4 * (x % (DK / 4));
    const float4 kv = in4(a.k, i, c), qv = in4(a.q, i, c);
    const float4 sg = *(const float4*)(SIG + i * DK + c), pn = *(const float4*)(PIN + i * DK + c);
    const float4 xv = G2 ? mul4(kv, in4(a.erase, i, c)) : kv;  // row operand of the second product
    if constexpr (CPX) {  // k sigma; q conj(pi), k conj(pi) (the key side of F takes conj(r))
      const cf k0 = {kv.x, kv.y}, k1 = {kv.z, kv.w}, q0 = {qv.x, qv.y}, q1 = {qv.z, qv.w};
      const cf s0 = {sg.x, sg.y}, s1 = {sg.z, sg.w}, p0 = {pn.x, pn.y}, p1 = {pn.z, pn.w};
      cf a0 = cmul(k0, s0), a1 = cmul(k1, s1);
      *(float4*)(RKS + i * LK + c) = make_float4(a0.x, a0.y, a1.x, a1.y);
      a0 = cmulc(q0, p0), a1 = cmulc(q1, p1);
      *(float4*)(RQP + i * LK + c) = make_float4(a0.x, a0.y, a1.x, a1.y);
      a0 = cmulc(k0, p0), a1 = cmulc(k1, p1);
      *(float4*)(RKP + i * LK + c) = make_float4(a0.x, a0.y, a1.x, a1.y);
    } else {
      *(float4*)(RKS + i * LK + c) = mul4(kv, sg);
      *(float4*)(RQP + i * LK + c) = mul4(qv, pn);
      *(float4*)(RKP + i * LK + c) = mul4(xv, pn);
    }
  }
  // complex product of the whole blocks between J and I for the pair of channel c
  auto between_c = [&](int J, int I, int c) {
    cf w = {1.f, 0.f};
    for (int x = J + 1; x < I; ++x) w = cmul(w, cpair(sPib + x * DK, c));
    return w;
  };
  __syncthreads();
  for (int job = wave; job < 12 * (DK / 16); job += NTG / 64) {
    const int ct = job % (DK / 16), p6 = (job / (DK / 16)) % 6, mat = job / (DK / 16) / 6;
    // (M, I): (1,1) (1,2) (1,3) (2,2) (2,3) (3,3)
    const int Mb = p6 < 3 ? 1 : (p6 < 5 ? 2 : 3), I = Mb + (p6 < 3 ? p6 : (p6 < 5 ? p6 - 3 : 0));
    const int c = 16 * ct + n;
    const float* src = mat ? sdD : sdA;
    f32x4_t acc = zero4f();
    for (int J = 0; J < Mb; ++J) {
      float av[4], bv[4];
      if constexpr (CPX) {
        const cf w = between_c(J, Mb, c);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int jx = 16 * J + 4 * g + t;
          av[t] = src[(16 * I + n) * LC + jx];
          bv[t] = comp(cmul(cpair(RKS + jx * LK, c), w), c & 1);
        }
      } else {
        const float w = between(J, Mb, c);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int jx = 16 * J + 4 * g + t;
          av[t] = src[(16 * I + n) * LC + jx];
          bv[t] = RKS[jx * LK + c] * w;
        }
      }
      mfma4(acc, av, bv);
    }
    float* out = (mat ? PD : PA) + (size_t)(Mb - 1) * C * DK;
#pragma unroll
    for (int r = 0; r < 4; ++r) out[(16 * I + 4 * g + r) * DK + c] = acc[r];
  }
  for (int job = wave; job < 3 * (DK / 16); job += NTG / 64) {
    const int Mb = job / (DK / 16), ct = job % (DK / 16), s = 16 * Mb, c = 16 * ct + n;
    f32x4_t acc = zero4f();
    for (int I = Mb + 1; I < NB; ++I) {
      float av[4], bv[4];
      if constexpr (CPX) {  // conj(r(i, e)) = conj(pi_i) conj(blocks between)
        const cf w = between_c(Mb, I, c);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int ix = 16 * I + 4 * g + t;
          av[t] = sdA[ix * LC + s + n];
          bv[t] = comp(cmulc(cpair(RQP + ix * LK, c), w), c & 1);
        }
        mfma4(acc, av, bv);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int ix = 16 * I + 4 * g + t;
          av[t] = sdD[ix * LC + s + n];
          bv[t] = comp(cmulc(cpair(RKP + ix * LK, c), w), c & 1);
        }
        mfma4(acc, av, bv);
      } else {
        const float w = between(Mb, I, c);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int ix = 16 * I + 4 * g + t;
          av[t] = sdA[ix * LC + s + n];
          bv[t] = RQP[ix * LK + c] * w;
        }
        mfma4(acc, av, bv);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int ix = 16 * I + 4 * g + t;
          av[t] = sdD[ix * LC + s + n];
          bv[t] = RKP[ix * LK + c] * w;
        }
        mfma4(acc, av, bv);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) F[(s + 4 * g + r) * DK + c] = acc[r];
  }
  __syncthreads();

  // ---- E: stage q, k, alpha; per (channel, block) items
  float *RQ = sR, *RK = sR + C * LK, *RA = sR + 2 * C * LK;
#pragma unroll
  for (int it = 0; it < C * DK / 4 / NTG; ++it) {
    const int x = tid + it * NTG, i = x / (DK / 4), c = 4 * (x % (DK / 4));
    *(float4*)(RQ + i * LK + c) = in4(a.q, i, c);
    *(float4*)(RK + i * LK + c) = in4(a.k, i, c);
    // rows past the end decay by the identity: 1 per channel, or 1 + 0i per complex pair
    *(float4*)(RA + i * LK + c) = i < len   ? ld4<T>(a.alpha, kb + i * ks + c)
                                  : CPX ? make_float4(1.f, 0.f, 1.f, 0.f)
                                        : make_float4(1.f, 1.f, 1.f, 1.f);
  }
  __syncthreads();
  if constexpr (CPX) {
    // SFDA: one (pair, block) item per thread, the real item's sums and recursion in complex
    // arithmetic: Zq_i = sum_j dA_ij r_ij k_j, Zc_j = sum_i (dA_ij q_i + dD_ij k_i) conj(r_ij);
    // pair weights E_ij = (dA_ij conj(q_i) + dD_ij conj(k_i)) k_j; the recursion's result
    // is the conjugate of the gate gradient (dL/dRe + i dL/dIm)
    for (int item = tid; item < (DK / 2) * NB; item += NTG) {
      const int c0 = 2 * (item % (DK / 2)), Mb = item / (DK / 2), s = Mb * SUB;
      auto lds = [&](const float* base, int i) { return cf{base[i * LK + c0], base[i * LK + c0 + 1]}; };
      auto wsc = [&](const float* base, int i) { return cf{base[i * DK + c0], base[i * DK + c0 + 1]}; };
      cf al[SUB], qv[SUB], kv[SUB];
#pragma unroll
      for (int r = 0; r < SUB; ++r) {
        al[r] = lds(RA, s + r);
        qv[r] = lds(RQ, s + r);
        kv[r] = lds(RK, s + r);
      }
      const float* PAm = PA + (size_t)(Mb > 0 ? Mb - 1 : 0) * C * DK;
      const float* PDm = PD + (size_t)(Mb > 0 ? Mb - 1 : 0) * C * DK;
      cf gs = {1.f, 0.f}, rend = {1.f, 0.f};
#pragma unroll
      for (int J = 0; J < NB; ++J) {
        if (J < Mb) gs = cmul(gs, cpair(sPib + J * DK, c0));
        if (J > Mb) rend = cmul(rend, cpair(sPib + J * DK, c0));
      }
#pragma unroll
      for (int r = 0; r < SUB; ++r) {
        const int i = s + r;
        cf zq = cscale(kv[r], sdA[i * LC + i]), zr = {0.f, 0.f}, P = {1.f, 0.f};
#pragma unroll
        for (int rj = r - 1; rj >= 0; --rj) {
          P = cmul(P, al[rj + 1]);
          const cf kp = cmul(kv[rj], P);
          zq = cadd(zq, cscale(kp, sdA[i * LC + s + rj]));
          zr = cadd(zr, cscale(kp, sdD[i * LC + s + rj]));
        }
        if (Mb > 0) {
          const cf pin = wsc(PIN, i);
          zq = cadd(zq, cmul(pin, wsc(PAm, i)));
          zr = cadd(zr, cmul(pin, wsc(PDm, i)));
        }
        cf zc = cscale(qv[r], sdA[i * LC + i]);
        P = cf{1.f, 0.f};
#pragma unroll
        for (int ri = r + 1; ri < SUB; ++ri) {
          P = cmul(P, al[ri]);
          const cf w = cadd(cscale(qv[ri], sdA[(s + ri) * LC + i]), cscale(kv[ri], sdD[(s + ri) * LC + i]));
          zc = cadd(zc, cmulc(w, P));
        }
        if (Mb < NB - 1) zc = cadd(zc, cmulc(wsc(F, i), wsc(SIG, i)));
        if (i < len) {
          const size_t o = kb + i * ks + c0;
          a.dq[o] += zq.x;
          a.dq[o + 1] += zq.y;
          a.dk[o] += zr.x + zc.x;
          a.dk[o + 1] += zr.y + zc.y;
        }
      }

      cf bvs = {0.f, 0.f};  // sum_{j < s} bv_j r(s-1, j)
      for (int J = 0; J < Mb; ++J) {
        cf part = {0.f, 0.f};
#pragma unroll
        for (int r = 0; r < SUB; ++r) part = cadd(part, cmul(wsc(BV, J * SUB + r), wsc(SIG, J * SUB + r)));
        bvs = cadd(bvs, cmul(part, between_c(J, Mb, c0)));
      }
      const cf dgl = cpair(sGl, c0);
      const cf tail = cadd(bvs, cmul(dgl, gs));  // the final-state terms of row C - 1
      cf u[SUB];
#pragma unroll
      for (int r = 0; r < SUB; ++r) {
        const int i = s + r;
        u[r] = cmul(wsc(AV, i), gs);
        if (Mb > 0) u[r] = cadd(u[r], cadd(cmulc(wsc(PAm, i), qv[r]), cmulc(wsc(PDm, i), kv[r])));
        if (i == C - 1) u[r] = cadd(u[r], tail);
      }
      cf f[SUB];
      if (Mb < NB - 1) {
        cf x = {0.f, 0.f};  // sum_{i > e} r(i, e) g_i
        for (int i = C - 1; i >= s + SUB; --i) {
          cf gv = cmul(wsc(AV, i), gs);
          if (Mb > 0) gv = cadd(gv, cadd(cmulc(wsc(PAm, i), lds(RQ, i)), cmulc(wsc(PDm, i), lds(RK, i))));
          if (i == C - 1) gv = cadd(gv, tail);
          x = cmul(lds(RA, i), cadd(gv, x));
        }
        u[SUB - 1] = cadd(u[SUB - 1], x);
#pragma unroll
        for (int r = 0; r < SUB; ++r) f[r] = cadd(cmulc(kv[r], wsc(F, s + r)), cmul(wsc(BV, s + r), rend));
      } else {
#pragma unroll
        for (int r = 0; r < SUB; ++r) f[r] = wsc(BV, s + r);
      }
#pragma unroll
      for (int m = 0; m < SUB; ++m) {
        cf acc = u[SUB - 1];
#pragma unroll
        for (int i = SUB - 2; i >= m; --i) acc = cadd(u[i], cmul(al[i + 1], acc));
        if (s + m < len) {
          a.dalpha[kb + (s + m) * ks + c0] = acc.x;
          a.dalpha[kb + (s + m) * ks + c0 + 1] = -acc.y;
        }
#pragma unroll
        for (int i = m + 1; i < SUB; ++i) {
          cf E = cmul(cadd(cscale(cconj(qv[i]), sdA[(s + i) * LC + s + m]), cscale(cconj(kv[i]), sdD[(s + i) * LC + s + m])),
                      kv[m]);
          if (i == SUB - 1) E = cadd(E, f[m]);
          u[i] = cadd(cmul(al[m], u[i]), E);
        }
      }
    }
  } else {
    for (int item = tid; item < DK * NB; item += NTG) {
      const int c = item % DK, Mb = item / DK, s = Mb * SUB;
      // xv: the row operand of the second product (k, or the GDN-2 erase vector b o k)
      float al[SUB], qv[SUB], kv[SUB], xv[SUB], eg[SUB], pin[SUB], pa[SUB], pd[SUB];
#pragma unroll
      for (int r = 0; r < SUB; ++r) {
        const int i = s + r;
        al[r] = RA[i * LK + c];
        qv[r] = RQ[i * LK + c];
        kv[r] = RK[i * LK + c];
        eg[r] = G2 ? in1(a.erase, i, c) : 1.f;
        xv[r] = G2 ? eg[r] * kv[r] : kv[r];
        pin[r] = PIN[i * DK + c];
      }
      const float* PAm = PA + (size_t)(Mb > 0 ? Mb - 1 : 0) * C * DK;
      const float* PDm = PD + (size_t)(Mb > 0 ? Mb - 1 : 0) * C * DK;
#pragma unroll
      for (int r = 0; r < SUB; ++r) {
        pa[r] = Mb > 0 ? PAm[(s + r) * DK + c] : 0.f;
        pd[r] = Mb > 0 ? PDm[(s + r) * DK + c] : 0.f;
      }
      float gs = 1.f, rend = 1.f;  // gamma_(s-1); r(C-1, e)
#pragma unroll
      for (int J = 0; J < NB; ++J) {
        if (J < Mb) gs *= sPib[J * DK + c];
        if (J > Mb) rend *= sPib[J * DK + c];
      }

      // Zq_i = sum_{j <= i} dA_ij k_j r_ij, Zr_i = sum_{j < i} dD_ij k_j r_ij,
      // Zc_j = sum_{i >= j} (dA_ij q_i + dD_ij k_i) r_ij
      float fr[SUB], sg[SUB];
#pragma unroll
      for (int r = 0; r < SUB; ++r) {
        fr[r] = Mb < NB - 1 ? F[(s + r) * DK + c] : 0.f;
        sg[r] = SIG[(s + r) * DK + c];
      }
#pragma unroll
      for (int r = 0; r < SUB; ++r) {
        const int i = s + r;
        float zq = sdA[i * LC + i] * kv[r], zr = 0.f, P = 1.f;
#pragma unroll
        for (int rj = r - 1; rj >= 0; --rj) {
          P *= al[rj + 1];
          zq += sdA[i * LC + s + rj] * kv[rj] * P;
          zr += sdD[i * LC + s + rj] * kv[rj] * P;
        }
        zq += pin[r] * pa[r];
        zr += pin[r] * pd[r];
        float zc = sdA[i * LC + i] * qv[r];
        P = 1.f;
#pragma unroll
        for (int ri = r + 1; ri < SUB; ++ri) {
          P *= al[ri];
          zc += (sdA[(s + ri) * LC + i] * qv[ri] + sdD[(s + ri) * LC + i] * xv[ri]) * P;
        }
        zc += sg[r] * fr[r];
        if (i < len) {
          a.dq[kb + i * ks + c] += zq;
          if (G2) {  // zr is the row-side sum of T: part of d e, e = b o k
            a.dk[kb + i * ks + c] += eg[r] * zr + zc;
            a.derase[kb + i * ks + c] += kv[r] * zr;
          } else {
            a.dk[kb + i * ks + c] += zr + zc;
          }
        }
      }

      // gate gradient.  g_i = sum over j < s (and the start-state column j = -1) of the
      // pair weights times r(s-1, j), for rows i >= s.
      float bvs = 0.f;  // sum_{j < s} bv_j r(s-1, j)
      for (int J = 0; J < Mb; ++J) {
        float part = 0.f;
#pragma unroll
        for (int r = 0; r < SUB; ++r) part += BV[(J * SUB + r) * DK + c] * SIG[(J * SUB + r) * DK + c];
        bvs += part * between(J, Mb, c);
      }
      const float dgl = sGl[c];
      float u[SUB];
#pragma unroll
      for (int r = 0; r < SUB; ++r) {
        const int i = s + r;
        u[r] = AV[i * DK + c] * gs + qv[r] * pa[r] + xv[r] * pd[r];
        if (i == C - 1) u[r] += bvs + dgl * gs;
      }
      float f[SUB];
      if (Mb < NB - 1) {
        // rows below the block fold into its last row: X = sum_{i > e} r(i, e) g_i
        float x = 0.f;
        for (int I = NB - 1; I > Mb; --I) {
          float gv[SUB];
#pragma unroll
          for (int r = 0; r < SUB; ++r) {
            const int i = I * SUB + r;
            gv[r] = AV[i * DK + c] * gs;
            if (Mb > 0) {
              const float xi = G2 ? RK[i * LK + c] * in1(a.erase, i, c) : RK[i * LK + c];
              gv[r] += RQ[i * LK + c] * PAm[i * DK + c] + xi * PDm[i * DK + c];
            }
            if (i == C - 1) gv[r] += bvs + dgl * gs;
          }
#pragma unroll
          for (int r = SUB - 1; r >= 0; --r) x = RA[(I * SUB + r) * LK + c] * (gv[r] + x);
        }
        u[SUB - 1] += x;
#pragma unroll
        for (int r = 0; r < SUB; ++r) f[r] = kv[r] * fr[r] + BV[(s + r) * DK + c] * rend;
      } else {
#pragma unroll
        for (int r = 0; r < SUB; ++r) f[r] = BV[(s + r) * DK + c];  // the final-state row C - 1
      }
#pragma unroll
      for (int m = 0; m < SUB; ++m) {
        float acc = u[SUB - 1];
#pragma unroll
        for (int i = SUB - 2; i >= m; --i) acc = u[i] + al[i + 1] * acc;
        if (s + m < len) a.dalpha[kb + (s + m) * ks + c] = acc;
#pragma unroll
        for (int i = m + 1; i < SUB; ++i) {
          float E = (qv[i] * sdA[(s + i) * LC + s + m] + xv[i] * sdD[(s + i) * LC + s + m]) * kv[m];
          if (i == SUB - 1) E += f[m];
          u[i] = al[m] * u[i] + E;
        }
      }
    }
  }
  // the slot is free again once every wave's accesses to it have completed
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) grad_slot_release(a.gscr, a.gslots, GS.total, sSlot);
}

// ---------------------------------------------------------------------------------------
// Segment lengths of the split walks over NC chunks: c0, c1, then segc each (the last one
// what remains), as in the forward's split walk: from G = 4 on, the two short segments are
// walked in full beside the end-state and the transfer walks of the middle segments.
static void bwd_split_lengths(int NC, int G, int& segc, int& c0, int& c1) {
  if (G < 4) {
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

template <typename T, int DK, bool G2, bool CPX>
static hipError_t launch_bwd_dk(const BwdArgs& a, int NC) {
  // per-chunk grid: B H NC (fixed) or H gmax (packed; workgroups past the chunk count
  // exit); walks: one workgroup per (chain, 64 value columns)
  const int chains = (a.ctab ? a.n_seqs : a.B) * a.H, walks = chains * (a.Dv / VTW);
  const long per_chunk = a.ctab ? (long)a.H * a.gmax : (long)chains * NC;
  hipStream_t st = (hipStream_t)a.stream;
  if (per_chunk > 0) {
    if constexpr (CPX)
      hipLaunchKernelGGL((bwd_records_cpx_kernel<T, DK>), dim3(per_chunk), dim3(DK == 128 ? NTG : NT), 0, st, a, NC);
    else
      hipLaunchKernelGGL((bwd_records_kernel<T, DK, G2>), dim3(per_chunk), dim3(DK == 128 ? NTG : NT), 0, st, a, NC);
  }
  const int G = a.ctab ? 1 : bwd_walk_segments(a.B, a.T, a.H, a.Dk, a.Dv);
  if (G < 2) {
    if (per_chunk > 0)
      hipLaunchKernelGGL((bwd_state_kernel<T, DK, G2, CPX>), dim3(walks), dim3(NTW), 0, st, a, NC, WalkSplit{},
                         WalkSplit{}, 1 << 30);
    hipLaunchKernelGGL((bwd_adjoint_kernel<T, DK, CPX>), dim3(walks), dim3(NT), 0, st, a, NC, WalkSplit{}, WalkSplit{},
                       1 << 30);
  } else {
    // split walks: scratch after the chunk blocks; B [chains G][d_k][d_v], P [chains G][d_k][d_k],
    // start states [chains G][d_k][d_v], used by the state walk and then by the adjoint walk
    float* Bst = a.ws + (size_t)chains * NC * BwdLayout(DK, a.Dv).total;
    float* P = Bst + (size_t)chains * G * DK * a.Dv;
    float* X = P + (size_t)chains * G * DK * DK;
    int segc, sc0, sc1;
    bwd_split_lengths(NC, G, segc, sc0, sc1);
    auto wsp = [&](int nsub, int seg_lo, int cols, int flags, const float* start, float* end, int mirror) {
      WalkSplit w;
      w.nseg = G;
      w.segc = segc;
      w.cols = cols;
      w.flags = flags;
      w.start = start;
      w.end = end;
      w.nsub = nsub;
      w.seg_lo = seg_lo;
      w.c0 = sc0;
      w.c1 = sc1;
      w.mirror = mirror;
      return w;
    };
    const int tv = a.Dv / VTW, tk = DK / VTW, all = 1 << 30;
    const WalkSplit none;
    if (G < 4) {  // every segment through the end-state and transfer walks, equal lengths
      const int wv = chains * G * tv, wk = chains * G * tk;
      const WalkSplit wb = wsp(G, 0, a.Dv, kWNoWrite, nullptr, Bst, 0);
      const WalkSplit wp = wsp(G, 0, DK, kWNoWrite | kWZeroIn | kWIdentity, nullptr, P, 0);
      const WalkSplit wf = wsp(G, 0, a.Dv, 0, X, nullptr, 0);
      hipLaunchKernelGGL((bwd_state_kernel<T, DK, G2, CPX, 1>), dim3(wv), dim3(NTW), 0, st, a, NC, wb, none, all);
      hipLaunchKernelGGL((bwd_state_kernel<T, DK, G2, CPX, 1>), dim3(wk), dim3(NTW), 0, st, a, NC, wp, none, all);
      hipLaunchKernelGGL(walk_scan_kernel<DK>, dim3(chains * (a.Dv / 16)), dim3(256), 0, st, a.s0, P, Bst, X, G, a.Dv, 0,
                         -1);
      hipLaunchKernelGGL((bwd_state_kernel<T, DK, G2, CPX, 1>), dim3(wv), dim3(NTW), 0, st, a, NC, wf, none, all);
      hipLaunchKernelGGL((bwd_adjoint_kernel<T, DK, CPX, 1>), dim3(wv), dim3(NT), 0, st, a, NC, wb, none, all);
      hipLaunchKernelGGL((bwd_adjoint_kernel<T, DK, CPX, 1>), dim3(wk), dim3(NT), 0, st, a, NC, wp, none, all);
      hipLaunchKernelGGL(walk_scan_kernel<DK>, dim3(chains * (a.Dv / 16)), dim3(256), 0, st, a.dsT, P, Bst, X, G, a.Dv,
                         1, -1);
      hipLaunchKernelGGL((bwd_adjoint_kernel<T, DK, CPX, 1>), dim3(wv), dim3(NT), 0, st, a, NC, wf, none, all);
    } else {
      // The state walk: segment 0 in full from S_0 beside the end states of segments
      // 2 ... G - 2 from zero, segment 1 in full beside their transfers, the scan of the
      // starts of segments 3 ... G - 1, then segments 2 ... G - 1 in full.  The adjoint
      // walk runs the mirror image: segments G - 1 and G - 2 (the two short ones at the
      // sequence's end) in full from dS_T, the middle ones through end states and
      // transfers, the reverse scan, then segments G - 3 ... 0 in full.
      const int nmid = G - 3, nf = chains * tv;
      hipLaunchKernelGGL((bwd_state_kernel<T, DK, G2, CPX, 2>), dim3(nf + chains * nmid * tv), dim3(NTW), 0, st, a, NC,
                         wsp(1, 0, a.Dv, kWHead | kWEndNext, nullptr, X, 0),
                         wsp(nmid, 2, a.Dv, kWNoWrite, nullptr, Bst, 0), nf);
      hipLaunchKernelGGL((bwd_state_kernel<T, DK, G2, CPX, 2>), dim3(nf + chains * nmid * tk), dim3(NTW), 0, st, a, NC,
                         wsp(1, 1, a.Dv, kWEndNext, X, X, 0),
                         wsp(nmid, 2, DK, kWNoWrite | kWZeroIn | kWIdentity, nullptr, P, 0), nf);
      hipLaunchKernelGGL(walk_scan_kernel<DK>, dim3(chains * (a.Dv / 16)), dim3(256), 0, st, a.s0, P, Bst, X, G, a.Dv, 0,
                         2);
      hipLaunchKernelGGL((bwd_state_kernel<T, DK, G2, CPX, 1>), dim3(chains * (G - 2) * tv), dim3(NTW), 0, st, a, NC,
                         wsp(G - 2, 2, a.Dv, 0, X, nullptr, 0), none, all);
      hipLaunchKernelGGL((bwd_adjoint_kernel<T, DK, CPX, 2>), dim3(nf + chains * nmid * tv), dim3(NT), 0, st, a, NC,
                         wsp(1, G - 1, a.Dv, kWHead | kWEndPrev, nullptr, X, 1),
                         wsp(nmid, 1, a.Dv, kWNoWrite, nullptr, Bst, 1), nf);
      hipLaunchKernelGGL((bwd_adjoint_kernel<T, DK, CPX, 2>), dim3(nf + chains * nmid * tk), dim3(NT), 0, st, a, NC,
                         wsp(1, G - 2, a.Dv, kWEndPrev, X, X, 1),
                         wsp(nmid, 1, DK, kWNoWrite | kWZeroIn | kWIdentity, nullptr, P, 1), nf);
      hipLaunchKernelGGL(walk_scan_kernel<DK>, dim3(chains * (a.Dv / 16)), dim3(256), 0, st, a.dsT, P, Bst, X, G, a.Dv,
                         1, G - 3);
      hipLaunchKernelGGL((bwd_adjoint_kernel<T, DK, CPX, 1>), dim3(chains * (G - 2) * tv), dim3(NT), 0, st, a, NC,
                         wsp(G - 2, 0, a.Dv, 0, X, nullptr, 1), none, all);
    }
  }
  if (per_chunk > 0) {
    BwdArgs ag = a;
    if (!ag.gscr)  // fixed-length batch: after the chunk blocks and the split walks' scratch
      ag.gscr = a.ws + (size_t)chains * NC * BwdLayout(DK, a.Dv).total +
                bwd_split_bytes(a.B, a.T, a.H, a.Dk, a.Dv) / sizeof(float);
    ag.gslots = (int)grad_slots(per_chunk);
    hipLaunchKernelGGL(clear_words_kernel, dim3(1), dim3(256), 0, st,
                       (int*)(ag.gscr + (size_t)ag.gslots * GradScratch(DK).total), 8 * GradScratch::lock_row(ag.gslots));
    if (a.Dv == 64)
      hipLaunchKernelGGL((bwd_grads_kernel<T, DK, 64, G2, CPX>), dim3(per_chunk), dim3(NTG), 0, st, ag, NC);
    else
      hipLaunchKernelGGL((bwd_grads_kernel<T, DK, 128, G2, CPX>), dim3(per_chunk), dim3(NTG), 0, st, ag, NC);
  }
  return hipGetLastError();
}

template <typename T, bool G2, bool CPX>
static hipError_t launch_bwd_t(const BwdArgs& a, int NC) {
  return a.Dk == 64 ? launch_bwd_dk<T, 64, G2, CPX>(a, NC) : launch_bwd_dk<T, 128, G2, CPX>(a, NC);
}

// Segments per chain of the split walks (1: one walk per chain): taken, as in the forward's
// state pass, when fewer than 256 walk tiles of 64 columns would run and at least 8
// segments of 16 or more chunks fit (three launches of G - 2 segments each on 256
// workgroups beat one walk of NC chunks on few).  KDA_BWD_SEG=0 keeps one walk, =G forces
// G segments.
int bwd_walk_segments(int B, int T, int H, int dk, int dv) {
  static const int o = [] {
    const char* e = getenv("KDA_BWD_SEG");
    return e ? atoi(e) : -1;
  }();
  const int NC = (T + C - 1) / C;
  if (o >= 0) {
    const int G = min(o, NC / 16);
    return G >= 2 ? G : 1;
  }
  const long tiles = (long)B * H * (dv / VTW);
  if (tiles <= 0 || tiles >= 256) return 1;
  const int G = min((int)((256 + tiles - 1) / tiles) + 2, NC / 16);
  return G >= 8 ? G : 1;
}

size_t bwd_split_bytes(int B, int T, int H, int dk, int dv) {
  const int G = bwd_walk_segments(B, T, H, dk, dv);
  return G < 2 ? 0 : (size_t)B * H * G * dk * (2 * (size_t)dv + dk) * sizeof(float);
}

hipError_t launch_bwd(const BwdArgs& a) {
  if ((long)(a.ctab ? a.n_seqs : a.B) * a.H == 0) return hipSuccess;
  const int NC = (a.T + C - 1) / C;
  if (a.cpx) {
    if (a.erase) return hipErrorInvalidValue;
    return a.bf16 ? launch_bwd_t<bf16_t, false, true>(a, NC) : launch_bwd_t<float, false, true>(a, NC);
  }
  if (a.erase) return a.bf16 ? launch_bwd_t<bf16_t, true, false>(a, NC) : launch_bwd_t<float, true, false>(a, NC);
  return a.bf16 ? launch_bwd_t<bf16_t, false, false>(a, NC) : launch_bwd_t<float, false, false>(a, NC);
}

}  // namespace kda
