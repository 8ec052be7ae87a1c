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

constexpr int NT = 256;  // threads per workgroup of every kernel here

// ---------------------------------------------------------------------------------------
// One 16x16 fp32 tile: acc[i][j] = sum_k fa(i, k) fb(k, j), K a multiple of 4.  Lane
// (n = lane & 15, g = lane >> 4) feeds A[n][k0 + g] and B[k0 + g][n]; the result holds
// element (4 g + r, n) in acc[r].
// K a multiple of 16: the operands of the next 16 k are loaded while the current four
// steps run.
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

// Product over a grid of tm x tn tiles spread over the workgroup's waves:
// fe(i, j, sum_k fa(i, k) fb(k, j)) for every i < 16 tm, j < 16 tn.
template <class FA, class FB, class FE>
__device__ __forceinline__ void wg_mm(int tm, int tn, int K, FA fa, FB fb, FE fe) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, n = lane & 15, g = lane >> 4;
  for (int t = wave; t < tm * tn; t += NT / 64) {
    const int i0 = (t / tn) * 16, j0 = (t % tn) * 16;
    const f32x4_t acc = tile_mm(
        K, [&](int r, int k) { return fa(i0 + r, k); }, [&](int k, int c) { return fb(k, j0 + c); });
#pragma unroll
    for (int r = 0; r < 4; ++r) fe(i0 + 4 * g + r, j0 + n, acc[r]);
  }
}

// Rows of one (b, h) sequence in a [B, T, H, d] tensor, restricted to one chunk: rows at
// or past `len` read as `pad` (q, k, v, dO: 0; alpha: 1; beta: 0).
template <typename T>
struct Rows {
  const void* p;
  size_t base, stride;  // element offset of chunk row 0, elements between rows
  int len;
  __device__ __forceinline__ float at(int i, int c, float pad = 0.f) const {
    return i < len ? Elem<T>::load(p, base + (size_t)i * stride + c) : pad;
  }
};

struct ChunkGeom {
  int b, h, n, t0, len;
};

__device__ __forceinline__ ChunkGeom chunk_geom(int g, int NC, int H, int T) {
  ChunkGeom q;
  q.n = g % NC;
  const int bh = g / NC;
  q.b = bh / H;
  q.h = bh % H;
  q.t0 = q.n * C;
  q.len = min(C, T - q.t0);
  return q;
}

// element offset of (b, t0, h, 0) in a [B, T, H, d] tensor
__device__ __forceinline__ size_t row0(const ChunkGeom& q, int T, int H, int d) {
  return (((size_t)q.b * T + q.t0) * H + q.h) * (size_t)d;
}

// prod_{J < x < I} Pib[x][c]: the gates of the whole blocks strictly between J and I
__device__ __forceinline__ float between(const float* pib, int dk, int J, int I, int c) {
  float p = 1.f;
  for (int x = J + 1; x < I; ++x) p *= pib[x * dk + c];
  return p;
}

}  // namespace

// ---------------------------------------------------------------------------------------
// bwd_records_kernel: one workgroup per (b, h, chunk).
template <typename T>
__global__ __launch_bounds__(NT) void bwd_records_kernel(BwdArgs a, int NC) {
  const int tid = threadIdx.x, dk = a.Dk;
  const BwdLayout L(dk, a.Dv);
  const ChunkGeom cg = chunk_geom(blockIdx.x, NC, a.H, a.T);
  float* ch = a.ws + (size_t)blockIdx.x * L.total;
  const Rows<T> Q{a.q, row0(cg, a.T, a.H, dk), (size_t)a.H * dk, cg.len};
  const Rows<T> K{a.k, Q.base, Q.stride, cg.len};
  const Rows<T> AL{a.alpha, Q.base, Q.stride, cg.len};
  const Rows<T> BE{a.beta, ((size_t)cg.b * a.T + cg.t0) * a.H + cg.h, (size_t)a.H, cg.len};
  float *GAM = ch + L.gam, *RHO = ch + L.rho, *PIN = ch + L.pin, *SIG = ch + L.sig, *PIB = ch + L.pib;

  __shared__ float sA[C][C + 1], sD[C][C + 1], sM[C][C + 1];
  __shared__ float sRed[136 * 129];  // 136 pairs of a 16-row block x up to 128 channels (+1 pad)
  __shared__ float sY[3][16][17];
  __shared__ float sB[C];

  // (a) gate products per key channel: gamma (from the chunk start), rho (to the chunk
  // end, exclusive), pi (from the block start, inclusive), sigma (to the block end,
  // exclusive) and the block totals.
  for (int c = tid; c < dk; c += NT) {
    float gm = 1.f, pib[NB];
    for (int I = 0; I < NB; ++I) {
      float al[SUB];
#pragma unroll
      for (int r = 0; r < SUB; ++r) al[r] = AL.at(I * SUB + r, c, 1.f);
      float p = 1.f;
#pragma unroll
      for (int r = 0; r < SUB; ++r) {
        const int i = I * SUB + r;
        p *= al[r];
        gm *= al[r];
        PIN[i * dk + c] = p;
        GAM[i * dk + c] = gm;
      }
      PIB[I * dk + c] = pib[I] = p;
      float sf = 1.f;
#pragma unroll
      for (int r = SUB - 1; r >= 0; --r) {
        SIG[(I * SUB + r) * dk + c] = sf;
        sf *= al[r];
      }
    }
    // rho_i = sigma_i * the whole blocks after i's block
    float tail = 1.f;
    for (int I = NB - 1; I >= 0; --I) {
      float sf = tail;
#pragma unroll
      for (int r = SUB - 1; r >= 0; --r) {
        const int i = I * SUB + r;
        RHO[i * dk + c] = sf;
        sf *= AL.at(i, c, 1.f);
      }
      tail *= pib[I];
    }
  }
  for (int i = tid; i < C; i += NT) sB[i] = BE.at(i, 0);
  for (int x = tid; x < C * C; x += NT) {
    const int i = x / C, j = x % C;
    if (j > i) sA[i][j] = sD[i][j] = 0.f;
  }
  __syncthreads();

  // (b) the six off-diagonal 16x16 tiles (I > J) of A and of D, anchored at row
  // s_I - 1: r_ij = pi_i * (sigma_j * the whole blocks between J and I).
  {
    const int lane = tid & 63, wave = tid >> 6, n = lane & 15, g = lane >> 4;
    for (int job = wave; job < 12; job += NT / 64) {
      // tiles (I, J) = (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
      const int mat = job / 6, p = job % 6, I = p < 1 ? 1 : (p < 3 ? 2 : 3), J = p - I * (I - 1) / 2;
      const int si = I * SUB, sj = J * SUB;
      const f32x4_t acc = tile_mm(
          dk,
          [&](int r, int c) {
            const int i = si + r;
            return (mat ? K.at(i, c) : Q.at(i, c)) * PIN[i * dk + c];
          },
          [&](int c, int col) {
            const int j = sj + col;
            return K.at(j, c) * SIG[j * dk + c] * between(PIB, dk, J, I, c);
          });
#pragma unroll
      for (int r = 0; r < 4; ++r) (mat ? sD : sA)[si + 4 * g + r][sj + n] = acc[r];
    }
  }

  // (c) the diagonal tiles: per channel products, then sums over the channels.
  for (int I = 0; I < NB; ++I) {
    const int s = I * SUB;
    for (int mat = 0; mat < 2; ++mat) {
      for (int c = tid; c < dk; c += NT) {
        float kv[SUB], xv[SUB], av[SUB];
#pragma unroll
        for (int r = 0; r < SUB; ++r) {
          kv[r] = K.at(s + r, c);
          xv[r] = mat ? kv[r] : Q.at(s + r, c);
          av[r] = AL.at(s + r, c, 1.f);
        }
#pragma unroll
        for (int rj = 0; rj < SUB; ++rj) {
          float P = 1.f;
#pragma unroll
          for (int ri = rj; ri < SUB; ++ri) {
            if (ri > rj) P *= av[ri];
            sRed[(ri * (ri + 1) / 2 + rj) * (dk + 1) + c] = (mat && ri == rj) ? 0.f : xv[ri] * kv[rj] * P;
          }
        }
      }
      __syncthreads();
      for (int p = tid; p < 136; p += NT) {
        int ri = 0;
        while ((ri + 1) * (ri + 2) / 2 <= p) ++ri;
        const int rj = p - ri * (ri + 1) / 2;
        float sum = 0.f, sum2 = 0.f;
#pragma unroll 8
        for (int c = 0; c < dk; c += 2) {
          sum += sRed[p * (dk + 1) + c];
          sum2 += sRed[p * (dk + 1) + c + 1];
        }
        sum += sum2;
        (mat ? sD : sA)[s + ri][s + rj] = sum;
      }
      __syncthreads();
    }
  }

  // (d) M = (I + diag(beta) D)^-1: the four diagonal 16x16 blocks by substitution, then
  // block rows I = 1..3: M_IJ = -M_II sum_{J <= K < I} (beta D)_IK M_KJ.
  if (tid < 4 * SUB) {
    const int s = (tid / SUB) * SUB, col = tid % SUB;
    for (int r = 0; r < SUB; ++r) {
      float acc = 0.f;
      for (int j = 0; j < r; ++j) acc += sD[s + r][s + j] * sM[s + j][s + col];
      sM[s + r][s + col] = (r == col ? 1.f : 0.f) - sB[s + r] * acc;
    }
  }
  for (int x = tid; x < C * C; x += NT) {
    const int i = x / C, j = x % C;
    if (j / SUB > i / SUB) sM[i][j] = 0.f;
  }
  __syncthreads();
  for (int I = 1; I < NB; ++I) {
    const int si = I * SUB, lane = tid & 63, wave = tid >> 6, n = lane & 15, g = lane >> 4;
    for (int J = wave; J < I; J += NT / 64) {
      const int sj = J * SUB;
      const f32x4_t y = tile_mm(
          si - sj, [&](int r, int kk) { return sB[si + r] * sD[si + r][sj + kk]; },
          [&](int kk, int col) { return sM[sj + kk][sj + col]; });
#pragma unroll
      for (int r = 0; r < 4; ++r) sY[J][4 * g + r][n] = y[r];
    }
    __syncthreads();
    for (int J = wave; J < I; J += NT / 64) {
      const int sj = J * SUB;
      const f32x4_t m = tile_mm(
          SUB, [&](int r, int kk) { return sM[si + r][si + kk]; }, [&](int kk, int col) { return sY[J][kk][col]; });
#pragma unroll
      for (int r = 0; r < 4; ++r) sM[si + 4 * g + r][sj + n] = -m[r];
    }
    __syncthreads();
  }

  // (e) W = M diag(beta) (K o gamma); A, D, M to the workspace
  wg_mm(
      C / 16, dk / 16, C, [&](int i, int j) { return sM[i][j] * sB[j]; },
      [&](int j, int c) { return K.at(j, c) * GAM[j * dk + c]; },
      [&](int i, int c, float x) { ch[L.W + i * dk + c] = x; });
  for (int x = tid; x < C * C; x += NT) {
    const int i = x / C, j = x % C;
    ch[L.A + x] = sA[i][j];
    ch[L.D + x] = sD[i][j];
    ch[L.M + x] = sM[i][j];
  }
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
}

}  // namespace

// bwd_state_kernel: chunks in order; writes the chunk-start state S_n and Delta_n.
template <typename T, int DK>
__global__ __launch_bounds__(NT) void bwd_state_kernel(BwdArgs a, int NC) {
  constexpr int LM = C + 4, LW = DK + 4, LV = VTW + 4;
  __shared__ float sM[C * LM], sW[C * LW], sKrT[DK * LM], sV[C * LV], sGl[DK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, g = lane >> 4;
  const int dv = a.Dv, ntile = dv / VTW, bh = blockIdx.x / ntile, v0 = (blockIdx.x % ntile) * VTW;
  const int col = v0 + 16 * wave + n;  // this lane's state column
  const BwdLayout L(DK, dv);
  f32x4_t S[DK / 16];
#pragma unroll
  for (int I = 0; I < DK / 16; ++I)
#pragma unroll
    for (int r = 0; r < 4; ++r) S[I][r] = a.s0 ? a.s0[((size_t)bh * DK + 16 * I + 4 * g + r) * dv + col] : 0.f;
  for (int nc = 0; nc < NC; ++nc) {
    const ChunkGeom cg = chunk_geom(bh * NC + nc, NC, a.H, a.T);
    float* ch = a.ws + (size_t)(bh * NC + nc) * L.total;
    const size_t kb = row0(cg, a.T, a.H, DK), ks = (size_t)a.H * DK;
    const size_t vb = row0(cg, a.T, a.H, dv), vs = (size_t)a.H * dv;
    const size_t bb = ((size_t)cg.b * a.T + cg.t0) * a.H + cg.h;
    __syncthreads();  // the previous chunk's LDS reads are done
    // M; W; (K o rho)^T; diag(beta) V (so that M (beta o V) = Mt V); gamma_last
#pragma unroll
    for (int it = 0; it < C * C / 4 / NT; ++it) {
      const int x = tid + it * NT, i = x / (C / 4), j = 4 * (x % (C / 4));
      *(float4*)(sM + i * LM + j) = *(const float4*)(ch + L.M + i * C + j);
    }
#pragma unroll
    for (int it = 0; it < C * DK / 4 / NT; ++it) {
      const int x = tid + it * NT, i = x / (DK / 4), c = 4 * (x % (DK / 4));
      *(float4*)(sW + i * LW + c) = *(const float4*)(ch + L.W + i * DK + c);
      const float4 kv = i < cg.len ? ld4<T>(a.k, kb + i * ks + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 rv = *(const float4*)(ch + L.rho + i * DK + c);
      sKrT[(c + 0) * LM + i] = kv.x * rv.x;
      sKrT[(c + 1) * LM + i] = kv.y * rv.y;
      sKrT[(c + 2) * LM + i] = kv.z * rv.z;
      sKrT[(c + 3) * LM + i] = kv.w * rv.w;
    }
#pragma unroll
    for (int it = 0; it < C * VTW / 4 / NT; ++it) {
      const int x = tid + it * NT, j = x / (VTW / 4), c = 4 * (x % (VTW / 4));
      float4 vv = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j < cg.len) {
        vv = ld4<T>(a.v, vb + j * vs + v0 + c);
        const float bt = Elem<T>::load(a.beta, bb + (size_t)j * a.H);
        vv.x *= bt;
        vv.y *= bt;
        vv.z *= bt;
        vv.w *= bt;
      }
      *(float4*)(sV + j * LV + c) = vv;
    }
    for (int c = tid; c < DK; c += NT) sGl[c] = ch[L.gam + (C - 1) * DK + c];
    __syncthreads();
#pragma unroll
    for (int I = 0; I < DK / 16; ++I)
#pragma unroll
      for (int r = 0; r < 4; ++r) ch[L.S + (16 * I + 4 * g + r) * dv + col] = S[I][r];
    // Delta = M (beta o V) - W S
    f32x4_t Dl[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4_t acc = zero4f();
      const float* mrow = sM + (16 * I + n) * LM;
#pragma unroll
      for (int k0 = 0; k0 < C; k0 += 16)
        mm16(acc, mrow, k0, [&](int t) { return sV[(k0 + 4 * g + t) * LV + 16 * wave + n]; });
      const float* wrow = sW + (16 * I + n) * LW;
#pragma unroll
      for (int kt = 0; kt < DK / 16; ++kt) mm16(acc, wrow, 16 * kt, [&](int t) { return S[kt][t]; }, -1.f);
      Dl[I] = acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) ch[L.DL + (16 * I + 4 * g + r) * dv + col] = acc[r];
    }
    if (nc + 1 < NC) {
      // S' = gamma_L o S + (K o rho)^T Delta
#pragma unroll
      for (int I = 0; I < DK / 16; ++I) {
        f32x4_t acc = zero4f();
        const float* krow = sKrT + (16 * I + n) * LM;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) mm16(acc, krow, 16 * kt, [&](int t) { return Dl[kt][t]; });
#pragma unroll
        for (int r = 0; r < 4; ++r) S[I][r] = sGl[16 * I + 4 * g + r] * S[I][r] + acc[r];
      }
    }
  }
}

// bwd_adjoint_kernel: chunks in reverse; writes the end-state adjoint dS'_n and dDelta_n
// of every chunk, and dS_0.
template <typename T, int DK>
__global__ __launch_bounds__(NT) void bwd_adjoint_kernel(BwdArgs a, int NC) {
  constexpr int LK = DK + 4, LM = C + 4, LV = VTW + 4;
  __shared__ float sKr[C * LK], sAT[C * LM], sQgT[DK * LM], sWT[DK * LM], sO[C * LV], sGl[DK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, g = lane >> 4;
  const int dv = a.Dv, ntile = dv / VTW, bh = blockIdx.x / ntile, v0 = (blockIdx.x % ntile) * VTW;
  const int col = v0 + 16 * wave + n;
  const BwdLayout L(DK, dv);
  f32x4_t dS[DK / 16];
#pragma unroll
  for (int I = 0; I < DK / 16; ++I)
#pragma unroll
    for (int r = 0; r < 4; ++r) dS[I][r] = a.dsT ? a.dsT[((size_t)bh * DK + 16 * I + 4 * g + r) * dv + col] : 0.f;
  for (int nc = NC - 1; nc >= 0; --nc) {
    const ChunkGeom cg = chunk_geom(bh * NC + nc, NC, a.H, a.T);
    float* ch = a.ws + (size_t)(bh * NC + nc) * L.total;
    const size_t kb = row0(cg, a.T, a.H, DK), ks = (size_t)a.H * DK;
    const size_t vb = row0(cg, a.T, a.H, dv), vs = (size_t)a.H * dv;
    __syncthreads();
    // K o rho; A^T; (Q o gamma)^T; W^T; dO; gamma_last
#pragma unroll
    for (int it = 0; it < C * DK / 4 / NT; ++it) {
      const int x = tid + it * NT, i = x / (DK / 4), c = 4 * (x % (DK / 4));
      const bool in = i < cg.len;
      const float4 kv = in ? ld4<T>(a.k, kb + i * ks + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 qv = in ? ld4<T>(a.q, kb + i * ks + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 rv = *(const float4*)(ch + L.rho + i * DK + c);
      const float4 gv = *(const float4*)(ch + L.gam + i * DK + c);
      const float4 wv = *(const float4*)(ch + L.W + i * DK + c);
      *(float4*)(sKr + i * LK + c) = make_float4(kv.x * rv.x, kv.y * rv.y, kv.z * rv.z, kv.w * rv.w);
      sQgT[(c + 0) * LM + i] = qv.x * gv.x;
      sQgT[(c + 1) * LM + i] = qv.y * gv.y;
      sQgT[(c + 2) * LM + i] = qv.z * gv.z;
      sQgT[(c + 3) * LM + i] = qv.w * gv.w;
      sWT[(c + 0) * LM + i] = wv.x;
      sWT[(c + 1) * LM + i] = wv.y;
      sWT[(c + 2) * LM + i] = wv.z;
      sWT[(c + 3) * LM + i] = wv.w;
    }
#pragma unroll
    for (int it = 0; it < C * C / 4 / NT; ++it) {
      const int x = tid + it * NT, j = x / (C / 4), i = 4 * (x % (C / 4));
      const float4 av = *(const float4*)(ch + L.A + j * C + i);
      sAT[(i + 0) * LM + j] = av.x;
      sAT[(i + 1) * LM + j] = av.y;
      sAT[(i + 2) * LM + j] = av.z;
      sAT[(i + 3) * LM + j] = av.w;
    }
#pragma unroll
    for (int it = 0; it < C * VTW / 4 / NT; ++it) {
      const int x = tid + it * NT, i = x / (VTW / 4), c = 4 * (x % (VTW / 4));
      *(float4*)(sO + i * LV + c) = i < cg.len ? ld4<T>(a.dO, vb + i * vs + v0 + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int c = tid; c < DK; c += NT) sGl[c] = ch[L.gam + (C - 1) * DK + c];
    __syncthreads();
#pragma unroll
    for (int I = 0; I < DK / 16; ++I)
#pragma unroll
      for (int r = 0; r < 4; ++r) ch[L.DS + (16 * I + 4 * g + r) * dv + col] = dS[I][r];
    // dDelta = (K o rho) dS' + A^T dO
    f32x4_t dD[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4_t acc = zero4f();
      const float* krow = sKr + (16 * I + n) * LK;
#pragma unroll
      for (int kt = 0; kt < DK / 16; ++kt) mm16(acc, krow, 16 * kt, [&](int t) { return dS[kt][t]; });
      const float* arow = sAT + (16 * I + n) * LM;
#pragma unroll
      for (int k0 = 0; k0 < C; k0 += 16)
        mm16(acc, arow, k0, [&](int t) { return sO[(k0 + 4 * g + t) * LV + 16 * wave + n]; });
      dD[I] = acc;
#pragma unroll
      for (int r = 0; r < 4; ++r) ch[L.DDL + (16 * I + 4 * g + r) * dv + col] = acc[r];
    }
    // dS = gamma_L o dS' + (Q o gamma)^T dO - W^T dDelta
#pragma unroll
    for (int I = 0; I < DK / 16; ++I) {
      f32x4_t acc = zero4f();
      const float* qrow = sQgT + (16 * I + n) * LM;
#pragma unroll
      for (int k0 = 0; k0 < C; k0 += 16)
        mm16(acc, qrow, k0, [&](int t) { return sO[(k0 + 4 * g + t) * LV + 16 * wave + n]; });
      const float* wrow = sWT + (16 * I + n) * LM;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) mm16(acc, wrow, 16 * kt, [&](int t) { return dD[kt][t]; }, -1.f);
#pragma unroll
      for (int r = 0; r < 4; ++r) dS[I][r] = sGl[16 * I + 4 * g + r] * dS[I][r] + acc[r];
    }
  }
  if (a.ds0) {
#pragma unroll
    for (int I = 0; I < DK / 16; ++I)
#pragma unroll
      for (int r = 0; r < 4; ++r) a.ds0[((size_t)bh * DK + 16 * I + 4 * g + r) * dv + col] = dS[I][r];
  }
}

// ---------------------------------------------------------------------------------------
// bwd_grads_kernel: one workgroup per (b, h, chunk).
template <typename T>
__global__ __launch_bounds__(NT) void bwd_grads_kernel(BwdArgs a, int NC) {
  const int tid = threadIdx.x, dk = a.Dk, dv = a.Dv;
  const BwdLayout L(dk, dv);
  const ChunkGeom cg = chunk_geom(blockIdx.x, NC, a.H, a.T);
  float* ch = a.ws + (size_t)blockIdx.x * L.total;
  const Rows<T> Q{a.q, row0(cg, a.T, a.H, dk), (size_t)a.H * dk, cg.len};
  const Rows<T> K{a.k, Q.base, Q.stride, cg.len};
  const Rows<T> AL{a.alpha, Q.base, Q.stride, cg.len};
  const Rows<T> V{a.v, row0(cg, a.T, a.H, dv), (size_t)a.H * dv, cg.len};
  const Rows<T> DO{a.dO, V.base, V.stride, cg.len};
  const size_t ob = ((size_t)cg.b * a.T + cg.t0) * a.H + cg.h;  // beta / dbeta row 0
  const Rows<T> BE{a.beta, ob, (size_t)a.H, cg.len};
  const size_t okb = Q.base, ovb = V.base;                      // dq / dk / dalpha and dv row 0
  const float *GAM = ch + L.gam, *RHO = ch + L.rho, *PIN = ch + L.pin, *SIG = ch + L.sig, *PIB = ch + L.pib;
  const float *S = ch + L.S, *DL = ch + L.DL, *DS = ch + L.DS, *DD = ch + L.DDL;
  float *AV = ch + L.AV, *BV = ch + L.BV, *DW = ch + L.DW, *F = ch + L.F, *PA = ch + L.PA, *PD = ch + L.PD;

  __shared__ float sdA[C][C + 1], sdT[C][C + 1], sdM[C][C + 1], sX[C][C + 1], sM[C][C + 1];
  __shared__ float sB[C], sdB[C], sGl[128];

  for (int x = tid; x < C * C; x += NT) sM[x / C][x % C] = ch[L.M + x];
  for (int i = tid; i < C; i += NT) sB[i] = BE.at(i, 0);
  __syncthreads();

  // ---- products over the value dimension
  // d(Q o gamma) = dO S^T: dq = . o gamma, av = . o q
  wg_mm(
      C / 16, dk / 16, dv, [&](int i, int v) { return DO.at(i, v); }, [&](int v, int c) { return S[c * dv + v]; },
      [&](int i, int c, float x) {
        if (i < cg.len) a.dq[okb + (size_t)i * Q.stride + c] = x * GAM[i * dk + c];
        AV[i * dk + c] = x * Q.at(i, c);
      });
  // d(K o rho) = Delta dS'^T: dk = . o rho, bv = . o k
  wg_mm(
      C / 16, dk / 16, dv, [&](int i, int v) { return DL[i * dv + v]; }, [&](int v, int c) { return DS[c * dv + v]; },
      [&](int i, int c, float x) {
        if (i < cg.len) a.dk[okb + (size_t)i * Q.stride + c] = x * RHO[i * dk + c];
        BV[i * dk + c] = x * K.at(i, c);
      });
  // dW = -dDelta S^T
  wg_mm(
      C / 16, dk / 16, dv, [&](int i, int v) { return DD[i * dv + v]; }, [&](int v, int c) { return S[c * dv + v]; },
      [&](int i, int c, float x) { DW[i * dk + c] = -x; });
  // dA = (dO Delta^T) o low
  wg_mm(
      C / 16, C / 16, dv, [&](int i, int v) { return DO.at(i, v); }, [&](int v, int j) { return DL[j * dv + v]; },
      [&](int i, int j, float x) { sdA[i][j] = j <= i ? x : 0.f; });
  // dV = Mt^T dDelta
  wg_mm(
      C / 16, dv / 16, C, [&](int j, int i) { return sM[i][j] * sB[j]; }, [&](int i, int v) { return DD[i * dv + v]; },
      [&](int j, int v, float x) {
        if (j < cg.len) a.dv[ovb + (size_t)j * V.stride + v] = x;
      });
  // dgamma_L = rowsum(dS' o S)
  for (int c = tid; c < dk; c += NT) {
    float s = 0.f;
#pragma unroll 16
    for (int v = 0; v < dv; v += 4) {
      const float4 x = *(const float4*)(DS + c * dv + v), y = *(const float4*)(S + c * dv + v);
      s += x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
    }
    sGl[c] = s;
  }
  __syncthreads();

  // ---- dMt = (dDelta V^T + dW (K o gamma)^T) o low;  d(K o gamma) = Mt^T dW
  wg_mm(
      C / 16, C / 16, dv + dk, [&](int i, int kk) { return kk < dv ? DD[i * dv + kk] : DW[i * dk + kk - dv]; },
      [&](int kk, int j) { return kk < dv ? V.at(j, kk) : K.at(j, kk - dv) * GAM[j * dk + kk - dv]; },
      [&](int i, int j, float x) { sdM[i][j] = j <= i ? x : 0.f; });
  wg_mm(
      C / 16, dk / 16, C, [&](int j, int i) { return sM[i][j] * sB[j]; }, [&](int i, int c) { return DW[i * dk + c]; },
      [&](int j, int c, float x) {
        if (j < cg.len) a.dk[okb + (size_t)j * Q.stride + c] += x * GAM[j * dk + c];
        AV[j * dk + c] += x * K.at(j, c);
      });
  __syncthreads();

  // ---- dbeta (first part) = colsum(dMt o M);  X = dMt Mt^T
  for (int j = tid; j < C; j += NT) {
    float s = 0.f;
    for (int i = j; i < C; ++i) s += sdM[i][j] * sM[i][j];
    sdB[j] = s;
  }
  wg_mm(
      C / 16, C / 16, C, [&](int i, int kk) { return sdM[i][kk]; }, [&](int kk, int j) { return sM[j][kk] * sB[kk]; },
      [&](int i, int j, float x) { sX[i][j] = x; });
  __syncthreads();
  // dT = -(M^T X) o strict-low
  wg_mm(
      C / 16, C / 16, C, [&](int i, int kk) { return sM[kk][i]; }, [&](int kk, int j) { return sX[kk][j]; },
      [&](int i, int j, float x) { sdT[i][j] = j < i ? -x : 0.f; });
  __syncthreads();
  // dbeta += rowsum(dT o D); dD = diag(beta) dT (in place)
  for (int i = tid; i < C; i += NT) {
    float s = 0.f;
#pragma unroll 16
    for (int j = 0; j < i; ++j) s += sdT[i][j] * ch[L.D + i * C + j];
    if (i < cg.len) a.dbeta[ob + (size_t)i * a.H] = sdB[i] + s;
    for (int j = 0; j < i; ++j) sdT[i][j] *= sB[i];
  }
  __syncthreads();
  float(*sdD)[C + 1] = sdT;

  // ---- block-anchored products for the decayed sums
  // PA^M = dA[>= s_M, < s_M] Khat^M, PD^M likewise with dD (M = 1..3), where
  // Khat^M_j = k_j r(s_M - 1, j) = k_j sigma_j (blocks between)
  for (int Mb = 1; Mb < NB; ++Mb) {
    const int s = Mb * SUB;
    for (int mat = 0; mat < 2; ++mat) {
      float* out = (mat ? PD : PA) + (size_t)(Mb - 1) * C * dk;
      wg_mm(
          NB - Mb, dk / 16, s, [&](int i, int j) { return mat ? sdD[s + i][j] : sdA[s + i][j]; },
          [&](int j, int c) { return K.at(j, c) * SIG[j * dk + c] * between(PIB, dk, j / SUB, Mb, c); },
          [&](int i, int c, float x) { out[(s + i) * dk + c] = x; });
    }
  }
  // F^M_j = sum_{i > e_M} (dA_ij q_i + dD_ij k_i) r(i, e_M) for j in block M (M = 0..2),
  // r(i, e_M) = pi_i (blocks between)
  for (int Mb = 0; Mb < NB - 1; ++Mb) {
    const int s = Mb * SUB, e1 = s + SUB, nM = C - e1;
    wg_mm(
        1, dk / 16, 2 * nM,
        [&](int j, int kk) { return kk < nM ? sdA[e1 + kk][s + j] : sdD[e1 + kk - nM][s + j]; },
        [&](int kk, int c) {
          const int i = e1 + (kk < nM ? kk : kk - nM);
          const float x = kk < nM ? Q.at(i, c) : K.at(i, c);
          return x * PIN[i * dk + c] * between(PIB, dk, Mb, i / SUB, c);
        },
        [&](int j, int c, float x) { F[(s + j) * dk + c] = x; });
  }
  __syncthreads();

  // ---- per (channel, block): the decayed sums' in-block parts, dq / dk, the gate gradient
  for (int item = tid; item < dk * NB; item += NT) {
    const int c = item % dk, Mb = item / dk, s = Mb * SUB;
    float al[SUB], qv[SUB], kv[SUB];
#pragma unroll
    for (int r = 0; r < SUB; ++r) {
      al[r] = AL.at(s + r, c, 1.f);
      qv[r] = Q.at(s + r, c);
      kv[r] = K.at(s + r, c);
    }
    float pib[NB];
#pragma unroll
    for (int J = 0; J < NB; ++J) pib[J] = PIB[J * dk + c];
    float gs = 1.f, rend = 1.f;  // gamma_(s-1); r(C-1, e)
#pragma unroll
    for (int J = 0; J < NB; ++J) {
      if (J < Mb) gs *= pib[J];
      if (J > Mb) rend *= pib[J];
    }
    const float* PAm = PA + (size_t)(Mb > 0 ? Mb - 1 : 0) * C * dk;
    const float* PDm = PD + (size_t)(Mb > 0 ? Mb - 1 : 0) * C * dk;

    // Zq_i = sum_{j <= i} dA_ij k_j r_ij, Zr_i = sum_{j < i} dD_ij k_j r_ij,
    // Zc_j = sum_{i >= j} (dA_ij q_i + dD_ij k_i) r_ij
#pragma unroll
    for (int r = 0; r < SUB; ++r) {
      const int i = s + r;
      float zq = sdA[i][i] * kv[r], zr = 0.f, P = 1.f;
#pragma unroll
      for (int rj = r - 1; rj >= 0; --rj) {
        P *= al[rj + 1];
        zq += sdA[i][s + rj] * kv[rj] * P;
        zr += sdD[i][s + rj] * kv[rj] * P;
      }
      if (Mb > 0) {
        const float pin = PIN[i * dk + c];
        zq += pin * PAm[i * dk + c];
        zr += pin * PDm[i * dk + c];
      }
      float zc = sdA[i][i] * qv[r];
      P = 1.f;
#pragma unroll
      for (int ri = r + 1; ri < SUB; ++ri) {
        P *= al[ri];
        zc += (sdA[s + ri][i] * qv[ri] + sdD[s + ri][i] * kv[ri]) * P;
      }
      if (Mb < NB - 1) zc += SIG[i * dk + c] * F[i * dk + c];
      if (i < cg.len) {
        a.dq[okb + (size_t)i * Q.stride + c] += zq;
        a.dk[okb + (size_t)i * Q.stride + c] += zr + zc;
      }
    }

    // gate gradient.  g_i = sum over j < s (and the start-state column j = -1) of the
    // pair weights times r(s-1, j), for rows i >= s.
    float bvs = 0.f;  // sum_{j < s} bv_j r(s-1, j)
    for (int J = 0; J < Mb; ++J) {
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < SUB; ++r) part += BV[(J * SUB + r) * dk + c] * SIG[(J * SUB + r) * dk + c];
      float w = 1.f;
      for (int x = J + 1; x < Mb; ++x) w *= pib[x];
      bvs += part * w;
    }
    const float dgl = sGl[c];
    auto g_at = [&](int i) {
      float g = AV[i * dk + c] * gs;
      if (Mb > 0) g += Q.at(i, c) * PAm[i * dk + c] + K.at(i, c) * PDm[i * dk + c];
      if (i == C - 1) g += bvs + dgl * gs;
      return g;
    };
    float u[SUB];
#pragma unroll
    for (int r = 0; r < SUB; ++r) u[r] = g_at(s + r);
    float f[SUB];
    if (Mb < NB - 1) {
      // rows below the block fold into its last row: X = sum_{i > e} r(i, e) g_i
      float x = 0.f;
      for (int I = NB - 1; I > Mb; --I) {
        float gv[SUB], av[SUB];
#pragma unroll
        for (int r = 0; r < SUB; ++r) {
          gv[r] = g_at(I * SUB + r);
          av[r] = AL.at(I * SUB + r, c, 1.f);
        }
#pragma unroll
        for (int r = SUB - 1; r >= 0; --r) x = av[r] * (gv[r] + x);
      }
      u[SUB - 1] += x;
#pragma unroll
      for (int r = 0; r < SUB; ++r) f[r] = kv[r] * F[(s + r) * dk + c] + BV[(s + r) * dk + c] * rend;
    } else {
#pragma unroll
      for (int r = 0; r < SUB; ++r) f[r] = BV[(s + r) * dk + c];  // the final-state row C - 1
    }
#pragma unroll
    for (int m = 0; m < SUB; ++m) {
      float acc = u[SUB - 1];
#pragma unroll
      for (int i = SUB - 2; i >= m; --i) acc = u[i] + al[i + 1] * acc;
      if (s + m < cg.len) a.dalpha[okb + (size_t)(s + m) * Q.stride + c] = acc;
#pragma unroll
      for (int i = m + 1; i < SUB; ++i) {
        float E = (qv[i] * sdA[s + i][s + m] + kv[i] * sdD[s + i][s + m]) * kv[m];
        if (i == SUB - 1) E += f[m];
        u[i] = al[m] * u[i] + E;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
template <typename T, int DK>
static hipError_t launch_bwd_dk(const BwdArgs& a, int NC) {
  const int BH = a.B * a.H, walks = BH * (a.Dv / VTW);
  hipStream_t st = (hipStream_t)a.stream;
  if (NC > 0) {
    hipLaunchKernelGGL((bwd_records_kernel<T>), dim3(BH * NC), dim3(NT), 0, st, a, NC);
    hipLaunchKernelGGL((bwd_state_kernel<T, DK>), dim3(walks), dim3(NT), 0, st, a, NC);
  }
  hipLaunchKernelGGL((bwd_adjoint_kernel<T, DK>), dim3(walks), dim3(NT), 0, st, a, NC);
  if (NC > 0) hipLaunchKernelGGL((bwd_grads_kernel<T>), dim3(BH * NC), dim3(NT), 0, st, a, NC);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_bwd_t(const BwdArgs& a, int NC) {
  return a.Dk == 64 ? launch_bwd_dk<T, 64>(a, NC) : launch_bwd_dk<T, 128>(a, NC);
}

hipError_t launch_bwd(const BwdArgs& a) {
  if ((long)a.B * a.H == 0) return hipSuccess;
  const int NC = (a.T + C - 1) / C;
  return a.bf16 ? launch_bwd_t<bf16_t>(a, NC) : launch_bwd_t<float>(a, NC);
}

}  // namespace kda
