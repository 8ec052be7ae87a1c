// kda_records.hip -- first pass of the two-pass chunk forward (bf16): the record of every
// chunk (A~ and M~ = (I + T)^-1 diag(beta) as a bf16 pair; the walk rebuilds the
// gate-scaled q and k itself), sized so that two workgroups share a compute unit
// (<= 80 KiB of LDS, <= 256 registers per lane): while one workgroup waits on a dependent
// LDS read or a barrier, the other issues.
//
// The math is that of the chunk-WY product form on the SFDA page ("El Teorema de
// Chunk-WY Constructivo"; "Principales Contribuciones" item 3) and the decay-absorbed WY
// construction on the Gated DeltaNet-2 page (section 3, efficient chunkwise parallel
// training), computed exactly as the fused chunk kernel does:
//   r_ij = prod_{m=j+1..i} alpha_m, T_ij = beta_i sum_c k_ic k_jc r_ijc (j < i),
//   A_ij = sum_c q_ic k_jc r_ijc (j <= i), M = (I + T)^-1, W = M diag(beta) (K o gamma),
// with the gate products local to 16-row sub-blocks (off-diagonal tiles anchored at
// the block edges, diagonal tiles split into the levels 8, 4, 2, 1 of the highest bit
// where the two local indices differ).
//
// What differs from the fused kernel's first half, to fit the smaller LDS:
//   * q, k, alpha are not staged in LDS: a gate item (16 rows x 2 channels of one
//     sub-block) reads them from global memory into registers, one chunk ahead;
//   * the diagonal of A (r_ii = 1) is the items' two-channel dot products summed
//     across the block's lanes, not a matrix-core pass over the raw q, k tiles;
//   * the four levels run as three passes through two level buffers, their results
//     stay in registers until every product is done;
//   * where every channel's gate product over the chunk stays >= 2^-64 in magnitude the
//     decay ratios are formed as one product per matrix (the ratio path) instead;
//   * A~ is assembled in LDS and copied out, M~ goes from registers to the record.
#include "kda_common.h"
#include "kda_internal.h"
#include "kda_record.h"
#include "kda_tile.h"

namespace kda {

namespace {

template <int DK>
struct RCfg {
  using T = bf16_t;
  static constexpr int ES = 2;
  static constexpr int NT = 256;
  static constexpr int KS = DK / 32;
  static constexpr int RS_DK = DK * ES + 16;  // [pos][channel] rows (padded)
  static constexpr int RS_C = C * ES + 16;    // [channel][pos] and [pos][pos] rows
  static constexpr int RS_F = C * 4 + 16;     // fp32 [pos][pos]
  static constexpr int RS_MB = SUB * 4 + 16;  // fp32 transposed 16x16 blocks
  static constexpr int LVL_ROWS = 24;         // per block: 8 q rows, 8 key rows (upper ranks), 8 k rows
  static constexpr int SZ_LV = NB * LVL_ROWS * RS_DK;
  static constexpr int mx(int a, int b) { return a > b ? a : b; }
  // region X.  Level path: Xq, Xk of blocks 1..3 and Y of blocks 0..2, then level buffer 1.
  // Ratio path: the row operands Q o gamma and E o gamma (E: the erase-side key).  Both:
  // M (fp32) for the inverse.
  static constexpr int OFF_XQ = 0;
  static constexpr int OFF_XK = OFF_XQ + 3 * SUB * RS_DK;
  static constexpr int OFF_Y = OFF_XK + 3 * SUB * RS_DK;
  static constexpr int SZ_X_A = OFF_Y + 3 * SUB * RS_DK;
  static constexpr int OFF_FQ = 0;
  static constexpr int OFF_FE = C * RS_DK;
  static constexpr int SZ_X_F = 2 * C * RS_DK;
  static constexpr int OFF_MM = 0;
  static constexpr int SZ_X_B = C * RS_F;
  static constexpr int SZ_X = mx(mx(SZ_X_A, SZ_LV), mx(SZ_X_F, SZ_X_B));
  // region L.  Level path: level buffer 0; ratio path: the column operand K o rho / gamma_last.
  // Then D (fp32: T before its beta row scale) and the transposed inverse blocks (MB).  A~
  // lies past all of them, so its zero entries (upper tiles, upper triangles of the diagonal
  // tiles) are written once and never overwritten.
  static constexpr int NMB = 5;
  static constexpr int OFF_TT = 0;
  static constexpr int OFF_FK = 0;
  static constexpr int OFF_MB = OFF_TT + C * RS_F;
  static constexpr int OFF_AT = mx(OFF_MB + NMB * SUB * RS_MB, SZ_LV);
  static constexpr int SZ_L = OFF_AT + C * RS_C;
  static_assert(C * RS_DK <= OFF_AT, "the ratio path's column operand stays clear of A~");
  static constexpr int BASE_X = 0;
  static constexpr int BASE_L = BASE_X + SZ_X;
  static constexpr int BASE_GT = BASE_L + SZ_L;          // block totals g[4][DK]
  static constexpr int BASE_BETA = BASE_GT + NB * DK * 4;  // beta [2][C], by chunk parity
  static constexpr int BASE_OK = BASE_BETA + 2 * C * 4;  // per-wave votes of the path choice
  static constexpr int LDS = BASE_OK + 16;
  static_assert(LDS <= 80 * 1024, "two workgroups per compute unit");
  // gate items: (block, channel pair); GRP items (lanes) per block
  static constexpr int GRP = DK / 2;
  static constexpr int NITEM = NB * GRP;
  static_assert(NITEM <= NT && GRP % 16 == 0, "item layout");
};

// Sum of d[m] over the GRP lanes of this lane's group, for 16 values at once: four
// exchange steps each halve the values a lane keeps, then plain butterfly adds.  The
// lane ends with the sum of value m = (lane % GRP) / (GRP / 16).
template <int GRP>
__device__ __forceinline__ float reduce16(const float (&d)[16], int lane) {
  float v8[8], v4[4], v2[2];
  {
    const bool up = lane & (GRP / 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float send = up ? d[j] : d[j + 8];
      v8[j] = (up ? d[j + 8] : d[j]) + __shfl_xor(send, GRP / 2);
    }
  }
  {
    const bool up = lane & (GRP / 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float send = up ? v8[j] : v8[j + 4];
      v4[j] = (up ? v8[j + 4] : v8[j]) + __shfl_xor(send, GRP / 4);
    }
  }
  {
    const bool up = lane & (GRP / 8);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float send = up ? v4[j] : v4[j + 2];
      v2[j] = (up ? v4[j + 2] : v4[j]) + __shfl_xor(send, GRP / 8);
    }
  }
  const bool up = lane & (GRP / 16);
  float v = (up ? v2[1] : v2[0]) + __shfl_xor(up ? v2[0] : v2[1], GRP / 16);
#pragma unroll
  for (int mask = GRP / 32; mask >= 1; mask >>= 1) v += __shfl_xor(v, mask);
  return v;
}

// Level-lam result tile of diagonal block I into A~ (bf16) and D (fp32): entry (row, n)
// holds the A value (row < 8) or D value (row >= 8) of upper-half rank u = row & 7 and
// lower-half rank n (n < 8).  It is a pair of the block when both ranks lie in segment
// s = n / lam; the pair's positions are then 16 I + u + lam (s + 1) and 16 I + n + lam s.
template <int lam, int RS_C, int LDF>
__device__ __forceinline__ void put_level(const f32x4_t& acc, int I, int g, int n, char* AT, float* TT) {
  if (n < 8) {
    const int s = n / lam;
    const int u0 = 4 * (g & 1);
    const int pi = 16 * I + lam * (s + 1) + u0;  // position of rank u0
    const int pj = 16 * I + n + lam * s;
    if (g < 2) {
      char* base = AT + pi * RS_C + pj * 2;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((u0 + e) / lam == s) *(uint16_t*)(base + e * RS_C) = f32_to_bf16(acc[e]);
    } else {
      float* base = TT + pi * LDF + pj;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if ((u0 + e) / lam == s) base[e * LDF] = acc[e];
    }
  }
}

// Column-side scale of eight consecutive channels of a bf16 fragment by the gate products p
// (channel pairs (2i, 2i+1) of p: complex numbers when CPX)
template <bool CPX>
__device__ __forceinline__ void scale_col(Frag<bf16_t>& f, const float (&p)[8]) {
  if constexpr (!CPX) {
    f.scale(p);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v0 = __uint_as_float(f.w[i] << 16), v1 = __uint_as_float(f.w[i] & 0xFFFF0000u);
      const Gp2<true> g{p[2 * i], p[2 * i + 1]};
      float r0, r1;
      g.col(v0, v1, r0, r1);
      f.w[i] = pack_bf16x2(r0, r1);
    }
  }
}

}  // namespace

// CPX: SFDA complex gates (the alpha tensor holds (Re, Im) of each channel pair's gate).
template <int DK, bool G2, bool CPX>
__global__ __launch_bounds__(256, G2 ? 1 : 2) void chunk_records_kernel(
    const void* __restrict__ gq, const void* __restrict__ gk, const void* __restrict__ galpha,
    const void* __restrict__ gbeta, const void* __restrict__ gerase, int Tlen, int H, char* __restrict__ ws,
    int cpw, const int* __restrict__ cu, const int* __restrict__ ctab, const int* __restrict__ ctotal, int gmax) {
  // cu != NULL: packed variable-length batch; chunk indices are global (ctab[c] =
  // (sequence, chunk of that sequence)) and records are [H][gmax]
  using K = RCfg<DK>;
  using RL = WalkRecord<DK>;
  using R = Raw<bf16_t>;
  using G = Gp2<CPX>;
  static_assert(!(G2 && CPX), "complex gates take the KDA erase/write form");
  constexpr int NT = K::NT;
  constexpr int LDF = K::RS_F / 4;
  constexpr int GRP = K::GRP;
  extern __shared__ __align__(16) char smem[];
  char* const R_X = smem + K::BASE_X;
  char* const R_L = smem + K::BASE_L;
  float* const GT = (float*)(smem + K::BASE_GT);
  float* const BETA2 = (float*)(smem + K::BASE_BETA);
  int* const OKW = (int*)(smem + K::BASE_OK);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int n = lane & 15;
  const int nchunks = cu ? gmax : (Tlen + C - 1) / C;
  const int nseg = (nchunks + cpw - 1) / cpw;
  const int bh = blockIdx.x / nseg;
  const int c_begin = (blockIdx.x % nseg) * cpw;
  const int c_end = min(cu ? *ctotal : nchunks, c_begin + cpw);
  const int b = bh / H, h = bh % H;  // varlen: bh = h (b = 0)
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

  // gate item of this thread: block iI, channels 2 icp, 2 icp + 1 (wave-uniform presence)
  const bool has_item = tid < K::NITEM;
  const int iI = tid / GRP;
  const int icp = tid % GRP;

  // one chunk ahead: the item's 16 rows of q, k, alpha (and erase gate), raw; beta of row tid & 63.
  // Loads are unconditional (rows past the end are clamped to the last row and replaced
  // when used) so that no wait is forced at issue time.
  uint32_t pq[SUB], pk[SUB], pa[SUB], pe[G2 ? SUB : 1];
  uint32_t pb = 0u;
  auto issue = [&](int c) {
    const Geo gn = geo(c);
    // chunk base (wave-uniform, 64-bit) + 32-bit row offsets: token rows are H * DK * 2
    // bytes apart and a chunk spans fewer than 2^32 bytes (checked at launch)
    const size_t base = grow(gn, gn.t0) * DK * 2;
    const uint32_t rs = (uint32_t)H * DK * 2;
    const int last = gn.len - 1 - gn.t0;
    if (has_item) {
      // the item's first row and column byte, from an opaque copy of the thread index:
      // otherwise the sixteen row offsets are hoisted out of the chunk loop and spilled,
      // and each reload waits for every load in flight
      int t = threadIdx.x;
      asm volatile("" : "+v"(t));
      const int row0 = SUB * (t / GRP);
      const uint32_t col = 4 * (t % GRP);
#pragma unroll
      for (int m = 0; m < SUB; ++m) {
        const uint32_t off = (uint32_t)min(row0 + m, last) * rs + col;
        pq[m] = *(const uint32_t*)((const char*)gq + base + off);
        pk[m] = *(const uint32_t*)((const char*)gk + base + off);
        pa[m] = *(const uint32_t*)((const char*)galpha + base + off);
        if constexpr (G2) pe[m] = *(const uint32_t*)((const char*)gerase + base + off);
      }
    }
    if constexpr (!G2) pb = ((const uint16_t*)gbeta)[grow(gn, min(gn.t0 + (tid & (C - 1)), gn.len - 1))];
  };
  if (c_begin < c_end) issue(c_begin);
  {
    // the entries of A~ that stay zero: six upper tiles (16 rows x 2 segments of 8 each)
    // and the strict upper triangles of the four diagonal tiles
    char* const AT = R_L + K::OFF_AT;
    for (int x = tid; x < 6 * 16 * 2; x += NT) {
      const int t = x >> 5, i = (x >> 1) & 15, j0 = 8 * (x & 1);
      const float z8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      st_row8<bf16_t>(AT + (16 * kUpI[t] + i) * K::RS_C + (16 * kUpJ[t] + j0) * 2, z8);
    }
    for (int x = tid; x < NB * SUB * SUB; x += NT) {
      const int I = x >> 8, i = (x >> 4) & 15, j = x & 15;
      if (j > i) *(uint16_t*)(AT + (16 * I + i) * K::RS_C + (16 * I + j) * 2) = 0;
    }
  }

  for (int chunk = c_begin; chunk < c_end; ++chunk) {
    const Geo gm = geo(chunk);
    const int t0 = gm.t0;
    char* const rec = ws + gm.rec * RL::BYTES;
    // (no barrier here: every LDS region this chunk writes before its first barrier -- beta,
    // in the buffer of this chunk's parity, and the block totals -- is one the previous
    // chunk no longer reads; the regions its record stores read are rewritten only after
    // that first barrier, which every wave reaches after its record stores)
    float* const BETA = BETA2 + ((chunk - c_begin) & 1) * C;
    // lane-dependent indices, recomputed per chunk from an opaque copy of the thread
    // index: otherwise every LDS address derived from them is hoisted out of the loop
    // and held (spilled) across it
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int n = lane & 15;
    const int iI = tid / GRP;
    const int icp = tid % GRP;

    // ---------------- item registers, fp32 (rows past the end: q = k = 0, alpha = 1)
    // Rows past the end keep the clamped copies of the last row's q and k: their beta is 0,
    // so their rows of T and of M~ are zero, they add nothing to any state, and their
    // outputs are never stored.  Only their gate must be the identity (it enters the gate
    // products): (1, 1) for real gates, 1 + 0i for complex ones.
    float qf[SUB][2], kf[SUB][2];
    G al[SUB];
    constexpr uint32_t kOne = CPX ? 0x00003F80u : R::kOneWord;
    const int lim = gm.len - t0 - SUB * iI;  // rows of this item that exist
#pragma unroll
    for (int m = 0; m < SUB; ++m) {
      R::unpack(pq[m], qf[m][0], qf[m][1]);
      R::unpack(pk[m], kf[m][0], kf[m][1]);
      R::unpack(m < lim ? pa[m] : kOne, al[m].x, al[m].y);
    }
    // the key as the erase side reads it: k (KDA), b o k (Gated DeltaNet-2; the erase gate
    // stays packed, the product is formed at each use)
    uint32_t er[G2 ? SUB : 1];
    if constexpr (G2) {
#pragma unroll
      for (int m = 0; m < SUB; ++m) er[m] = pe[m];
    }
    auto read_key = [&](int m, float& e0, float& e1) {
      e0 = kf[m][0];
      e1 = kf[m][1];
      if constexpr (G2) {
        float b0, b1;
        R::unpack(er[m], b0, b1);
        e0 *= b0;
        e1 *= b1;
      }
    };
    if (tid < C) BETA[tid] = (t0 + tid < gm.len) ? (G2 ? 1.f : __uint_as_float(pb << 16)) : 0.f;

    // ================= phase B0: block totals, and the choice of path.  The ratio path
    // factors r_ij = gamma_i * (rho_j / gamma_last) with gamma_i the running product from
    // the chunk start and rho_j the one from j + 1 to the chunk end: one product per matrix
    // instead of the block and level split.  It is taken only when every channel's
    // product over the whole chunk has magnitude >= 2^-64: gamma_last divides nothing
    // smaller, no factor leaves the fp32 / bf16 range (|gamma_i| >= |gamma_last| when
    // |alpha| <= 1), and each decayed product keeps its relative rounding.  A zero gate,
    // or a run of tiny ones, sends the chunk down the level path, which never divides.
    if (has_item) {
      G f = G::one();
#pragma unroll
      for (int m = 0; m < SUB; ++m) f *= al[m];
      *(float2*)(GT + iI * DK + 2 * icp) = make_float2(f.x, f.y);
    }
    lds_barrier();
    G t0v = G::one(), t1v = G::one(), t2v = G::one(), t3v = G::one();
    if (has_item) {
      const float2 a0 = *(const float2*)(GT + 2 * icp), a1 = *(const float2*)(GT + DK + 2 * icp);
      const float2 a2 = *(const float2*)(GT + 2 * DK + 2 * icp), a3 = *(const float2*)(GT + 3 * DK + 2 * icp);
      t0v = G{a0.x, a0.y};
      t1v = G{a1.x, a1.y};
      t2v = G{a2.x, a2.y};
      t3v = G{a3.x, a3.y};
    }
    bool ratio = false;
    if constexpr (!CPX) {
      const G gl = t0v * t1v * t2v * t3v;
      const bool ok = !has_item || (fabsf(gl.x) >= 0x1p-64f && fabsf(gl.y) >= 0x1p-64f);
      const bool wave_ok = __ballot(!ok) == 0;
      if constexpr (K::NITEM == NT) {
        // every wave holds the items of one block over all channel pairs, so its own vote
        // is the chunk's: no exchange
        ratio = wave_ok;
      } else {
        if (lane == 0) OKW[wave] = wave_ok ? 1 : 0;
        lds_barrier();
        ratio = (OKW[0] & OKW[1] & OKW[2] & OKW[3]) != 0;
      }
    }
    float* const TT = (float*)(R_L + K::OFF_TT);
    char* const AT = R_L + K::OFF_AT;
    // the next chunk's inputs, from one place and unconditionally (the last chunk loads
    // itself again): loads issued on both sides of the path choice would meet in
    // register copies, which wait for every load in flight
    issue(min(chunk + 1, c_end - 1));

    if (ratio) {
      // ================= ratio path, phase F1: row operands Q o gamma, E o gamma and the
      // column operand K o rho / gamma_last, each as [pos][channel] bf16
      if (has_item) {
        const G gp = iI == 0 ? G::one() : iI == 1 ? t0v : iI == 2 ? t0v * t1v : t0v * t1v * t2v;
        const G rp = iI == 3 ? G::one() : iI == 2 ? t3v : iI == 1 ? t2v * t3v : t1v * t2v * t3v;
        const G gl = t0v * t1v * t2v * t3v;
        char* fq = R_X + K::OFF_FQ + (SUB * iI) * K::RS_DK + 4 * icp;
        char* fe = R_X + K::OFF_FE + (SUB * iI) * K::RS_DK + 4 * icp;
        char* fk = R_L + K::OFF_FK + (SUB * iI) * K::RS_DK + 4 * icp;
        G f = gp;
#pragma unroll
        for (int m = 0; m < SUB; ++m) {
          f *= al[m];
          float e0, e1;
          read_key(m, e0, e1);
          R::st(fq + m * K::RS_DK, qf[m][0] * f.x, qf[m][1] * f.y);
          R::st(fe + m * K::RS_DK, e0 * f.x, e1 * f.y);
        }
        // (|gamma_last| >= 2^-64 here: the hardware reciprocal, about one ulp, is ample for
        // operands that are rounded to bf16)
        G bb{rp.x * __builtin_amdgcn_rcpf(gl.x), rp.y * __builtin_amdgcn_rcpf(gl.y)};
#pragma unroll
        for (int m = SUB - 1; m >= 0; --m) {
          R::st(fk + m * K::RS_DK, kf[m][0] * bb.x, kf[m][1] * bb.y);
          bb *= al[m];
        }
      }
      lds_barrier();
      // ================= phase F2: the ten lower 16 x 16 tiles of A (Q o gamma rows) and of
      // D (E o gamma rows) against the column operand; five jobs per wave
      f32x4_t acc[5];
#pragma unroll
      for (int s = 0; s < 5; ++s) {
        const int j = wave + 4 * s, t = j % 10;
        const int I = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
        const int J = t - (I * (I + 1)) / 2;
        const char* arow = R_X + (j < 10 ? K::OFF_FQ : K::OFF_FE) + (16 * I + n) * K::RS_DK;
        const char* brow = R_L + K::OFF_FK + (16 * J + n) * K::RS_DK;
        Frag<bf16_t> fa[K::KS], fb[K::KS];
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) {
          fa[ks].load8(arow + (32 * ks + 8 * g) * 2);
          fb[ks].load8(brow + (32 * ks + 8 * g) * 2);
        }
        acc[s] = zero4();
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) mma(acc[s], fa[ks], fb[ks]);
      }
      lds_barrier();  // the column operand is read out before D lands over it
#pragma unroll
      for (int s = 0; s < 5; ++s) {
        const int j = wave + 4 * s, t = j % 10;
        const int I = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
        const int J = t - (I * (I + 1)) / 2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int li = 4 * g + e, gi = 16 * I + li, gj = 16 * J + n;
          if (j < 10)
            *(uint16_t*)(AT + gi * K::RS_C + gj * 2) = f32_to_bf16(I > J || n <= li ? acc[s][e] : 0.f);
          else
            TT[gi * LDF + gj] = acc[s][e];
        }
      }
    } else {
      // ================= level path, phase B: block-anchored operands, diagonal of A, level 8
      // level-lam operands of the item's block into level buffer `buf`: rows u (q) and
      // 8 + u (erase-side key) of the upper-half ranks, prefix products from the upper
      // half's start; rows 16 + v (k) of the lower-half ranks, suffix products to its end
      auto write_level = [&](char* buf, int lam) {
        char* LA = buf + iI * K::LVL_ROWS * K::RS_DK + 4 * icp;
        char* LB = LA + 16 * K::RS_DK;
        G f = G::one();
#pragma unroll
        for (int m = 0; m < SUB; ++m) {
          if (m & lam) {
            if ((m & (lam - 1)) == 0)
              f = al[m];
            else
              f *= al[m];
            const int u = (m / (2 * lam)) * lam + (m & (lam - 1));
            float k0, k1, r0, r1;
            read_key(m, k0, k1);
            f.row(qf[m][0], qf[m][1], r0, r1);
            R::st(LA + u * K::RS_DK, r0, r1);
            f.row(k0, k1, r0, r1);
            R::st(LA + (8 + u) * K::RS_DK, r0, r1);
          }
        }
        G bb = G::one();
#pragma unroll
        for (int m = SUB - 1; m >= 0; --m) {
          if (!(m & lam)) {
            if ((m & (lam - 1)) == lam - 1)
              bb = G::one();
            else
              bb *= al[m + 1];
            const int v = (m / (2 * lam)) * lam + (m & (lam - 1));
            float r0, r1;
            bb.col(kf[m][0], kf[m][1], r0, r1);
            R::st(LB + v * K::RS_DK, r0, r1);
          }
        }
      };

      float adiag = 0.f;
      if (has_item) {
        if (iI >= 1) {
          char* xq = R_X + K::OFF_XQ + (SUB * (iI - 1)) * K::RS_DK + 4 * icp;
          char* xk = R_X + K::OFF_XK + (SUB * (iI - 1)) * K::RS_DK + 4 * icp;
          G f = G::one();
#pragma unroll
          for (int m = 0; m < SUB; ++m) {
            f *= al[m];
            float k0, k1, r0, r1;
            read_key(m, k0, k1);
            f.row(qf[m][0], qf[m][1], r0, r1);
            R::st(xq + m * K::RS_DK, r0, r1);
            f.row(k0, k1, r0, r1);
            R::st(xk + m * K::RS_DK, r0, r1);
          }
        }
        if (iI <= 2) {
          char* y = R_X + K::OFF_Y + (SUB * iI) * K::RS_DK + 4 * icp;
          G bb = G::one();
#pragma unroll
          for (int m = SUB - 1; m >= 0; --m) {
            float r0, r1;
            bb.col(kf[m][0], kf[m][1], r0, r1);
            R::st(y + m * K::RS_DK, r0, r1);
            bb *= al[m];
          }
        }
        float d[SUB];
#pragma unroll
        for (int m = 0; m < SUB; ++m) {
          const float q0 = qf[m][0], q1 = qf[m][1];
          const float k0 = kf[m][0], k1 = kf[m][1];
          d[m] = fmaf(q1, k1, q0 * k0);
        }
        adiag = reduce16<GRP>(d, lane);
        write_level(R_L, 8);
      }
      lds_barrier();

      // ================= phase M1: the six off-diagonal tiles of A and T, level 8 tiles.
      // Waves 0, 1: two off-diagonal jobs; waves 2, 3: one off-diagonal job and two
      // level-8 blocks.  Job j: (I, J) = (1,0) (2,1) (3,2) (2,0) (3,1) (3,0).
      auto lvl_job = [&](const char* buf, int I, f32x4_t& acc) {
        const char* LA = buf + I * K::LVL_ROWS * K::RS_DK;
        const char* LB = LA + 16 * K::RS_DK;
        Frag<bf16_t> fa[K::KS], fb[K::KS];
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) {
          const int c0 = 32 * ks + 8 * g;
          fa[ks].load8(LA + n * K::RS_DK + c0 * 2);
          if (n < 8)
            fb[ks].load8(LB + n * K::RS_DK + c0 * 2);
          else
            fb[ks].zero();
        }
        acc = zero4();
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) mma(acc, fa[ks], fb[ks]);
      };
      auto off_job = [&](int j, f32x4_t& ra, f32x4_t& rt) {
        const int I = kOffI[j], J = kOffJ[j], pi = kOffPi[j];
        const char* xq = R_X + K::OFF_XQ + (SUB * (I - 1) + n) * K::RS_DK;
        const char* xk = R_X + K::OFF_XK + (SUB * (I - 1) + n) * K::RS_DK;
        const char* y = R_X + K::OFF_Y + (SUB * J + n) * K::RS_DK;
        Frag<bf16_t> fa[K::KS], fk[K::KS], fb[K::KS];
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) {
          const int c0 = 32 * ks + 8 * g;
          fb[ks].load8(y + c0 * 2);
          fa[ks].load8(xq + c0 * 2);
          fk[ks].load8(xk + c0 * 2);
        }
        ra = zero4();
        rt = zero4();
#pragma unroll
        for (int ks = 0; ks < K::KS; ++ks) {
          if (pi >= 0) {
            // whole blocks between J and I: g1 (pi 0), g1 g2 (pi 1), g2 (pi 2)
            const int c0 = 32 * ks + 8 * g;
            const float* G1 = GT + (pi == 2 ? 2 : 1) * DK + c0;
            float4 p0 = *(const float4*)G1, p1 = *(const float4*)(G1 + 4);
            if (pi == 1) {
              const float4 e0 = *(const float4*)(GT + 2 * DK + c0), e1 = *(const float4*)(GT + 2 * DK + c0 + 4);
              const G a0 = G{p0.x, p0.y} * G{e0.x, e0.y}, a1 = G{p0.z, p0.w} * G{e0.z, e0.w};
              const G a2 = G{p1.x, p1.y} * G{e1.x, e1.y}, a3 = G{p1.z, p1.w} * G{e1.z, e1.w};
              p0 = make_float4(a0.x, a0.y, a1.x, a1.y);
              p1 = make_float4(a2.x, a2.y, a3.x, a3.y);
            }
            const float pv8[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
            scale_col<CPX>(fb[ks], pv8);
          }
          mma(ra, fa[ks], fb[ks]);
          mma(rt, fk[ks], fb[ks]);
        }
      };
      f32x4_t acc1[4];
      off_job(wave, acc1[0], acc1[1]);
      if (wave < 2) {
        off_job(wave + 4, acc1[2], acc1[3]);
      } else {
        lvl_job(R_L, 2 * (wave - 2), acc1[2]);
        lvl_job(R_L, 2 * (wave - 2) + 1, acc1[3]);
      }
      lds_barrier();

      // ================= phase C: level 4 (buffer 1) and level 2 (buffer 0) operands
      if (has_item) {
        write_level(R_X, 4);
        write_level(R_L, 2);
      }
      lds_barrier();

      // ================= phase M2: level 4 and level 2 tiles of block `wave`
      f32x4_t acc2[2];
      lvl_job(R_X, wave, acc2[0]);
      lvl_job(R_L, wave, acc2[1]);
      lds_barrier();

      // ================= phase C2: level 1 operands (buffer 0), then the next chunk's inputs
      if (has_item) write_level(R_L, 1);
      lds_barrier();

      // ================= phase M3: level 1 tile of block `wave`
      f32x4_t acc3;
      lvl_job(R_L, wave, acc3);
      lds_barrier();

      // ================= phase D: every product into D (fp32) and A~ (bf16)
      auto put_off = [&](int j, const f32x4_t& ra, const f32x4_t& rt) {
        const int I = kOffI[j], J = kOffJ[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int gi = 16 * I + 4 * g + e, gj = 16 * J + n;
          *(uint16_t*)(AT + gi * K::RS_C + gj * 2) = f32_to_bf16(ra[e]);
          TT[gi * LDF + gj] = rt[e];
        }
      };
      put_off(wave, acc1[0], acc1[1]);
      if (wave < 2) {
        put_off(wave + 4, acc1[2], acc1[3]);
      } else {
        put_level<8, K::RS_C, LDF>(acc1[2], 2 * (wave - 2), g, n, AT, TT);
        put_level<8, K::RS_C, LDF>(acc1[3], 2 * (wave - 2) + 1, g, n, AT, TT);
      }
      put_level<4, K::RS_C, LDF>(acc2[0], wave, g, n, AT, TT);
      put_level<2, K::RS_C, LDF>(acc2[1], wave, g, n, AT, TT);
      put_level<1, K::RS_C, LDF>(acc3, wave, g, n, AT, TT);
      if (has_item && (tid % (GRP / 16)) == 0) {
        const int i = SUB * iI + (tid % GRP) / (GRP / 16);
        *(uint16_t*)(AT + i * K::RS_C + i * 2) = f32_to_bf16(adiag);
      }
    }
    lds_barrier();

    // ================= phase I: M = (I + T)^-1 with T = diag(beta) D
    float* const MM = (float*)(R_X + K::OFF_MM);
    char* const MB = R_L + K::OFF_MB;  // transposed 16x16 blocks: 0 N00, 1 N11, 2 N22, 3 M10, 4 M20
    auto mb_row = [&](int blk, int r) -> float* { return (float*)(MB + (blk * SUB + r) * K::RS_MB); };
    if (wave == 0) {
      // diagonal blocks by forward substitution: lane = (block I, column col); the lane
      // also holds row `col` of T_II, broadcast across the 16-lane row
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
      dpp_sources_ready(tr);
      float x[SUB], nx[SUB];  // column of N_II and its negation
#define KDA_FS_ROW(i)                                                                     \
  {                                                                                       \
    float acc = (col == i) ? 1.f : 0.f;                                                   \
    _Pragma("unroll") for (int p = 0; p < i; ++p) acc = fmac_bcast<i>(acc, tr[p], nx[p]); \
    x[i] = acc;                                                                           \
    nx[i] = -acc;                                                                         \
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
    lds_barrier();
    // off-diagonal blocks, M_IJ = -N_II sum_{K=J}^{I-1} T_IK M_KJ, in three dependency
    // stages.  In product instruction s the k-slot is 4 g + s, so an accumulator tile
    // is directly the B operand of the next product.
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
      } else {  // P20 = T20 N00
        a_T(2, 0, a);
        b_MB(0, bb);
        mm4(keep, a, bb);
      }
    }
    lds_barrier();
    if (wave == 3) {  // M20 = -N22 (P20 + T21 M10)
      float a[4], bb[4];
      a_T(2, 1, a);
      b_MB(3, bb);
      mm4(keep, a, bb);
      put_M(2, 0, neg_N_times(2, keep), 4);
    }
    lds_barrier();
    if (wave == 0) {  // M30 = -N33 (P30 + T32 M20)
      float a[4], bb[4];
      a_T(3, 2, a);
      b_MB(4, bb);
      mm4(keep, a, bb);
      put_M(3, 0, neg_N_times(3, keep), -1);
    }
    lds_barrier();
    // ================= the record: M~ = M diag(beta) as a bf16 pair (hi, and the rounding
    // residual lo), straight from registers; A~ copied from LDS.  Both lower matrices are
    // stored as their rows 0..31 x columns 0..31 and rows 32..63 x columns 0..63, in
    // 16-byte units permuted per row (WalkRecord::unit).
    // Every thread stores exactly two units (the second repeating the first where the
    // 384 units run out: the same bytes to the same place), so the number of stores in
    // flight is the same in every wave and the next chunk's wait for its prefetched inputs
    // (loaded before these stores) need not wait for the stores as well.
    constexpr int NU_TOP = 32 * 4, NU_ALL = NU_TOP + 32 * 8;
    static_assert(NU_ALL <= 2 * NT, "two units per thread");
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int x = it == 0 || tid + NT >= NU_ALL ? tid : tid + NT;
      const bool top = x < NU_TOP;
      const int i = top ? x / 4 : 32 + (x - NU_TOP) / 8, u = top ? x % 4 : (x - NU_TOP) % 8;
      const int off = (top ? i * RL::RS_TOP : RL::BOT + (i - 32) * RL::RS_BOT) + 16 * RL::unit(i, u);
      const int j0 = 8 * u;
      const float4 m0 = *(const float4*)(MM + i * LDF + j0), m1 = *(const float4*)(MM + i * LDF + j0 + 4);
      const float4 b0 = *(const float4*)(BETA + j0), b1 = *(const float4*)(BETA + j0 + 4);
      float v8[8] = {m0.x * b0.x, m0.y * b0.y, m0.z * b0.z, m0.w * b0.w,
                     m1.x * b1.x, m1.y * b1.y, m1.z * b1.z, m1.w * b1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (j0 + e > i) v8[e] = 0.f;
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hw[e] = pack_bf16x2(v8[2 * e], v8[2 * e + 1]);
        lw[e] = pack_bf16x2(v8[2 * e] - __uint_as_float(hw[e] << 16), v8[2 * e + 1] - __uint_as_float(hw[e] & 0xFFFF0000u));
      }
      *(uint4*)(rec + RL::MH + off) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      *(uint4*)(rec + RL::ML + off) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      *(uint4*)(rec + RL::A + off) = *(const uint4*)(AT + i * K::RS_C + j0 * 2);
    }
  }
}

template <int DK, bool G2, bool CPX>
static hipError_t launch_records_t(const ChunkArgs& a, char* ws, int cpw) {
  using K = RCfg<DK>;
  auto kern = chunk_records_kernel<DK, G2, CPX>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, K::LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  // varlen: workgroups over (head, runs of global chunks); b = 0
  const int BH = a.cu ? a.H : a.B * a.H;
  const int nchunks = a.cu ? a.gmax : (a.T + C - 1) / C;
  const int nseg = (nchunks + cpw - 1) / cpw;
  if ((long)BH * nseg == 0) return hipSuccess;
  if ((long)C * a.H * DK * 2 >= (1L << 32)) return hipErrorInvalidValue;  // 32-bit row offsets
  hipLaunchKernelGGL(kern, dim3(BH * nseg), dim3(K::NT), K::LDS, (hipStream_t)a.stream, a.q, a.k, a.alpha, a.beta,
                     a.erase, a.T, a.H, ws, cpw, a.cu, a.ctab, a.ctab_total, a.gmax);
  return hipGetLastError();
}

// bf16 records with the two-workgroups-per-CU kernel (d_k = 64 or 128)
hipError_t launch_records(const ChunkArgs& a, void* ws, int cpw) {
  if (!a.bf16 || (a.dk != 64 && a.dk != 128) || (a.cpx && a.erase)) return hipErrorInvalidValue;
  char* w = (char*)ws;
  if (a.cpx) return a.dk == 64 ? launch_records_t<64, false, true>(a, w, cpw) : launch_records_t<128, false, true>(a, w, cpw);
  if (a.erase) return a.dk == 64 ? launch_records_t<64, true, false>(a, w, cpw) : launch_records_t<128, true, false>(a, w, cpw);
  return a.dk == 64 ? launch_records_t<64, false, false>(a, w, cpw) : launch_records_t<128, false, false>(a, w, cpw);
}

}  // namespace kda
