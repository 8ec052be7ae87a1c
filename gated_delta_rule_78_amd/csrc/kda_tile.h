// kda_tile.h -- tile helpers shared by the chunk kernels (gfx950 only): chunk geometry,
// the off-diagonal tile jobs of the intra-chunk products, packed element pairs, row
// stores, fence-free workgroup barriers and the fp32 matrix-core step of the inverse.
#pragma once
#include "kda_common.h"

namespace kda {

namespace {

constexpr int C = 64;
constexpr int SUB = 16;
constexpr int NB = C / SUB;

// Off-diagonal tile jobs (I, J) and the block-product Pi they need
// (-1: adjacent, none; 0: g1; 1: g1 g2; 2: g2).
__constant__ int kOffI[6] = {1, 2, 3, 2, 3, 3};
__constant__ int kOffJ[6] = {0, 1, 2, 0, 1, 0};
__constant__ int kOffPi[6] = {-1, -1, -1, 0, 2, 1};
// Upper 16x16 tiles of A~ that must read as zero.
__constant__ int kUpI[6] = {0, 0, 0, 1, 1, 2};
__constant__ int kUpJ[6] = {1, 2, 3, 2, 3, 3};

// Two adjacent channels of one row, kept packed until used.
template <typename T>
struct Raw;
template <>
struct Raw<bf16_t> {
  typedef uint32_t type;
  __device__ __forceinline__ static type ld(const char* p) { return *(const uint32_t*)p; }
  __device__ __forceinline__ static void unpack(type w, float& a, float& b) {
    a = __uint_as_float(w << 16);
    b = __uint_as_float(w & 0xFFFF0000u);
  }
  __device__ __forceinline__ static void st(char* p, float a, float b) { *(uint32_t*)p = pack_bf16x2(a, b); }
  static constexpr uint32_t kOneWord = 0x3F803F80u;  // two bf16 ones
};
template <>
struct Raw<float> {
  typedef float2 type;
  __device__ __forceinline__ static type ld(const char* p) { return *(const float2*)p; }
  __device__ __forceinline__ static void unpack(type w, float& a, float& b) {
    a = w.x;
    b = w.y;
  }
  __device__ __forceinline__ static void st(char* p, float a, float b) { *(float2*)p = make_float2(a, b); }
  static constexpr uint32_t kOneWord = 0x3F800000u;
};

__device__ __forceinline__ void st_elem(char* p, float x, int es) {
  if (es == 2)
    *(uint16_t*)p = f32_to_bf16(x);
  else
    *(float*)p = x;
}

// eight consecutive elements of one row (16-byte aligned for bf16, 32-byte for fp32)
template <typename T>
__device__ __forceinline__ void st_row8(char* p, const float (&v)[8]);
template <>
__device__ __forceinline__ void st_row8<bf16_t>(char* p, const float (&v)[8]) {
  *(uint4*)p = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                          pack_bf16x2(v[6], v[7]));
}
template <>
__device__ __forceinline__ void st_row8<float>(char* p, const float (&v)[8]) {
  ((float4*)p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  ((float4*)p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// `bytes` (a multiple of 16) from LDS to global memory, 16 bytes per thread and step
template <int NT>
__device__ __forceinline__ void copy_flat(char* dst, const char* src, int bytes, int tid) {
  for (int j = tid; j < bytes / 16; j += NT) *(uint4*)(dst + j * 16) = *(const uint4*)(src + j * 16);
}

// value of `x` held by lane `src` (0..15) of this lane's 16-lane DPP row
template <int src>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + src, 0xF,
                                                               0xF, true));
}

// acc + (x of lane `src` of this lane's 16-lane DPP row) * y in one v_fmac_f32 with a
// row_newbcast source, one rounding as fmaf.  x must have been written at least two
// wait states before (dpp_sources_ready): the compiler does not see the DPP read inside
// the asm.
template <int src>
__device__ __forceinline__ float fmac_bcast(float acc, float x, float y) {
#ifndef KDA_HOST_PASS
  asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "+v"(acc) : "v"(x), "v"(y), "n"(src));
#endif
  return acc;
}

// Two wait states after the writes of the sixteen values read by fmac_bcast (ordered
// after them: they are the asm's operands, left in place).
__device__ __forceinline__ void dpp_sources_ready(float (&t)[16]) {
#ifndef KDA_HOST_PASS
  asm volatile("s_nop 1"
               : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]), "+v"(t[4]), "+v"(t[5]), "+v"(t[6]), "+v"(t[7]),
                 "+v"(t[8]), "+v"(t[9]), "+v"(t[10]), "+v"(t[11]), "+v"(t[12]), "+v"(t[13]), "+v"(t[14]), "+v"(t[15]));
#endif
}

// 16x16 fp32 product step: acc += A B with A[row n][k-slot 4 g + s], B[k-slot 4 g + s][col n]
__device__ __forceinline__ void mm4(f32x4_t& acc, const float (&a)[4], const float (&b)[4]) {
#ifndef KDA_HOST_PASS
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
#endif
}

// Workgroup barriers without a memory fence (a fence would also wait for the DMA still
// streaming the next chunk).  The empty asm statements keep the compiler from moving
// memory accesses across them; the explicit waits make this wave's LDS writes (and, for
// full_barrier, its DMA and global accesses) complete before the barrier.
__device__ __forceinline__ void lds_barrier() {
#ifndef KDA_HOST_PASS
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
#endif
}

__device__ __forceinline__ void full_barrier() {
#ifndef KDA_HOST_PASS
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
#endif
}

// Running gate products on an item's channel pair (2c, 2c+1).  Real gates (KDA / CKDA /
// Gated DeltaNet-2): two independent channels, (x, y) their products.  Complex gates
// (SFDA page, "Arquitectura Central": the pair is one complex coordinate and its gate the
// complex number lambda = (Re, Im) in channels (2c, 2c+1)): (x, y) = (Re, Im) of the
// product.  The row side of a decayed product takes the conjugate (the transpose of a
// rotation-decay block), the column side the product itself:
//   r_ij = F_i B_j,  x_i^T R_ij y_j = (conj(F_i) x_i) . (B_j y_j)  over real channel pairs.
template <bool CPX>
struct Gp2 {
  float x, y;
  __device__ __forceinline__ static Gp2 one() { return Gp2{1.f, CPX ? 0.f : 1.f}; }
  __device__ __forceinline__ Gp2 operator*(const Gp2& o) const {
    if constexpr (CPX) return Gp2{x * o.x - y * o.y, x * o.y + y * o.x};
    else return Gp2{x * o.x, y * o.y};
  }
  __device__ __forceinline__ void operator*=(const Gp2& o) { *this = *this * o; }
  // row-side operand of the pair (v0, v1): conj(F) v (complex) or (F0 v0, F1 v1)
  __device__ __forceinline__ void row(float v0, float v1, float& r0, float& r1) const {
    if constexpr (CPX) {
      r0 = x * v0 + y * v1;
      r1 = x * v1 - y * v0;
    } else {
      r0 = v0 * x;
      r1 = v1 * y;
    }
  }
  // column-side operand: B v (complex) or (B0 v0, B1 v1)
  __device__ __forceinline__ void col(float v0, float v1, float& r0, float& r1) const {
    if constexpr (CPX) {
      r0 = x * v0 - y * v1;
      r1 = x * v1 + y * v0;
    } else {
      r0 = v0 * x;
      r1 = v1 * y;
    }
  }
};

}  // namespace

}  // namespace kda
