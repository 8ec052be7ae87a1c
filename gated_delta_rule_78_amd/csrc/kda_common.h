// kda_common.h -- device helpers shared by the KDA kernels (gfx950 only).
//
// bf16 values live as raw uint16 bit patterns in global memory and LDS; they
// are widened to fp32 for arithmetic and fed to the matrix cores as packed
// 8-element fragments.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef __HIP_DEVICE_COMPILE__
#define KDA_HOST_PASS 1
#endif

namespace kda {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 pair -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return (uint16_t)(pack_bf16x2(f, 0.f) & 0xFFFFu); }

// Element type policy: storage / operand type of q, k, v, alpha, beta, o and of
// the matrix-core operands.
template <typename T>
struct Elem;

template <>
struct Elem<bf16_t> {
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static float load(const void* base, size_t i) {
    return bf16_to_f32(((const uint16_t*)base)[i]);
  }
  __device__ __forceinline__ static void store(void* base, size_t i, float x) {
    ((uint16_t*)base)[i] = f32_to_bf16(x);
  }
};

template <>
struct Elem<float> {
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static float load(const void* base, size_t i) {
    return ((const float*)base)[i];
  }
  __device__ __forceinline__ static void store(void* base, size_t i, float x) {
    ((float*)base)[i] = x;
  }
};

// ---------------------------------------------------------------------------
// 16x16 output tile, K = 32 per step.  Fragment layout (per lane l, g = l >> 4,
// n = l & 15):  A slot e in 0..7 holds A[row l & 15][k-slot 8g + e],
// B slot e holds B[k-slot 8g + e][col n]; the accumulator holds
// D[4g + i][n], i = 0..3.  The k-slot -> k mapping is free as long as A and B
// agree, which lets accumulator tiles be reused as B fragments directly.
// ---------------------------------------------------------------------------
template <typename T>
struct Frag;

template <>
struct Frag<bf16_t> {
  uint32_t w[4];  // 8 bf16, slot e in half (e & 1) of word e >> 1
  __device__ __forceinline__ void set(int e, float x) {
    uint32_t h = f32_to_bf16(x);
    w[e >> 1] = (e & 1) ? ((w[e >> 1] & 0xFFFFu) | (h << 16)) : ((w[e >> 1] & 0xFFFF0000u) | h);
  }
  __device__ __forceinline__ float get(int e) const {
    uint32_t x = w[e >> 1];
    return __uint_as_float((e & 1) ? (x & 0xFFFF0000u) : (x << 16));
  }
  __device__ __forceinline__ void zero() { w[0] = w[1] = w[2] = w[3] = 0u; }
  __device__ __forceinline__ void scale(const float (&s)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = pack_bf16x2(__uint_as_float(w[i] << 16) * s[2 * i], __uint_as_float(w[i] & 0xFFFF0000u) * s[2 * i + 1]);
  }
  // slots from eight raw bf16 values
  __device__ __forceinline__ void from_raw(const uint16_t (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (uint32_t)v[2 * i] | ((uint32_t)v[2 * i + 1] << 16);
  }
  // slot e from the element at p + e * stride (bytes): a column segment of a row-major tile
  __device__ __forceinline__ void load_col8(const char* p, int stride) {
    uint16_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = *(const uint16_t*)(p + e * stride);
    from_raw(v);
  }
  // slots 0..7 from 8 consecutive elements at p (16-byte aligned)
  __device__ __forceinline__ void load8(const void* p) {
    uint4 v = *(const uint4*)p;
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
  // slots 0..3 from p0, 4..7 from p1 (each 8-byte aligned, 4 elements)
  __device__ __forceinline__ void load4x2(const void* p0, const void* p1) {
    uint2 a = *(const uint2*)p0, b = *(const uint2*)p1;
    w[0] = a.x; w[1] = a.y; w[2] = b.x; w[3] = b.y;
  }
  __device__ __forceinline__ void from_acc(const f32x4_t& lo, const f32x4_t& hi) {
    w[0] = pack_bf16x2(lo[0], lo[1]);
    w[1] = pack_bf16x2(lo[2], lo[3]);
    w[2] = pack_bf16x2(hi[0], hi[1]);
    w[3] = pack_bf16x2(hi[2], hi[3]);
  }
};

template <>
struct Frag<float> {
  float w[8];
  __device__ __forceinline__ void set(int e, float x) { w[e] = x; }
  __device__ __forceinline__ float get(int e) const { return w[e]; }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = 0.f;
  }
  __device__ __forceinline__ void scale(const float (&s)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] *= s[e];
  }
  __device__ __forceinline__ void load_col8(const char* p, int stride) {
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = *(const float*)(p + e * stride);
  }
  __device__ __forceinline__ void load8(const void* p) {
    float4 a = ((const float4*)p)[0], b = ((const float4*)p)[1];
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
  __device__ __forceinline__ void load4x2(const void* p0, const void* p1) {
    float4 a = *(const float4*)p0, b = *(const float4*)p1;
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
  __device__ __forceinline__ void from_acc(const f32x4_t& lo, const f32x4_t& hi) {
    w[0] = lo[0]; w[1] = lo[1]; w[2] = lo[2]; w[3] = lo[3];
    w[4] = hi[0]; w[5] = hi[1]; w[6] = hi[2]; w[7] = hi[3];
  }
};

__device__ __forceinline__ void mma(f32x4_t& acc, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
#ifndef KDA_HOST_PASS
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.w),
                                                __builtin_bit_cast(bf16x8_t, b.w), acc, 0, 0, 0);
#endif
}

__device__ __forceinline__ void mma(f32x4_t& acc, const Frag<float>& a, const Frag<float>& b) {
#ifndef KDA_HOST_PASS
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w[e], b.w[e], acc, 0, 0, 0);
#endif
}

__device__ __forceinline__ f32x4_t zero4() {
  f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

}  // namespace kda
