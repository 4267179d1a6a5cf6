// Device helpers for the gfx950 (CDNA4) kernels: vector types, bf16
// conversion, MFMA wrappers and wave-level exchanges.  Wave64 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ira {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 values p0, p1 as sums of two bf16 terms, packed two per word
// (p0 in the low half): hi = RNE(p), lo = RNE(p - hi).  p - hi is exact in
// fp32, so hi + lo equals p to 2^-17 relative.  One packed conversion each
// for hi and lo, and hi widened back by a shift and a mask.  The two halves
// are separate calls so that a caller can issue work on hi before lo exists.
__device__ __forceinline__ uint32_t bf16x2_hi(float p0, float p1) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p0, p1}, bf16x2));
}
__device__ __forceinline__ uint32_t bf16x2_lo(float p0, float p1, uint32_t hi) {
  const float h0 = __builtin_bit_cast(float, hi << 16);
  const float h1 = __builtin_bit_cast(float, hi & 0xffff0000u);
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p0 - h0, p1 - h1}, bf16x2));
}

// 2^x on the transcendental unit.  Callers pass -inf (giving 0) or x below
// about 58 (a logit at most kOver = 40 natural units above its softmax
// reference), far from overflow.
__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// Value held by lane (lane ^ mask) of the same wave.
__device__ __forceinline__ float xor_lane(float x, int mask) {
  return __shfl_xor(x, mask, 64);
}

// --- MFMA wrappers (accumulate in fp32) -----------------------------------
// 32x32 output tile: lane l holds column l % 32, rows 8*(i/4) + 4*(l/32) + i%4
// for i = 0..15.  16x16 output tile: lane l holds column l % 16, rows
// 4*(l/16) + i for i = 0..3.  For the operands, both A and B are indexed by
// (lane group, element) -> k with the same rule, so a consistent assignment
// of contraction indices to (lane group, element) on both sides is all that
// correctness needs.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// --- Buffer loads ------------------------------------------------------
// A raw buffer resource covers [base, base + bytes); a lane whose offset is
// outside the range reads 0 and touches no memory.  Passing kOOB as the
// offset switches a lane off without control flow, which keeps the
// compiler's load counting exact across a software pipeline.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t kOOB = 0x80000000u;
// Descriptor word 3 for untyped raw buffers on gfx9-family GPUs.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ uint4 bload128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// The same load with the non-temporal cache policy (aux bit 1 on gfx950):
// for data read exactly once, such as a decode step's K/V rows and bias.
__device__ __forceinline__ uint4 bload128_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t bload32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}

// A wave-uniform value forced into an SGPR (buffer descriptors must be
// scalar; a uniform value the compiler computed with VALU ops would
// otherwise make it emit a waterfall loop around each buffer access).
__device__ __forceinline__ uint32_t sgpr_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}
__device__ __forceinline__ uint64_t sgpr_u64(uint64_t x) {
  return (uint64_t)sgpr_u32((uint32_t)x) | ((uint64_t)sgpr_u32((uint32_t)(x >> 32)) << 32);
}

__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }
__device__ __forceinline__ int imax(int a, int b) { return a > b ? a : b; }
__device__ __forceinline__ int iclamp(int x, int lo, int hi) {
  return imin(imax(x, lo), hi);
}
// Largest multiple of m (a power of two) not above x, for any sign of x.
__device__ __forceinline__ int floor_to(int x, int m) { return x & ~(m - 1); }

}  // namespace ira
