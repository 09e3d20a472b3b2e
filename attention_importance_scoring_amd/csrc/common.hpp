// Device helpers shared by the gfx950 kernels of the scoring library.
//
// MFMA fragments.  Both v_mfma_f32_32x32x16_bf16 and v_mfma_f32_32x32x2_f32
// take, in lane l, operand row (l % 32) and a slice of the contraction
// index chosen by the half-wave h = l / 32, and return the 32x32 fp32
// product with lane l holding column n = l % 32 and rows
//   m(i) = 8 * (i / 4) + 4 * h + (i % 4),  i = 0 .. 15.
// The contraction only needs A and B to use the same slice mapping, so each
// lane reads one contiguous half of a row: half h covers head-dim elements
// [h * D / 2, (h + 1) * D / 2) as NV 16-byte vectors.  One bf16 vector feeds
// one 32x32x16 MFMA; one fp32 vector (4 floats) feeds four 32x32x2 MFMAs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

struct bf16_t {  // storage tag: bfloat16 kept as raw 16-bit words
  uint16_t bits;
};

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kBytes = 4;
};
template <>
struct Elem<bf16_t> {
  static constexpr int kBytes = 2;
};

// Geometry of one head-dim row split over the two half-waves.
template <typename T, int D>
struct RowFrag {
  static constexpr int kRowBytes = D * Elem<T>::kBytes;
  static constexpr int kHalfBytes = kRowBytes / 2;
  static constexpr int kNV = kHalfBytes / 16;  // 16-byte vectors per lane per row
  static_assert(kHalfBytes % 16 == 0, "half row must be a whole number of 16-byte vectors");
};

// acc += A * B for one 16-byte vector of each operand (same slice mapping).
template <typename T>
struct Mfma;

template <>
struct Mfma<bf16_t> {
  static __device__ __forceinline__ f32x16 step(u32x4 a, u32x4 b, f32x16 acc) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   acc, 0, 0, 0);
  }
};

template <>
struct Mfma<float> {
  static __device__ __forceinline__ f32x16 step(u32x4 a, u32x4 b, f32x16 acc) {
    f32x4 fa = __builtin_bit_cast(f32x4, a);
    f32x4 fb = __builtin_bit_cast(f32x4, b);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[0], fb[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[1], fb[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[2], fb[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[3], fb[3], acc, 0, 0, 0);
    return acc;
  }
};

__device__ __forceinline__ int acc_row(int i, int half) { return 8 * (i >> 2) + 4 * half + (i & 3); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Value held by lane l ^ 32 (the other half-wave), without a trip through
// LDS: v_permlane32_swap of v with itself gives r[0] = (v[0..31], v[0..31])
// and r[1] = (v[32..63], v[32..63]) over lanes (0..31, 32..63).
__device__ __forceinline__ float shfl_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Order-preserving map of an fp32 bit pattern to uint32 (-0 is folded to +0).
__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Block index remap so that each XCD (the hardware deals blocks round-robin
// over the 8 XCDs) works on one contiguous range of logical blocks; blocks
// that share inputs then share that XCD's L2.
__device__ __forceinline__ uint32_t xcd_contiguous_block(uint32_t b, uint32_t n) {
  constexpr uint32_t kXcd = 8;
  const uint32_t per = n / kXcd, rem = n % kXcd;
  const uint32_t x = b % kXcd, local = b / kXcd;
  return (x < rem) ? x * (per + 1) + local : rem * (per + 1) + (x - rem) * per + local;
}

}  // namespace skv
