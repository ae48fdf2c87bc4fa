// Internal helpers shared by the HIP kernels of the MoE layer (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;
constexpr size_t kAlign = 256;

// Tokens per gate block; also the granularity of the per-block expert
// histograms and probability partial sums that dispatch and statistics consume.
constexpr int kGateTokens = 64;

struct bf16 {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even; NaN stays NaN (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ float to_f32<bf16>(bf16 v) {
  return bf16_to_f32(v.bits);
}

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float v) {
  return bf16{f32_to_bf16(v)};
}

// Four fp32 values to four consecutive outputs (bf16: rounded to nearest even).
template <typename T>
__device__ __forceinline__ void store4(T* p, float4 v);
template <>
__device__ __forceinline__ void store4<float>(float* p, float4 v) {
  *reinterpret_cast<float4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, float4 v) {
  uint2 u;
  u.x = static_cast<uint32_t>(f32_to_bf16(v.x)) | (static_cast<uint32_t>(f32_to_bf16(v.y)) << 16);
  u.y = static_cast<uint32_t>(f32_to_bf16(v.z)) | (static_cast<uint32_t>(f32_to_bf16(v.w)) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}

__host__ __device__ constexpr inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ constexpr inline size_t align_up(size_t a, size_t b) { return (a + b - 1) / b * b; }

// One row tile of the grouped GEMM: group (expert, or E for the shared expert),
// first row, number of rows, and the index of the group's first row tile and
// the group's number of row tiles.
struct RowTile {
  int32_t group, row0, rows, first, count, pad0, pad1, pad2;
};

}  // namespace moe
