// MFMA operand types and the two matrix instructions the GEMMs use (gfx950).
#pragma once
#include "common.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename T>
struct Mfma;

// v_mfma_f32_32x32x16_bf16: lane l supplies row (l % 32), k = (l / 32) * 8 + 0..7
template <>
struct Mfma<bf16> {
  static constexpr int kStep = 16;
  static constexpr int kVec = 8;
  typedef bf16x8_t frag;
  static __device__ __forceinline__ frag load(const bf16* p) {
    return *reinterpret_cast<const bf16x8_t*>(p);
  }
  static __device__ __forceinline__ f32x16 op(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

// v_mfma_f32_32x32x2f32: lane l supplies row (l % 32), k = l / 32
template <>
struct Mfma<float> {
  static constexpr int kStep = 2;
  static constexpr int kVec = 1;
  typedef float frag;
  static __device__ __forceinline__ frag load(const float* p) { return *p; }
  static __device__ __forceinline__ f32x16 op(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

}  // namespace moe
