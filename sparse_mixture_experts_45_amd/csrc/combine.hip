// Combine: y[t] = sum over kept slots i (ascending) of y_rows[inv[t, i]], then
// the shared expert's row, in fp32 and in that fixed order; no atomics, so the
// result is reproducible bit for bit.
//
// Pages: roadtointelligence "Mixture of Experts", output equation
// y = sum_i G(x)_i E_i(x); botmartz "Expert Routing" (outputs start at
// zeros_like(x) and accumulate prob * expert(x) slot by slot).
#include "kernels.h"

namespace moe {

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

template <typename OT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_rows,
                                                      const int32_t* __restrict__ inv,
                                                      const int32_t* __restrict__ offsets,
                                                      int64_t T, int d, int E, int k, int shared,
                                                      OT* __restrict__ y) {
  __shared__ int32_t rows_s[kMaxTopK + 1];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < k) rows_s[threadIdx.x] = inv[t * k + threadIdx.x];
  if (threadIdx.x == 0) rows_s[kMaxTopK] = shared ? offsets[E] + static_cast<int32_t>(t) : -1;
  __syncthreads();
  for (int c = threadIdx.x * 4; c < d; c += 256 * 4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i = 0; i < k; ++i) {
      const int r = rows_s[i];
      if (r >= 0) {
        const float4 v = *reinterpret_cast<const float4*>(y_rows + static_cast<int64_t>(r) * d + c);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
      }
    }
    const int rs = rows_s[kMaxTopK];
    if (rs >= 0) {
      const float4 v = *reinterpret_cast<const float4*>(y_rows + static_cast<int64_t>(rs) * d + c);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    store4<OT>(y + t * d + c, acc);
  }
}

hipError_t launch_combine(int64_t T, int d, int E, int k, int shared, int dtype,
                          const float* y_rows, const int32_t* inv, const int32_t* offsets,
                          void* y, hipStream_t st) {
  if (T > 0) {
    if (dtype == MOE_BF16)
      combine_kernel<bf16><<<static_cast<unsigned>(T), 256, 0, st>>>(y_rows, inv, offsets, T, d, E,
                                                                     k, shared, static_cast<bf16*>(y));
    else
      combine_kernel<float><<<static_cast<unsigned>(T), 256, 0, st>>>(y_rows, inv, offsets, T, d, E,
                                                                      k, shared, static_cast<float*>(y));
  }
  return hipGetLastError();
}

}  // namespace moe
