// Combine: y[t] = sum over kept slots i (ascending) of y_rows[inv[t, i]], then
// the shared expert's row, in fp32 and in that fixed order; no atomics, so the
// result is reproducible bit for bit.
//
// Pages: roadtointelligence "Mixture of Experts", output equation
// y = sum_i G(x)_i E_i(x); botmartz "Expert Routing" (outputs start at
// zeros_like(x) and accumulate prob * expert(x) slot by slot).
#include "kernels.h"

namespace moe {

// One thread per 4 columns of one token; the grid is (T, ceil(d / 1024)) so a
// wide row is spread over several blocks.  The token's row indices are uniform
// over the block; all k (+1) row loads are issued before the additions, which
// then run in slot order.  KM >= k slots are unrolled.
template <typename OT, int KM>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_rows,
                                                      const int32_t* __restrict__ inv,
                                                      const int32_t* __restrict__ offsets,
                                                      int64_t T, int d, int E, int k, int shared,
                                                      OT* __restrict__ y) {
  const int64_t t = blockIdx.x;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (c >= d) return;
  int rows[KM];
  float4 v[KM];
#pragma unroll
  for (int i = 0; i < KM; ++i) {
    rows[i] = i < k ? inv[t * k + i] : -1;
    v[i] = rows[i] >= 0
               ? *reinterpret_cast<const float4*>(y_rows + static_cast<int64_t>(rows[i]) * d + c)
               : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int rs = shared ? offsets[E] + static_cast<int32_t>(t) : -1;
  const float4 vs = rs >= 0
                        ? *reinterpret_cast<const float4*>(y_rows + static_cast<int64_t>(rs) * d + c)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < KM; ++i) {
    if (rows[i] >= 0) {
      acc.x += v[i].x;
      acc.y += v[i].y;
      acc.z += v[i].z;
      acc.w += v[i].w;
    }
  }
  if (rs >= 0) {
    acc.x += vs.x;
    acc.y += vs.y;
    acc.z += vs.z;
    acc.w += vs.w;
  }
  store4<OT>(y + t * d + c, acc);
}

template <typename OT>
static void run_combine(int64_t T, int d, int E, int k, int shared, const float* y_rows,
                        const int32_t* inv, const int32_t* offsets, OT* y, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(T), static_cast<unsigned>(ceil_div(d, 1024)));
#define MOE_COMB(KM) \
  combine_kernel<OT, KM><<<grid, 256, 0, st>>>(y_rows, inv, offsets, T, d, E, k, shared, y)
  if (k <= 1) MOE_COMB(1);
  else if (k <= 2) MOE_COMB(2);
  else if (k <= 4) MOE_COMB(4);
  else if (k <= 8) MOE_COMB(8);
  else if (k <= 16) MOE_COMB(16);
  else MOE_COMB(32);
#undef MOE_COMB
}

hipError_t launch_combine(int64_t T, int d, int E, int k, int shared, int dtype,
                          const float* y_rows, const int32_t* inv, const int32_t* offsets,
                          void* y, hipStream_t st) {
  if (T > 0) {
    if (dtype == MOE_BF16)
      run_combine<bf16>(T, d, E, k, shared, y_rows, inv, offsets, static_cast<bf16*>(y), st);
    else
      run_combine<float>(T, d, E, k, shared, y_rows, inv, offsets, static_cast<float*>(y), st);
  }
  return hipGetLastError();
}

}  // namespace moe
