// Expert-choice routing: each expert takes its top-C tokens by router
// probability instead of each token taking its top-k experts, so every expert
// processes exactly C rows (matteuscruz "Mixture of Experts", "Load balancing",
// expert choice routing).  Among equal probabilities the lower token index
// goes first.  A token's output is the sum, over the experts that took it in
// expert order, of p[t, e] E_e(x_t) (plus the shared expert).
//
//   ec_select_kernel   one block per expert: radix select of the C-th largest
//                      probability (integer histograms in LDS: order-free),
//                      then one pass in token order writes the expert's rows
//                      (token-ascending), their gates, a selection bitmap and
//                      per-word prefix counts;
//   ec_finish_kernel   one block: offsets (C rows per expert), the GEMM
//                      row-tile list, the shared expert's rows, counts and the
//                      load statistics;
//   combine_ec_kernel  y[t] = sum over experts in order of the rows the bitmap
//                      marks for t, then the shared row, in fp32; no atomics.
#include "kernels.h"
#include "block_ops.h"

namespace moe {

constexpr int kEcKeysLds = 16384;  // tokens whose keys are cached in LDS (64 KB)

// probsT [E, T] fp32 (row e = expert e's probabilities, non-negative, so their
// bit patterns order like the values).  Rows e*Ce .. e*Ce + Ce - 1 receive the
// expert's tokens in ascending order (copied to ec_idx / ec_w when given).
// sel [E, W] and pre [E, W] (W = ceil(T / 32)):
// bit t % 32 of sel[e][t / 32] is set when expert e took token t; pre[e][w] =
// tokens expert e took before token 32 w.
__global__ __launch_bounds__(kMaxExperts) void ec_select_kernel(
    const float* __restrict__ probsT, int64_t T, int Ce, int W, int32_t* __restrict__ row_token,
    float* __restrict__ row_gate, uint32_t* __restrict__ sel, int32_t* __restrict__ pre,
    int32_t* __restrict__ ec_idx, float* __restrict__ ec_w) {
  __shared__ uint32_t keys[kEcKeysLds];
  __shared__ int32_t hist[256];
  __shared__ int32_t wsum[kMaxExperts / 64];
  __shared__ uint32_t s_prefix;
  __shared__ int32_t s_rem;
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const float* pe = probsT + static_cast<int64_t>(e) * T;
  const bool cached = T <= kEcKeysLds;
  if (cached) {
    for (int t = tid; t < T; t += kMaxExperts) keys[t] = __float_as_uint(pe[t]);
    __syncthreads();
  }
  auto key_of = [&](int64_t t) -> uint32_t {
    return cached ? keys[t] : __float_as_uint(pe[t]);
  };

  // The C-th largest key K, most significant byte first: each pass counts the
  // keys that share the bytes fixed so far, per value of the next byte, and
  // keeps the byte value whose bin holds the C-th largest (a block scan over the
  // bins in descending order finds it).  Afterwards every key above K is taken
  // and the first `need_eq` tokens whose key equals K.
  uint32_t K = 0;
  int need_eq = 0;
  const bool all = Ce >= T;
  if (Ce > 0 && !all) {
    uint32_t prefix = 0, mask = 0;
    int rem = Ce;  // rank of the C-th largest among the keys matching prefix
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int b = tid; b < 256; b += kMaxExperts) hist[b] = 0;
      __syncthreads();
      for (int64_t t = tid; t < T; t += kMaxExperts) {
        const uint32_t k = key_of(t);
        if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1);
      }
      __syncthreads();
      // thread i holds bin 255 - i: `above` = keys in higher bins
      const int h = tid < 256 ? hist[255 - tid] : 0;
      int all_bins;
      const int above = block_excl_scan(h, wsum, all_bins);
      if (tid < 256 && above < rem && rem <= above + h) {
        s_prefix = prefix | (static_cast<uint32_t>(255 - tid) << shift);
        s_rem = rem - above;
      }
      __syncthreads();
      prefix = s_prefix;
      rem = s_rem;
      mask |= 255u << shift;
      __syncthreads();
    }
    K = prefix;
    need_eq = rem;
  }

  // One pass in token order, 1024 tokens at a time.  Tokens taken before t =
  // keys above K before t + min(keys equal to K before t, need_eq); both counts
  // come from one scan of (above) | (equal << 16) (at most 1024 each per chunk).
  int carry_gt = 0, carry_eq = 0;
  for (int64_t t0 = 0; t0 < T; t0 += kMaxExperts) {
    const int64_t t = t0 + tid;
    const bool valid = t < T;
    const uint32_t k = valid ? key_of(t) : 0u;
    const bool gt = valid && (all || (Ce > 0 && k > K));
    const bool eq = valid && !all && Ce > 0 && k == K;
    int tot;
    const int packed = block_excl_scan((gt ? 1 : 0) | (eq ? 1 << 16 : 0), wsum, tot);
    const int eq_before = carry_eq + (packed >> 16);
    const bool take = gt || (eq && eq_before < need_eq);
    const int pos = carry_gt + (packed & 0xffff) + min(eq_before, need_eq);
    if (take) {
      const int64_t r = static_cast<int64_t>(e) * Ce + pos;
      row_token[r] = static_cast<int32_t>(t);
      row_gate[r] = __uint_as_float(k);
      if (ec_idx) ec_idx[r] = static_cast<int32_t>(t);
      if (ec_w) ec_w[r] = __uint_as_float(k);
    }
    const uint64_t m = __ballot(take);
    // lanes 0 and 32 start a 32-token word (t0 and the wave's base are multiples of 64)
    if ((lane & 31) == 0 && valid) {
      const int64_t w = static_cast<int64_t>(e) * W + (t >> 5);
      sel[w] = static_cast<uint32_t>(lane ? (m >> 32) : m);
      pre[w] = pos;
    }
    carry_gt += tot & 0xffff;
    carry_eq += tot >> 16;
  }
}

// One block: offsets, counts, the row-tile list, the shared expert's rows and
// the statistics of an expert-choice call.
__global__ __launch_bounds__(kMaxExperts) void ec_finish_kernel(EcArgs a) {
  __shared__ int32_t soff[kMaxExperts + 2];
  __shared__ int32_t wsum[kMaxExperts / 64];
  __shared__ double wsd[kMaxExperts / 64];
  const int tid = threadIdx.x;
  const int E = a.E, Ce = a.Ce;
  const int32_t routed = E * Ce;
  for (int e = tid; e < E; e += kMaxExperts) {
    soff[e] = e * Ce;
    a.offsets[e] = e * Ce;
    if (a.counts) a.counts[e] = Ce;
    if (a.kept) a.kept[e] = Ce;
  }
  if (tid == 0) {
    const int32_t end = routed + (a.shared ? static_cast<int32_t>(a.T) : 0);
    soff[E] = routed;
    soff[E + 1] = end;
    a.offsets[E] = routed;
    a.offsets[E + 1] = end;
  }
  __syncthreads();
  build_tile_list(soff, E + (a.shared ? 1 : 0), a.BM, a.extra, a.tiles, a.ntiles, wsum);
  if (a.shared)
    for (int64_t t = tid; t < a.T; t += kMaxExperts) {
      a.row_token[routed + t] = static_cast<int32_t>(t);
      a.row_gate[routed + t] = 1.0f;
    }
  if (a.mean_prob || a.balance) load_stats(a.stat_part, a.nb, E, a.T, a.mean_prob, a.balance, wsd);
  if (a.cv2) counts_cv2(tid < E ? Ce : 0, E, a.cv2, wsd);
}

// One block per token (and 1024-column slice): the block's threads each test
// one expert's bitmap word for the token (all loads at once), the taking
// experts' rows are compacted into LDS in expert order, then each thread sums
// its 4 columns of those rows in that order (8 row loads in flight), then the
// shared row.
template <typename OT>
__global__ __launch_bounds__(256) void combine_ec_kernel(const float* __restrict__ y_rows,
                                                         const uint32_t* __restrict__ sel,
                                                         const int32_t* __restrict__ pre,
                                                         int64_t T, int d, int E, int W, int Ce,
                                                         int shared, OT* __restrict__ y) {
  __shared__ int32_t rows[kMaxExperts];
  __shared__ int32_t wcnt[4];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t w = t >> 5;
  const uint32_t bit = 1u << (t & 31);
  int n = 0;
  for (int e0 = 0; e0 < E; e0 += 256) {
    const int e = e0 + tid;
    int row = -1;
    if (e < E) {
      const uint32_t m = sel[static_cast<int64_t>(e) * W + w];
      const int32_t p = pre[static_cast<int64_t>(e) * W + w];
      if (m & bit) row = e * Ce + p + __popc(m & (bit - 1u));
    }
    const uint64_t b = __ballot(row >= 0);
    if (lane == 0) wcnt[wave] = __popcll(b);
    __syncthreads();
    int off = n, tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      off += i < wave ? wcnt[i] : 0;
      tot += wcnt[i];
    }
    if (row >= 0) rows[off + __popcll(b & ((uint64_t(1) << lane) - 1))] = row;
    n += tot;
    __syncthreads();
  }
  const int c = (blockIdx.y * 256 + tid) * 4;
  if (c >= d) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i0 = 0; i0 < n; i0 += 8) {
    float4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = i0 + j < n ? *reinterpret_cast<const float4*>(
                              y_rows + static_cast<int64_t>(rows[i0 + j]) * d + c)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (i0 + j < n) {
        acc.x += v[j].x;
        acc.y += v[j].y;
        acc.z += v[j].z;
        acc.w += v[j].w;
      }
    }
  }
  if (shared) {
    const int64_t rs = static_cast<int64_t>(E) * Ce + t;
    const float4 vs = *reinterpret_cast<const float4*>(y_rows + rs * d + c);
    acc.x += vs.x;
    acc.y += vs.y;
    acc.z += vs.z;
    acc.w += vs.w;
  }
  store4<OT>(y + t * d + c, acc);
}

hipError_t launch_expert_choice(const EcArgs& a, const float* probsT, hipStream_t st) {
  if (a.T > 0 && a.E > 0)
    ec_select_kernel<<<static_cast<unsigned>(a.E), kMaxExperts, 0, st>>>(
        probsT, a.T, a.Ce, a.W, a.row_token, a.row_gate, a.sel, a.pre, a.ec_idx, a.ec_w);
  ec_finish_kernel<<<1, kMaxExperts, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_combine_ec(int64_t T, int d, int E, int Ce, int shared, int dtype,
                             const float* y_rows, const uint32_t* sel, const int32_t* pre,
                             void* y, hipStream_t st) {
  if (T > 0) {
    const int W = static_cast<int>(ceil_div(T, 32));
    const dim3 grid(static_cast<unsigned>(T), static_cast<unsigned>(ceil_div(d, 1024)));
    if (dtype == MOE_BF16)
      combine_ec_kernel<bf16><<<grid, 256, 0, st>>>(y_rows, sel, pre, T, d, E, W, Ce, shared,
                                                    static_cast<bf16*>(y));
    else
      combine_ec_kernel<float><<<grid, 256, 0, st>>>(y_rows, sel, pre, T, d, E, W, Ce, shared,
                                                     static_cast<float*>(y));
  }
  return hipGetLastError();
}

}  // namespace moe
