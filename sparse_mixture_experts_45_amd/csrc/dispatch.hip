// Dispatch: group the (token, slot) pairs by expert, token-ascending inside an
// expert, and drop the pairs beyond an expert's capacity in token order.
//
// Pages: botmartz "Expert Routing" (tokens gathered per expert with a mask);
// matteuscruz "Load balancing" (expert capacity buffer, overflow dropped) and
// "Distributed training and inference" (grouping tokens by expert);
// roadtointelligence "Keeping the experts busy" (tokens beyond capacity skip
// the layer).
//
// Three steps, all integer and order-free or fixed-order, so the grouping is
// bit-exact and reproducible:
//   1. per 64-token block, count pairs per expert (LDS integer atomics:
//      counts do not depend on order) -- or take the counts the gate kernel
//      already produced;
//   2. one block scans: counts, kept = min(counts, C), offsets = exclusive scan
//      of kept, and for every block the number of earlier pairs per expert;
//   3. one wave per 64-token block ranks each pair among the earlier tokens of
//      the block with the same expert (ballot match on the expert id bits),
//      adds the block base, and scatters kept pairs to their rows.
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void dispatch_hist_kernel(const int32_t* __restrict__ topk_idx,
                                                            int64_t T, int k, int E,
                                                            int32_t* __restrict__ hist) {
  __shared__ int32_t h[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int64_t b = blockIdx.x;
  const int64_t f0 = b * kGateTokens * k;
  const int64_t f1 = min(T, (b + 1) * kGateTokens) * k;
  for (int64_t f = f0 + threadIdx.x; f < f1; f += 256) {
    const int e = topk_idx[f];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) hist[b * E + e] = h[e];
}

// One block.  Thread (e, c) owns expert e and the c-th contiguous range of the
// per-block counts; ranges are summed, scanned across c, then re-walked to
// write each block's base.  Integer sums: exact in any order.
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(
    const int32_t* __restrict__ hist, int nb, int E, int64_t T, int capacity, int shared,
    int32_t* __restrict__ base, int32_t* __restrict__ counts, int32_t* __restrict__ kept,
    int32_t* __restrict__ offsets) {
  __shared__ int32_t part[kMaxExperts];
  __shared__ int32_t sc[2][kMaxExperts];
  const int tid = threadIdx.x;
  const int chunks = kMaxExperts / E;  // >= 1
  const int e = tid % E, c = tid / E;
  const int len = (nb + chunks - 1) / chunks;
  const int b0 = c * len, b1 = min(nb, b0 + len);
  int sum = 0;
  if (c < chunks)
    for (int b = b0; b < b1; ++b) sum += hist[static_cast<int64_t>(b) * E + e];
  if (c < chunks) part[tid] = sum;
  __syncthreads();
  int kp = 0;
  if (tid < E) {
    int run = 0;
    for (int cc = 0; cc < chunks; ++cc) {
      const int v = part[cc * E + tid];
      part[cc * E + tid] = run;  // exclusive prefix over ranges
      run += v;
    }
    kp = capacity < 0 ? run : min(run, capacity);
    counts[tid] = run;
    kept[tid] = kp;
  }
  __syncthreads();
  if (c < chunks) {
    int run = part[tid];
    for (int b = b0; b < b1; ++b) {
      base[static_cast<int64_t>(b) * E + e] = run;
      run += hist[static_cast<int64_t>(b) * E + e];
    }
  }
  // inclusive Hillis-Steele scan of kept over the experts
  int src = 0;
  sc[0][tid] = kp;
  __syncthreads();
  for (int o = 1; o < kMaxExperts; o <<= 1) {
    const int v = sc[src][tid] + (tid >= o ? sc[src][tid - o] : 0);
    sc[src ^ 1][tid] = v;
    src ^= 1;
    __syncthreads();
  }
  if (tid < E) offsets[tid] = sc[src][tid] - kp;
  if (tid == 0) {
    const int total = sc[src][E - 1];
    offsets[E] = total;
    offsets[E + 1] = total + (shared ? static_cast<int32_t>(T) : 0);
  }
}

template <int KM>
__global__ __launch_bounds__(64) void dispatch_scatter_kernel(
    const int32_t* __restrict__ topk_idx, int64_t T, int k, int E, int nbits,
    const int32_t* __restrict__ base, const int32_t* __restrict__ kept,
    const int32_t* __restrict__ offsets, int shared, int32_t* __restrict__ row_token,
    int32_t* __restrict__ row_slot, int32_t* __restrict__ inv) {
  const int lane = threadIdx.x;
  const int64_t b = blockIdx.x;
  const int64_t t = b * kGateTokens + lane;
  const bool valid = t < T;
  const uint64_t vmask = __ballot(valid);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  int mine[KM];
  int rank[KM];
#pragma unroll
  for (int i = 0; i < KM; ++i) {
    mine[i] = (valid && i < k) ? topk_idx[t * k + i] : -1;
    rank[i] = 0;
  }
  // rank[i] = number of lower lanes that picked expert mine[i] in any slot
  for (int j = 0; j < k; ++j) {
    const int v = valid ? topk_idx[t * k + j] : 0;
    uint64_t bits[10];
#pragma unroll
    for (int q = 0; q < 10; ++q) bits[q] = (q < nbits) ? __ballot((v >> q) & 1) : 0ull;
#pragma unroll
    for (int i = 0; i < KM; ++i) {
      if (i < k) {
        uint64_t m = vmask & below;
#pragma unroll
        for (int q = 0; q < 10; ++q)
          if (q < nbits) m &= ((mine[i] >> q) & 1) ? bits[q] : ~bits[q];
        rank[i] += __popcll(m);
      }
    }
  }
  if (valid) {
#pragma unroll
    for (int i = 0; i < KM; ++i) {
      if (i < k) {
        const int e = mine[i];
        const bool ok = static_cast<unsigned>(e) < static_cast<unsigned>(E);
        const int gr = ok ? base[b * E + e] + rank[i] : 0;
        if (ok && gr < kept[e]) {
          const int row = offsets[e] + gr;
          row_token[row] = static_cast<int32_t>(t);
          row_slot[row] = i;
          inv[t * k + i] = row;
        } else {
          inv[t * k + i] = -1;
        }
      }
    }
    if (shared) {
      const int row = offsets[E] + static_cast<int>(t);
      row_token[row] = static_cast<int32_t>(t);
      row_slot[row] = -1;
    }
  }
}

hipError_t launch_dispatch(int64_t T, int E, int k, int capacity, int shared, int nb,
                           const int32_t* topk_idx, bool need_hist, int32_t* hist, int32_t* base,
                           int32_t* counts, int32_t* kept, int32_t* offsets, int32_t* row_token,
                           int32_t* row_slot, int32_t* inv, hipStream_t st) {
  if (need_hist && nb > 0) dispatch_hist_kernel<<<nb, 256, 0, st>>>(topk_idx, T, k, E, hist);
  dispatch_scan_kernel<<<1, kMaxExperts, 0, st>>>(hist, nb, E, T, capacity, shared, base, counts,
                                                  kept, offsets);
  if (nb > 0) {
    int nbits = 1;
    while ((1 << nbits) < E) ++nbits;
#define MOE_SCAT(KM)                                                                          \
  dispatch_scatter_kernel<KM><<<nb, 64, 0, st>>>(topk_idx, T, k, E, nbits, base, kept, offsets, \
                                                 shared, row_token, row_slot, inv)
    if (k <= 1) MOE_SCAT(1);
    else if (k <= 2) MOE_SCAT(2);
    else if (k <= 4) MOE_SCAT(4);
    else if (k <= 8) MOE_SCAT(8);
    else if (k <= 16) MOE_SCAT(16);
    else MOE_SCAT(32);
#undef MOE_SCAT
  }
  return hipGetLastError();
}

}  // namespace moe
