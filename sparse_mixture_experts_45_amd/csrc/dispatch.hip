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
//   2. scan: counts, kept = min(counts, C), offsets = exclusive scan of kept,
//      and for every block the number of earlier pairs per expert;
//   3. one wave per 64-token block ranks each pair among the earlier tokens of
//      the block with the same expert (ballot match on the expert id bits),
//      adds the block base, and scatters kept pairs to their rows.
// Up to kDispatchLdsBases histogram entries, steps 2 and 3 run in one launch
// (dispatch_blocks_kernel: every workgroup reduces the histogram for its own
// block); beyond, as a scan kernel and a scatter kernel.
#include "kernels.h"
#include "block_ops.h"

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

// Scan of the per-block histogram by one block of kMaxExperts threads.  The
// blocks are cut into `chunks` contiguous ranges.  Pass 1: thread (c, e) =
// (tid / E, tid % E) sums expert e over range c (consecutive threads read
// consecutive experts: coalesced, and free of LDS bank conflicts).  The range
// sums go to sh in expert-major order with an odd row stride; one block-wide
// scan in that order gives, for every (expert, range), the pairs of the expert
// in earlier ranges (minus the value at the expert's first range) and the
// expert's total.  Pass 2: thread (c, e) walks its range again and writes
// base[b][e] = pairs of expert e in blocks before b.  kept = min(count, C);
// offsets = exclusive scan of kept, offsets[E] = routed rows, offsets[E + 1] =
// routed + shared rows.  sh: 2 * kMaxExperts ints of LDS.  Integer sums:
// exact in any order.  Ends with a barrier and returns counts[tid] to threads
// tid < E.
__device__ __forceinline__ int scan_hist(const int32_t* __restrict__ hist, int nb, int E,
                                         int64_t T, int capacity, int shared, int32_t* base,
                                         int32_t* __restrict__ counts,
                                         int32_t* __restrict__ kept,
                                         int32_t* __restrict__ offsets, int32_t* sh,
                                         int32_t* wsum) {
  const int tid = threadIdx.x;
  const int chunks = max(1, min(kMaxExperts / E, nb));
  const int len = (nb + chunks - 1) / chunks;
  const int P = chunks + 1;  // odd row stride of the expert-major range sums
  // pass 1: range sums, thread (c, e)
  const int c1 = tid / E, e1 = tid - c1 * E;
  const bool own1 = c1 < chunks;
  const int b0 = c1 * len, b1 = min(nb, b0 + len);
  if (own1) {
    int sum = 0;
#pragma unroll 8
    for (int b = b0; b < b1; ++b) sum += hist[static_cast<int64_t>(b) * E + e1];
    sh[e1 * P + c1] = sum;
  }
  __syncthreads();
  // expert-major scan, thread (e, c)
  const int e2 = tid / chunks, c2 = tid - e2 * chunks;
  const bool own2 = e2 < E;
  int total;
  const int ex = block_excl_scan(own2 ? sh[e2 * P + c2] : 0, wsum, total);
  if (own2) sh[e2 * P + c2] = ex;
  __syncthreads();
  // pass 2: bases, thread (c, e)
  if (own1) {
    int run = sh[e1 * P + c1] - sh[e1 * P];
#pragma unroll 8
    for (int b = b0; b < b1; ++b) {
      const int h = hist[static_cast<int64_t>(b) * E + e1];  // read before base overwrites it
      base[static_cast<int64_t>(b) * E + e1] = run;
      run += h;
    }
  }
  int kp = 0, cnt = 0;
  if (tid < E) {
    const int s1 = tid + 1 < E ? sh[(tid + 1) * P] : total;
    cnt = s1 - sh[tid * P];
    kp = capacity < 0 ? cnt : min(cnt, capacity);
    counts[tid] = cnt;
    kept[tid] = kp;
  }
  int ktot;
  const int kx = block_excl_scan(kp, wsum, ktot);
  if (tid < E) offsets[tid] = kx;
  if (tid == 0) {
    const int end = ktot + (shared ? static_cast<int32_t>(T) : 0);
    offsets[E] = ktot;
    offsets[E + 1] = end;
  }
  __syncthreads();
  return cnt;  // counts[tid] for tid < E
}

__global__ __launch_bounds__(1024) void dispatch_scan_kernel(
    const int32_t* __restrict__ hist, int nb, int E, int64_t T, int capacity, int shared,
    int32_t* __restrict__ base, int32_t* __restrict__ counts, int32_t* __restrict__ kept,
    int32_t* __restrict__ offsets, float* __restrict__ cv2) {
  __shared__ int32_t sh[2 * kMaxExperts];
  __shared__ int32_t wsum[kMaxExperts / 64];
  __shared__ double wsd[kMaxExperts / 64];
  const int cnt = scan_hist(hist, nb, E, T, capacity, shared, base, counts, kept, offsets, sh,
                            wsum);
  if (cv2) counts_cv2(cnt, E, cv2, wsd);
}

// Expert ids (and, with topk_w set, gates) of the pairs of 64-token block b,
// lane = token; -1 / 0 past T or past k.
template <int KM>
__device__ __forceinline__ void load_block(int64_t b, const int32_t* __restrict__ topk_idx,
                                           const float* __restrict__ topk_w, int64_t T, int k,
                                           int (&mine)[KM], float (&wsel)[KM]) {
  const int64_t t = b * kGateTokens + (threadIdx.x & 63);
  const bool valid = t < T;
#pragma unroll
  for (int i = 0; i < KM; ++i) {
    mine[i] = (valid && i < k) ? topk_idx[t * k + i] : -1;
    wsel[i] = (topk_w && valid && i < k) ? topk_w[t * k + i] : 0.f;
  }
}

// Lanes below this one (in `live`) whose expert id v equals e: the id bits are
// compared through nbits ballots, one per bit.
__device__ __forceinline__ int lower_matches(int v, int e, int nbits, uint64_t live) {
  uint64_t m = live;
#pragma unroll
  for (int q = 0; q < 10; ++q) {
    if (q < nbits) {
      const uint64_t bq = __ballot((v >> q) & 1);
      m &= ((e >> q) & 1) ? bq : ~bq;
    }
  }
  return __popcll(m);
}

// Row of pair (t, i) of expert e with `rank` earlier pairs of e in its 64-token
// block, or -1 when e is out of range or the pair falls beyond the capacity;
// writes the row's token, slot and (with row_gate) gate, and inv.
__device__ __forceinline__ void place_pair(int64_t t, int i, int k, int e, int rank, int E,
                                           const int32_t* base, const int32_t* kept,
                                           const int32_t* offsets, float gate,
                                           int32_t* __restrict__ row_token,
                                           int32_t* __restrict__ row_slot,
                                           int32_t* __restrict__ inv,
                                           float* __restrict__ row_gate) {
  const bool ok = static_cast<unsigned>(e) < static_cast<unsigned>(E);
  const int gr = ok ? base[e] + rank : 0;
  if (ok && gr < kept[e]) {
    const int row = offsets[e] + gr;
    row_token[row] = static_cast<int32_t>(t);
    row_slot[row] = i;
    inv[t * k + i] = row;
    if (row_gate) row_gate[row] = gate;
  } else {
    inv[t * k + i] = -1;
  }
}

__device__ __forceinline__ void place_shared(int64_t t, int E, const int32_t* offsets,
                                             int32_t* __restrict__ row_token,
                                             int32_t* __restrict__ row_slot,
                                             float* __restrict__ row_gate) {
  const int row = offsets[E] + static_cast<int>(t);
  row_token[row] = static_cast<int32_t>(t);
  row_slot[row] = -1;
  if (row_gate) row_gate[row] = 1.0f;
}

// Ranks and scatters the pairs of 64-token block b; one wave, lane = token.
// A pair's rank is the number of lower lanes that picked the same expert in any
// slot (a token never picks an expert twice), so pairs of an expert land
// token-ascending.  `base` points at the block's per-expert count of earlier
// pairs.  With row_gate set, also writes each kept row's gate (its pair's
// topk_w; 1 for the shared expert's row).
//
// Up to 4 slots: ids and gates preloaded by load_block, all slots unrolled.
template <int KM>
__device__ __forceinline__ void scatter_block_few(int64_t b, const int (&mine)[KM],
                                                  const float (&wsel)[KM], int64_t T, int k,
                                                  int E, int nbits, const int32_t* base,
                                                  const int32_t* kept, const int32_t* offsets,
                                                  int shared, int32_t* __restrict__ row_token,
                                                  int32_t* __restrict__ row_slot,
                                                  int32_t* __restrict__ inv,
                                                  float* __restrict__ row_gate) {
  static_assert(KM <= 4, "few slots only");
  const int lane = threadIdx.x & 63;
  const int64_t t = b * kGateTokens + lane;
  const bool valid = t < T;
  const uint64_t live = __ballot(valid) & ((lane == 0) ? 0ull : (~0ull >> (64 - lane)));
  int rank[KM];
#pragma unroll
  for (int i = 0; i < KM; ++i) rank[i] = 0;
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    if (j < k) {
      const int v = valid ? mine[j] : 0;
#pragma unroll
      for (int i = 0; i < KM; ++i)
        if (i < k) rank[i] += lower_matches(v, mine[i], nbits, live);
    }
  }
  if (valid) {
#pragma unroll
    for (int i = 0; i < KM; ++i)
      if (i < k)
        place_pair(t, i, k, mine[i], rank[i], E, base, kept, offsets, wsel[i], row_token,
                   row_slot, inv, row_gate);
    if (shared) place_shared(t, E, offsets, row_token, row_slot, row_gate);
  }
}

// Slot i of every token of 64-token block b (one wave, lane = token): ranked
// against all k slots of the lower lanes, then placed.  Slot j of the block's
// token `lane` is read from ids[lane * ids_stride + j] and its gate from
// gates[lane * ids_stride + j] (gates only needed with row_gate): LDS copies of
// the block's ids and gates when they fit, else topk_idx / topk_w themselves.
__device__ __forceinline__ void scatter_slot(int64_t b, int i, const int32_t* ids,
                                             int ids_stride, const float* gates, int64_t T,
                                             int k, int E, int nbits, const int32_t* base,
                                             const int32_t* kept, const int32_t* offsets,
                                             int32_t* __restrict__ row_token,
                                             int32_t* __restrict__ row_slot,
                                             int32_t* __restrict__ inv,
                                             float* __restrict__ row_gate) {
  const int lane = threadIdx.x & 63;
  const int64_t t = b * kGateTokens + lane;
  const bool valid = t < T;
  const uint64_t live = __ballot(valid) & ((lane == 0) ? 0ull : (~0ull >> (64 - lane)));
  const int32_t* my = ids + lane * ids_stride;
  const int ei = valid ? my[i] : 0;
  int rank = 0;
  for (int j = 0; j < k; ++j) rank += lower_matches(valid ? my[j] : 0, ei, nbits, live);
  if (valid)
    place_pair(t, i, k, ei, rank, E, base, kept, offsets,
               gates ? gates[lane * ids_stride + i] : 0.f, row_token, row_slot, inv, row_gate);
}

// Any k on one wave: slots rolled, each pair placed as soon as its rank is known
// (keeps the registers few for large k).
__device__ __forceinline__ void scatter_block_any(int64_t b, const int32_t* ids, int ids_stride,
                                                  const float* gates, int64_t T,
                                                  int k, int E, int nbits, const int32_t* base,
                                                  const int32_t* kept, const int32_t* offsets,
                                                  int shared, int32_t* __restrict__ row_token,
                                                  int32_t* __restrict__ row_slot,
                                                  int32_t* __restrict__ inv,
                                                  float* __restrict__ row_gate) {
  for (int i = 0; i < k; ++i)
    scatter_slot(b, i, ids, ids_stride, gates, T, k, E, nbits, base, kept, offsets, row_token,
                 row_slot, inv, row_gate);
  const int64_t t = b * kGateTokens + (threadIdx.x & 63);
  if (t < T && shared) place_shared(t, E, offsets, row_token, row_slot, row_gate);
}

// Copy the ids (and, with wdst set, the gates) of 64-token block b (64 x k,
// k <= kIdsK) into a wave's LDS area, row stride kIdsK + 1 (odd: the per-slot
// reads of 64 lanes spread over banks).
constexpr int kIdsK = 8;
__device__ __forceinline__ void stage_ids(int64_t b, const int32_t* __restrict__ topk_idx,
                                          const float* __restrict__ topk_w, int64_t T, int k,
                                          int32_t* dst, float* wdst) {
  const int lane = threadIdx.x & 63;
  const int64_t f0 = b * kGateTokens * k;
  const int64_t fend = T * k;
  // all loads first (one latency), then the LDS stores
  int iv[kIdsK];
  float wv[kIdsK];
#pragma unroll
  for (int c = 0; c < kIdsK; ++c) {
    const int f = lane + c * 64;
    const bool in = f < kGateTokens * k && f0 + f < fend;
    iv[c] = in ? topk_idx[f0 + f] : 0;
    wv[c] = (in && wdst) ? topk_w[f0 + f] : 0.f;
  }
#pragma unroll
  for (int c = 0; c < kIdsK; ++c) {
    const int f = lane + c * 64;
    if (f < kGateTokens * k) {
      const int r = f / k, j = f - r * k;
      dst[r * (kIdsK + 1) + j] = iv[c];
      if (wdst) wdst[r * (kIdsK + 1) + j] = wv[c];
    }
  }
}

// One 64-token block per workgroup: one wave, or with more than 4 slots and at
// most kIdsK of them, one wave per slot (ids staged in LDS by wave 0).
template <int KM>
__global__ __launch_bounds__(KM <= 4 ? 64 : 64 * kIdsK) void dispatch_scatter_kernel(
    const int32_t* __restrict__ topk_idx, int64_t T, int k, int E, int nbits,
    const int32_t* __restrict__ base, const int32_t* __restrict__ kept,
    const int32_t* __restrict__ offsets, int shared, int32_t* __restrict__ row_token,
    int32_t* __restrict__ row_slot, int32_t* __restrict__ inv) {
  const int64_t b = blockIdx.x;
  if constexpr (KM <= 4) {
    int mine[KM];
    float wsel[KM];
    load_block<KM>(b, topk_idx, nullptr, T, k, mine, wsel);
    scatter_block_few<KM>(b, mine, wsel, T, k, E, nbits, base + b * E, kept, offsets, shared,
                          row_token, row_slot, inv, nullptr);
  } else {
    __shared__ int32_t sids[kGateTokens * (kIdsK + 1)];
    if (k <= kIdsK) {
      const int wave = threadIdx.x >> 6;
      if (wave == 0) stage_ids(b, topk_idx, nullptr, T, k, sids, nullptr);
      __syncthreads();
      if (wave < k)
        scatter_slot(b, wave, sids, kIdsK + 1, nullptr, T, k, E, nbits, base + b * E, kept,
                     offsets, row_token, row_slot, inv, nullptr);
      const int64_t t = b * kGateTokens + (threadIdx.x & 63);
      if (wave == 0 && shared && t < T) place_shared(t, E, offsets, row_token, row_slot, nullptr);
    } else {
      scatter_block_any(b, topk_idx + b * kGateTokens * k, k, nullptr, T, k, E, nbits,
                        base + b * E, kept, offsets, shared, row_token, row_slot, inv, nullptr);
    }
  }
}

// The whole dispatch of a batch whose per-block histogram has at most
// kDispatchLdsBases entries: one workgroup of kMaxExperts threads per 64-token
// block (one for an empty batch).  Each workgroup reduces the gate's per-block
// histogram to the expert totals and to its block's count of earlier pairs per
// expert (thread (c, e) sums expert e over a range c of blocks), takes kept =
// min(count, C) and the offsets, and its first wave ranks and scatters the
// block's pairs and writes every kept row's gate.  Workgroup 0 also writes
// counts, kept and offsets, the load statistics (mean router probability per
// expert and its unbiased variance, fp64; cv^2 of the counts) and the GEMM
// row-tile list.  Every workgroup derives the same integers from the same
// histogram, so none waits for another, and the scattered stores spread over
// as many compute units as there are blocks.  Same outputs as the multi-kernel
// path.
template <int KM>
__global__ __launch_bounds__(1024) void dispatch_blocks_kernel(DispatchArgs a) {
  __shared__ int32_t part[2][kMaxExperts];  // (expert, range) sums: earlier blocks, all blocks
  __shared__ int32_t sbase[kMaxExperts];
  __shared__ int32_t skept[kMaxExperts];
  __shared__ int32_t soff[kMaxExperts + 2];
  __shared__ int32_t wsum[kMaxExperts / 64];
  __shared__ double wsd[kMaxExperts / 64];
  __shared__ int32_t sids[KM <= 4 ? 1 : kGateTokens * (kIdsK + 1)];
  __shared__ float sgts[KM <= 4 ? 1 : kGateTokens * (kIdsK + 1)];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int E = a.E, nb = a.nb, b = blockIdx.x;
  const bool scatter = wave == 0 && b < nb;
  // the block's ids and gates do not depend on the reduction: loaded first
  constexpr int KP = KM <= 4 ? KM : 1;
  int mine[KP];
  float wsel[KP];
  if constexpr (KM <= 4) {
    if (scatter) load_block<KP>(b, a.topk_idx, a.topk_w, a.T, a.k, mine, wsel);
  }
  if (b == 0 && (a.mean_prob || a.balance))
    load_stats(a.stat_part, nb, E, a.T, a.mean_prob, a.balance, wsd);

  const int chunks = max(1, min(kMaxExperts / E, nb));
  const int len = (nb + chunks - 1) / chunks;
  const int c1 = tid / E, e1 = tid - c1 * E;
  if (c1 < chunks) {
    int before = 0, all = 0;
    const int b0 = c1 * len, b1 = min(nb, b0 + len);
#pragma unroll 8
    for (int bb = b0; bb < b1; ++bb) {
      const int h = a.hist[static_cast<int64_t>(bb) * E + e1];
      all += h;
      before += bb < b ? h : 0;
    }
    part[0][e1 * chunks + c1] = before;
    part[1][e1 * chunks + c1] = all;
  }
  __syncthreads();
  int cnt = 0, kp = 0;
  if (tid < E) {
    int before = 0;
    for (int c = 0; c < chunks; ++c) {
      before += part[0][tid * chunks + c];
      cnt += part[1][tid * chunks + c];
    }
    kp = a.capacity < 0 ? cnt : min(cnt, a.capacity);
    sbase[tid] = before;
    skept[tid] = kp;
  }
  int ktot;
  const int kx = block_excl_scan(kp, wsum, ktot);
  if (tid < E) soff[tid] = kx;
  if (tid == 0) {
    soff[E] = ktot;
    soff[E + 1] = ktot + (a.shared ? static_cast<int32_t>(a.T) : 0);
  }
  __syncthreads();
  if (b == 0) {
    if (tid < E) {
      a.counts[tid] = cnt;
      a.kept[tid] = kp;
      a.offsets[tid] = kx;
    }
    if (tid == 0) {
      a.offsets[E] = soff[E];
      a.offsets[E + 1] = soff[E + 1];
    }
    if (a.cv2) counts_cv2(cnt, E, a.cv2, wsd);
    build_tile_list(soff, E + (a.shared ? 1 : 0), a.BM, a.extra, a.tiles, a.ntiles, wsum);
  }
  if (b >= nb) return;
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  if constexpr (KM > 4) {
    if (a.k <= kIdsK) {
      // the block's ids and gates to LDS, then wave i ranks and places slot i
      if (wave == 0) stage_ids(b, a.topk_idx, a.topk_w, a.T, a.k, sids, sgts);
      __syncthreads();
      if (wave < a.k)
        scatter_slot(b, wave, sids, kIdsK + 1, sgts, a.T, a.k, E, nbits, sbase, skept, soff,
                     a.row_token, a.row_slot, a.inv, a.row_gate);
      if (wave == 0 && a.shared) {
        const int64_t t = static_cast<int64_t>(b) * kGateTokens + (tid & 63);
        if (t < a.T) place_shared(t, E, soff, a.row_token, a.row_slot, a.row_gate);
      }
      return;
    }
  }
  if (!scatter) return;
  if constexpr (KM <= 4) {
    scatter_block_few<KP>(b, mine, wsel, a.T, a.k, E, nbits, sbase, skept, soff, a.shared,
                          a.row_token, a.row_slot, a.inv, a.row_gate);
  } else {
    const int64_t f0 = static_cast<int64_t>(b) * kGateTokens * a.k;
    scatter_block_any(b, a.topk_idx + f0, a.k, a.topk_w + f0, a.T, a.k, E, nbits, sbase, skept,
                      soff, a.shared, a.row_token, a.row_slot, a.inv, a.row_gate);
  }
}

hipError_t launch_dispatch_blocks(const DispatchArgs& a, hipStream_t st) {
  const unsigned grid = static_cast<unsigned>(a.nb > 0 ? a.nb : 1);
#define MOE_BLOCKS(KM) dispatch_blocks_kernel<KM><<<grid, kMaxExperts, 0, st>>>(a)
  if (a.k <= 1) MOE_BLOCKS(1);
  else if (a.k <= 2) MOE_BLOCKS(2);
  else if (a.k <= 4) MOE_BLOCKS(4);
  else MOE_BLOCKS(kMaxTopK);  // slots rolled
#undef MOE_BLOCKS
  return hipGetLastError();
}

hipError_t launch_dispatch(int64_t T, int E, int k, int capacity, int shared, int nb,
                           const int32_t* topk_idx, bool need_hist, int32_t* hist, int32_t* base,
                           int32_t* counts, int32_t* kept, int32_t* offsets, int32_t* row_token,
                           int32_t* row_slot, int32_t* inv, float* cv2, hipStream_t st) {
  if (need_hist && nb > 0) dispatch_hist_kernel<<<nb, 256, 0, st>>>(topk_idx, T, k, E, hist);
  dispatch_scan_kernel<<<1, kMaxExperts, 0, st>>>(hist, nb, E, T, capacity, shared, base, counts,
                                                  kept, offsets, cv2);
  if (nb > 0) {
    int nbits = 1;
    while ((1 << nbits) < E) ++nbits;
#define MOE_SCAT(KM)                                                                 \
  dispatch_scatter_kernel<KM><<<nb, KM > 4 && k <= kIdsK ? 64 * k : 64, 0, st>>>(     \
      topk_idx, T, k, E, nbits, base, kept, offsets, shared, row_token, row_slot, inv)
    if (k <= 1) MOE_SCAT(1);
    else if (k <= 2) MOE_SCAT(2);
    else if (k <= 4) MOE_SCAT(4);
    else MOE_SCAT(kMaxTopK);  // slots rolled
#undef MOE_SCAT
  }
  return hipGetLastError();
}

}  // namespace moe
