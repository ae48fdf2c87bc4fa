// Block-wide helpers for blocks of kMaxExperts threads: integer scans of the
// dispatch, the row-tile list of the grouped GEMM, and the load statistics.
#pragma once
#include "kernels.h"

namespace moe {

// Exclusive prefix sum of v over the block's threads in thread order (wave
// shuffle scans, then the 16 wave totals); `total` gets the block sum.  wsum:
// 16 ints of LDS.  Integer sums, exact.
__device__ inline int block_excl_scan(int v, int32_t* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kMaxExperts / 64; ++w) {
    const int s = wsum[w];
    pre += w < wave ? s : 0;
    tot += s;
  }
  total = tot;
  __syncthreads();
  return pre + x - v;
}

// Group g (expert g, or the shared expert as group E) owns rows
// off[g] .. off[g+1] and is cut into ceil(rows / BM) tiles of at most BM rows;
// with extra > 0, a group whose last tile would hold at most `extra` rows
// merges them into its previous tile instead, which then holds more than BM
// rows (a heavy tile).  The heavy tiles come first, one per such group in
// group order, then every other tile, group by group and row-ascending;
// `first` and `count` of a tile give the group's run of tiles in that second
// part (a heavy tile: its own index, 1).  `off` may sit in global memory or
// LDS.  ntiles[0] gets the tile count, ntiles[1 .. kSplitSlots] (the grouped
// GEMM's split counters) zero, ntiles[kSplitSlots + 1] the heavy tile count.
__device__ inline void build_tile_list(const int32_t* off, int G, int BM, int extra,
                                       RowTile* __restrict__ tiles, int32_t* __restrict__ ntiles,
                                       int32_t* wsum) {
  const int g = threadIdx.x;
  int rows = 0, m = 0, h = 0;
  if (g < G) {
    rows = off[g + 1] - off[g];
    m = (rows + BM - 1) / BM;
    if (extra > 0 && m >= 2 && rows - (m - 1) * BM <= extra) {
      --m;
      h = 1;  // the last of the m tiles holds rows - (m - 1) BM > BM rows
    }
  }
  int heavy, normal;
  const int hstart = block_excl_scan(h, wsum, heavy);
  const int start = heavy + block_excl_scan(m - h, wsum, normal);
  if (g < G) {
    const int r0 = off[g];
    for (int j = 0; j < m; ++j) {
      RowTile t;
      t.group = g;
      t.row0 = r0 + j * BM;
      t.rows = j + 1 < m ? BM : rows - j * BM;
      const bool hv = h && j + 1 == m;
      t.first = hv ? hstart : start;
      t.count = hv ? 1 : m - h;
      t.pad0 = t.pad1 = t.pad2 = 0;
      tiles[hv ? hstart : start + j] = t;
    }
  }
  if (g == 0) {
    ntiles[0] = heavy + normal;
    ntiles[kSplitSlots + 1] = heavy;
  }
  // arrival counters of the grouped GEMM's K split start from zero
  for (int i = threadIdx.x; i < kSplitSlots; i += blockDim.x) ntiles[1 + i] = 0;
}

// Sum of v over the block: xor-shuffle tree in each wave (every lane ends with
// the same value), then the 16 wave sums in wave order.  Fixed order, so the
// result does not change from run to run.  wsd: 16 doubles of LDS.
__device__ inline double block_sum_d(double v, double* wsd) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  if (lane == 0) wsd[wave] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < kMaxExperts / 64; ++w) t += wsd[w];
  __syncthreads();
  return t;
}

// Load statistics from the gate's per-block probability sums (fp64):
// mean_prob[e] = (sum over the nb blocks, a fixed order) / T, and balance =
// unbiased variance of mean_prob over the E experts.  Either output may be null;
// T = 0 gives NaN means, E = 1 a NaN variance.  Called by every thread of a
// block of kMaxExperts threads.
__device__ inline void load_stats(const double* __restrict__ stat_part, int nb, int E, int64_t T,
                                  float* __restrict__ mean_prob, float* __restrict__ balance,
                                  double* wsd) {
  const int e = threadIdx.x;
  // thread (c, e') adds expert e' over range c of the blocks; thread e then
  // adds its ranges in order
  __shared__ double rsum[kMaxExperts];
  const int chunks = max(1, min(kMaxExperts / E, nb));
  const int len = (nb + chunks - 1) / chunks;
  const int c1 = threadIdx.x / E, e1 = threadIdx.x - c1 * E;
  if (c1 < chunks) {
    double r = 0.0;
    const int b0 = c1 * len, b1 = min(nb, b0 + len);
#pragma unroll 4
    for (int b = b0; b < b1; ++b) r += stat_part[static_cast<int64_t>(b) * E + e1];
    rsum[e1 * chunks + c1] = r;
  }
  __syncthreads();
  double mp = 0.0;
  if (e < E) {
    double acc = 0.0;
    for (int c = 0; c < chunks; ++c) acc += rsum[e * chunks + c];
    mp = acc / static_cast<double>(T);
    if (mean_prob) mean_prob[e] = static_cast<float>(mp);
  }
  if (balance) {
    const double mean = block_sum_d(e < E ? mp : 0.0, wsd) / static_cast<double>(E);
    const double dv = e < E ? mp - mean : 0.0;
    const double var = block_sum_d(dv * dv, wsd);
    if (e == 0) balance[0] = static_cast<float>(var / static_cast<double>(E - 1));
  }
}

// Squared coefficient of variation of the per-expert counts: unbiased variance
// over the E experts divided by the squared mean, in fp64 (integer counts make
// the mean exact; 0/0 gives NaN for E = 1 or no pairs).  Thread e < E passes
// counts[e].  Called by every thread of the block.
__device__ inline void counts_cv2(int cnt, int E, float* __restrict__ cv2, double* wsd) {
  const int e = threadIdx.x;
  const double c = e < E ? static_cast<double>(cnt) : 0.0;
  const double mean = block_sum_d(c, wsd) / static_cast<double>(E);
  const double dv = e < E ? c - mean : 0.0;
  const double var = block_sum_d(dv * dv, wsd) / static_cast<double>(E - 1);
  if (e == 0) cv2[0] = static_cast<float>(var / (mean * mean));
}

}  // namespace moe
