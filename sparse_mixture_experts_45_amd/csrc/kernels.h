// Launch plans and entry points of the HIP kernels (internal to the library).
#pragma once
#include "common.h"

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;

struct RoutePlan {
  int64_t T;
  int d, E, k, renorm;
  int S, kchunk;  // router score split over d: S chunks of kchunk columns
  int lpt, vpl;   // gate: lanes per token (16 or 64), values per lane
  int fused;      // scores and gate in one kernel (bf16, E <= 64, S = 1)
  int64_t ps_t, ps_e;  // element strides of the optional probabilities output
  int nb;         // gate blocks = ceil(T / kGateTokens)
};

// Row-tile shapes of the grouped GEMM.  Chosen on the host from the shape only.
enum GemmShape {
  kGemmF32 = 0,        // fp32 MFMA, register-staged tiles
  kGemmBf16Large = 1,  // bf16, register-staged (any K multiple of 8)
  kGemmBf16Mid = 2,
  kGemmBf16Small = 3,
  kGemmDmaLarge = 4,   // bf16, K multiple of 64, LDS-DMA tiles (kDma* below)
  kGemmDmaMid = 5,
  kGemmDmaSmall = 6,
  kGemmDmaSkinny = 7,
  kGemmDmaTall = 8
};

// Tile configurations of the LDS-DMA grouped GEMM.  The host plan (row-tile
// height for the tile list) and the launcher read the same table.
struct DmaCfg {
  // rows, up/down columns, K step, stages, the up GEMM's wave grid, the waves
  // per SIMD the register budget is sized for, whether blocks stay resident and
  // walk several tiles (1) or each block takes one tile (0), and the down
  // GEMM's wave grid; SPLIT: partial tiles reserved for the K split below (0:
  // the tier never splits); NTB: the weight (B) tiles of the forward and
  // input-gradient GEMMs are loaded with the non-temporal cache policy (1):
  // measured faster where the layer's weights are streamed (the 32-, 192- and
  // 256-row tiers), slower where they are read again from the caches (the
  // 64- and 128-row tiers)
  int BM, BNU, BND, BK, NS, WM, WN, OCC, PERSIST, WMD, WND, SPLIT, NTB;
};
constexpr DmaCfg kDmaLarge{256, 256, 256, 64, 2, 2, 4, 2, 0, 2, 4, 256, 1};  // >= 768 rows per expert
constexpr DmaCfg kDmaMid{128, 128, 128, 64, 2, 2, 4, 2, 0, 2, 4, 512, 0};    // >= 256
constexpr DmaCfg kDmaSmall{64, 128, 128, 64, 3, 1, 4, 2, 1, 1, 4, 0, 0};     // >= 48 (3 stages: 2 blocks per CU)
constexpr DmaCfg kDmaSkinny{32, 128, 128, 64, 3, 1, 4, 2, 0, 1, 4, 0, 1};    // fewer: weight streaming
// 192-row tiles where an expert's rows (about 128-165) fit one: a quarter
// fewer MFMAs on padding rows than 256
constexpr DmaCfg kDmaTall{192, 256, 256, 64, 2, 2, 4, 2, 0, 2, 4, 256, 1};

// K split of a last, partly filled round.  When a launch's tiles leave the
// final round of resident blocks (`slots` of them) at most half full, each of
// those R tiles is cut into S <= slots / R parts along K, run by S blocks; a
// part parks its fp32 accumulators in a partial-tile slot, and the part that
// arrives last (an arrival counter per tile) adds the S slots in part order and
// runs the tile's epilogue.  The sum order is fixed, so results do not depend
// on which part finishes first.  Counters are zeroed with every tile list and
// reset by the last part.
constexpr int kSplitMax = 4;       // parts per tile
constexpr int kSplitMinSteps = 32;  // K steps per part, at least (the fences cost)
constexpr int kSplitSlots = 512;   // counters kept after the tile count (>= every SPLIT)
static_assert(kDmaLarge.SPLIT <= kSplitSlots && kDmaMid.SPLIT <= kSplitSlots &&
                  kDmaTall.SPLIT <= kSplitSlots,
              "split slots");

struct GemmPlan {
  int shape;        // GemmShape
  int BM;             // rows per tile (the row-tile list is cut at BM)
  int extra;          // rows past BM a group's last tile may take instead of a tile of
                      // their own (heavy tiles of the forward's 256-row tier), or 0
  int64_t tiles_max;  // upper bound on row tiles over all groups
  int64_t kpart_floats;  // fp32 partial tiles of the K split (0: no split)
};

// Passes of the grouped-GEMM pair.  kPassDgrad is the input-gradient pass of
// the backward, run with the forward's argument roles re-bound: x = dy
// (gathered), W1 = the forward's W2 and W2 = the forward's W1 (likewise the
// shared expert's), both read in their stored layout as [K, N] matrices
// (W2[e] is [d, F]: K = d, N = F), no biases, H = the forward's
// pre-activations (overwritten with dz = gate * (dy W2) * act'(z)), y_rows =
// dz W1 per row (fp32, no gate).
enum { kPassForward = 0, kPassForwardTrain = 1, kPassDgrad = 2 };

struct FfnArgs {
  int64_t T;
  int d, F, E, k, Fs, act, dtype;
  const void* x;
  const void *W1, *b1, *W2, *b2, *Ws1, *bs1, *Ws2, *bs2;
  const int32_t *offsets, *row_token, *row_slot;
  const float* topk_w;
  void* H;           // [rows_max, max(F, Fs)] in dtype
  float* y_rows;     // [rows_max, d]
  RowTile* tiles;    // [tiles_max]
  int32_t* ntiles;   // [2 + kSplitSlots]: the tile count, the split counters, the
                     // heavy tile count
  float* row_gate;   // [rows_max]
  int64_t rows_max;  // bound on the routed plus shared rows (grid of the tile-list kernel)
  int tiles_ready;   // tiles, ntiles and row_gate already written by the dispatch
  int row_gates;     // topk_w holds one gate per routed row (expert choice)
  int pass;          // kPassForward, kPassForwardTrain (also keeps z in Z) or
                     // kPassDgrad (the roles above)
  void* Z;           // [rows_max, max(F, Fs)] pre-activations (train / dgrad)
  float* kpart;      // [GemmPlan::kpart_floats] partial tiles of the K split, or null
  int32_t* ksem;     // [kSplitSlots] arrival counters of split tiles (ntiles + 1)
};

// Everything the fused dispatch reads and writes.
struct DispatchArgs {
  const int32_t* topk_idx;  // [T, k]
  const float* topk_w;      // [T, k]
  const int32_t* hist;      // [nb, E] pairs per 64-token block and expert
  const double* stat_part;  // [nb, E] per-block sums of router probabilities
  int64_t T;
  int nb, E, k, capacity, shared, BM, extra;
  int32_t *counts, *kept, *offsets, *row_token, *row_slot, *inv;
  float* row_gate;
  RowTile* tiles;
  int32_t* ntiles;
  float *mean_prob, *balance, *cv2;  // optional
};

// Every workgroup of the fused dispatch reads the whole per-block histogram
// (nb * E ints); up to this size that costs less than separate scan and
// scatter launches.  kDispatchLdsBases also bounds the LDS copy of the
// multi-kernel path's scan.
constexpr int kDispatchLdsBases = 8192;
inline bool dispatch_fused(int64_t nb, int E) { return nb * E <= kDispatchLdsBases; }

hipError_t launch_router(const RoutePlan& p, const void* x, int dtype, const float* Wg,
                         const float* bg, float* part, int32_t* topk_idx, float* topk_w,
                         float* probs, double* stat_part, int32_t* hist, float* mean_prob,
                         float* balance, hipStream_t st);

hipError_t launch_dispatch(int64_t T, int E, int k, int capacity, int shared, int nb,
                           const int32_t* topk_idx, bool need_hist, int32_t* hist, int32_t* base,
                           int32_t* counts, int32_t* kept, int32_t* offsets, int32_t* row_token,
                           int32_t* row_slot, int32_t* inv, float* cv2, hipStream_t st);

hipError_t launch_dispatch_blocks(const DispatchArgs& a, hipStream_t st);

// Everything the expert-choice selection and its finishing block read and write.
struct EcArgs {
  int64_t T;
  int E, Ce, W, shared, BM, extra, nb;  // Ce tokens per expert; W = ceil(T / 32) bitmap words
  int32_t *row_token, *offsets, *counts, *kept;  // counts, kept optional
  float* row_gate;
  uint32_t* sel;   // [E, W] selection bitmap
  int32_t* pre;    // [E, W] taken tokens before each word
  RowTile* tiles;
  int32_t* ntiles;
  const double* stat_part;     // [nb, E] gate-block probability sums
  float *mean_prob, *balance, *cv2;  // optional
  int32_t* ec_idx;  // optional [E, Ce] copy of row_token's routed rows
  float* ec_w;      // optional [E, Ce] copy of their gates
};

hipError_t launch_expert_choice(const EcArgs& a, const float* probsT, hipStream_t st);
hipError_t launch_combine_ec(int64_t T, int d, int E, int Ce, int shared, int dtype,
                             const float* y_rows, const uint32_t* sel, const int32_t* pre,
                             void* y, hipStream_t st);

hipError_t launch_ffn(const GemmPlan& gp, const FfnArgs& a, hipStream_t st);

// Weight gradients on the LDS-DMA GEMM (bf16): C[g] [M, N] = A[:, Kg] B[:, Kg]^T
// for groups g = 0 .. groups-1, Kg = columns poff[g0 + g] .. poff[g0 + g + 1]
// (multiples of 64) of A [M, lda] and B [N, ldb].  `shape` picks the 256- or
// 128-row tile configuration; wgrad_dma_fits says whether this path applies.
struct WgradGemm {
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  const int32_t* poff;
  int g0, groups, M, N;
  void* C;
};
bool wgrad_dma_fits(int shape, const WgradGemm& w);
hipError_t launch_wgrad_dma(int shape, const WgradGemm& w, hipStream_t st);

// Backward (token choice).  moe_backward enqueues, in order: kBwdRouter (gate
// gradients, the balance term,
// router-score gradients dl, dW_g and db_g), the input-gradient GEMM pass
// (launch_ffn with kPassDgrad), kBwdDx (dx), kBwdExpertWeights (transposed
// activations, expert weight and bias gradients).
enum { kBwdRouter = 1, kBwdDx = 2, kBwdExpertWeights = 3 };
struct BwdArgs {
  int64_t T;
  int64_t rows_avg;             // routed rows per expert, at most, on average
  int d, F, E, k, Fs, dtype, renorm, nb;
  float alpha;                  // coefficient of the balance term
  const void *x, *dy;           // [T, d] layer dtype
  const float* Wg;              // [E, d]
  const float* probs;           // [T, E] the forward's softmax (token choice)
  const int32_t* topk_idx;      // [T, k]
  const float* topk_w;          // [T, k]
  const int32_t* inv;           // [T, k] row of each pair, -1 when dropped
  // expert choice: rows e * Ce + j, gates p[t, e], the selection as bitmaps
  int ec, Ce, W;                // W = ceil(T / 32)
  const uint32_t* sel;          // [E, W] bit t of expert e: e took token t
  const int32_t* pre;           // [E, W] tokens expert e took before word w
  const float* probsT;          // [E, T] the forward's softmax
  const int32_t *offsets, *row_token;  // the forward's grouping
  const float* row_gate;        // [rows] gate of each row (1 for shared rows)
  const double* stat_part;      // [nb, E] the gate's per-block probability sums
  const float* y_rows;          // [rows, d] the forward's gated expert outputs
  float *dg, *dl, *aux_dp;      // scratch [T, k] (expert choice: [E * Ce]), [T, E], [E]
  float* wg_part;               // scratch [wg_split, E, d + 1]
  int wg_split;
  int64_t wg_chunk;             // tokens per split
  const float* dX;              // [rows, d] dz W1 per row (the dgrad pass's y_rows)
  const void *Z, *H;            // [rows, ldh] dz (after the dgrad pass) and h
  int32_t* poff;                // [G + 1] padded column offsets
  int64_t Rp;                   // columns of the transposed buffers (multiple of 64)
  void *ZT, *HT, *XT, *DT;      // [ldh, Rp], [ldh, Rp], [d, Rp], [d, Rp]
  float* bsum;                  // [Rp / 64, max(ldh, d)] 64-row block sums (bias gradients)
  // outputs, NULL = not wanted
  void* dx;
  float *dWg, *dbg;
  void *dW1, *db1, *dW2, *db2, *dWs1, *dbs1, *dWs2, *dbs2;
};
hipError_t launch_backward(const BwdArgs& b, int part, hipStream_t st);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);

hipError_t launch_combine(int64_t T, int d, int E, int k, int shared, int dtype,
                          const float* y_rows, const int32_t* inv, const int32_t* offsets,
                          void* y, hipStream_t st);

}  // namespace moe
