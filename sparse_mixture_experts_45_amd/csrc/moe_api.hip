// C ABI of the MoE layer: argument checks, workspace carve-up, launch order.
// Nothing here allocates, synchronises or reads device memory.
#include <string.h>

#include <cmath>
#include <mutex>

#include "kernels.h"
#include "router_tile.h"

using namespace moe;

// Workspace of moe_forward_noalloc: one static array per GPU, held until the
// process ends.  In host code its name is only a stand-in for the device
// array: the address on each device comes from hipGetSymbolAddress, looked up
// once per device (with it current) and kept below.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

struct Layout {
  RoutePlan rp;
  GemmPlan gp;
  int64_t rows_max;  // routed rows (T*k, or E*C under expert choice) + (Fs ? T : 0)
  int64_t ec_C;      // tokens per expert under expert choice
  int ec_W;          // 32-token words of the expert-choice bitmaps
  size_t part, stat, hist, base, topk_idx, topk_w, counts, kept, offsets, row_token, row_slot,
      inv, tiles, ntiles, row_gate, probsT, sel, pre, H, y_rows, kpart, total;
  // training: what the forward keeps for the backward, and the backward's scratch
  bool train;
  int wg_split;
  int64_t wg_chunk, Rp;
  size_t Z, probs, dg, dl, aux_dp, wg_part, poff, ZT, HT, XT, DT, bsum;
};

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

moe_status noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return MOE_OK;
}

bool expert_choice(const moe_config* c) { return c->routing == MOE_ROUTE_EXPERT; }

// Tokens each expert takes under expert choice: the capacity if set, else
// floor(T * k / E); at most T.
int64_t ec_capacity(const moe_config* c) {
  const int64_t C = c->capacity >= 0 ? c->capacity : c->T * c->top_k / c->n_experts;
  return std::min<int64_t>(C, c->T);
}

// Routed (expert, token) rows the expert MLPs can receive.
int64_t routed_rows_max(const moe_config* c) {
  if (expert_choice(c)) return int64_t(c->n_experts) * ec_capacity(c);
  const int64_t pairs = c->T * c->top_k;
  return c->capacity >= 0 ? std::min<int64_t>(pairs, int64_t(c->n_experts) * c->capacity) : pairs;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status check_config(const moe_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->T < 0 || c->d_model < 8 || c->d_ff < 8 || c->n_experts < 1 || c->top_k < 1 ||
      c->shared_d_ff < 0)
    return MOE_ERR_INVALID_ARG;
  if (c->d_model % 8 || c->d_ff % 8 || c->shared_d_ff % 8) return MOE_ERR_INVALID_ARG;
  if (c->act != MOE_ACT_GELU && c->act != MOE_ACT_RELU) return MOE_ERR_INVALID_ARG;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (c->renormalize != 0 && c->renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (c->routing != MOE_ROUTE_TOKEN && c->routing != MOE_ROUTE_EXPERT) return MOE_ERR_INVALID_ARG;
  if (c->top_k > c->n_experts) return MOE_ERR_INVALID_ARG;
  if (c->n_experts + (c->shared_d_ff > 0 ? 1 : 0) > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (expert_choice(c)) {
    // the gate runs with k = 1; k only sets the default C
    if (c->n_experts * ec_capacity(c) + c->T >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
  }
  if (c->top_k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
  if (c->T * (c->top_k + 1) >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

GemmPlan gemm_plan(const moe_config* c) {
  GemmPlan g{};
  const int64_t rmax = routed_rows_max(c);
  const int64_t avg = rmax / c->n_experts;
  // The LDS-DMA tiers read 64-element K steps and address gathered token rows
  // (x, dy: [T, d]) and one expert's weights ([F, d] or [d, F]) with 32-bit
  // byte offsets; other shapes take the tiers with 64-bit addressing.
  const int64_t four_gib = int64_t(1) << 32;
  const int64_t fmax = std::max<int64_t>(c->d_ff, c->shared_d_ff);
  const bool k64 = c->d_model % 64 == 0 && c->d_ff % 64 == 0 && c->shared_d_ff % 64 == 0 &&
                   c->T * c->d_model * 2 <= four_gib && fmax * c->d_model * 2 <= four_gib;
  // expert choice gives every expert exactly C rows: whole 256-row tiles pay
  // when their padding is at most 1/8 of the rows
  const int64_t C = expert_choice(c) ? ec_capacity(c) : 0;
  const bool ec_whole = C >= 256 && (ceil_div(C, 256) * 256 - C) * 8 <= C;
  // 256 x 256 tiles read an expert's weights once per 256 rows, against two
  // to four times for the narrower tiers; they pay from 128 rows per expert
  // once the smaller of the two GEMMs still has >= 128 of them (the K split
  // fills the rest of the machine).  Under a capacity limit the rows per
  // expert are only bounded above (a skewed router leaves most experts far
  // below it), so such layers keep the row-count thresholds.
  const bool uncapped = c->capacity < 0 && !expert_choice(c);
  const int64_t large_rows = int64_t(c->n_experts) * ceil_div(std::max<int64_t>(avg, 1), 256);
  const bool large_fills =
      uncapped && avg >= 128 &&
      large_rows * std::min(ceil_div(fmax, 256), ceil_div(int64_t(c->d_model), 256)) >= 128;
  if (c->dtype == MOE_F32) {
    g.shape = kGemmF32;
    g.BM = 64;
  } else if (k64 && (avg >= 768 || ec_whole || large_fills)) {
    // 192-row tiles when an expert's rows, two standard deviations of an
    // even routing above the mean, fit one of them
    const bool tall = large_fills && avg + 2.0 * std::sqrt(static_cast<double>(avg)) <= 192.0;
    const DmaCfg& L = tall ? kDmaTall : kDmaLarge;
    g.shape = tall ? kGemmDmaTall : kGemmDmaLarge;
    g.BM = L.BM;
    g.kpart_floats = int64_t(L.SPLIT) * L.BM * std::max(L.BNU, L.BND);
  } else if (k64 && avg >= 256) {
    g.shape = kGemmDmaMid;
    g.BM = kDmaMid.BM;
    g.kpart_floats = int64_t(kDmaMid.SPLIT) * kDmaMid.BM * std::max(kDmaMid.BNU, kDmaMid.BND);
  } else if (k64 && avg >= 48) {
    g.shape = kGemmDmaSmall;
    g.BM = kDmaSmall.BM;
  } else if (k64) {
    g.shape = kGemmDmaSkinny;
    g.BM = kDmaSkinny.BM;
  } else if (avg >= 128) {
    g.shape = kGemmBf16Large;
    g.BM = 128;
  } else if (avg >= 48) {
    g.shape = kGemmBf16Mid;
    g.BM = 64;
  } else {
    g.shape = kGemmBf16Small;
    g.BM = 32;
  }
  // sum_e ceil(r_e / BM) <= ceil(R / BM) + (number of non-empty experts)
  g.tiles_max = ceil_div(rmax, g.BM) + std::min<int64_t>(c->n_experts, rmax) +
                (c->shared_d_ff > 0 ? ceil_div(c->T, g.BM) : 0);
  return g;
}

RoutePlan route_plan(const moe_config* c) {
  RoutePlan p{};
  p.T = c->T;
  p.d = c->d_model;
  p.E = c->n_experts;
  p.k = expert_choice(c) ? 1 : c->top_k;
  p.renorm = expert_choice(c) ? 0 : c->renormalize;
  p.nb = static_cast<int>(ceil_div(c->T, kGateTokens));
  if (expert_choice(c)) {  // probabilities [E, T]: one expert's are contiguous
    p.ps_t = 1;
    p.ps_e = c->T;
  } else {  // [T, E] row-major
    p.ps_t = c->n_experts;
    p.ps_e = 1;
  }
  // Split d so the score kernel has >= ~256 blocks, each K slice of a block
  // keeping >= 2 K steps.  bf16 layers whose experts fit one score tile
  // (E <= 64) and that gain nothing from a split run the gate inside the score
  // kernel (one launch).
  const int TE = router_tile(c->n_experts, c->dtype);
  const int QK = 16 / (TE / 16);
  const int64_t base_blocks = ceil_div(c->T, 64) * ceil_div(c->n_experts, TE);
  int S = static_cast<int>(std::max<int64_t>(1, ceil_div(256, std::max<int64_t>(1, base_blocks))));
  S = std::min(S, std::max(1, c->d_model / (QK * 64)));
  S = std::min(S, 16);
  p.fused = c->dtype == MOE_BF16 && c->n_experts <= 64 && S == 1;
  p.kchunk = static_cast<int>(align_up(ceil_div(c->d_model, S), 32));
  p.S = static_cast<int>(ceil_div(c->d_model, p.kchunk));
  // gate: 16 lanes per token up to 256 experts (DPP-only reductions), else 64
  p.lpt = c->n_experts <= 256 ? 16 : 64;
  const int need = static_cast<int>(ceil_div(c->n_experts, p.lpt));
  int vpl = 1;
  while (vpl < need) vpl <<= 1;
  p.vpl = vpl;
  return p;
}

Layout layout(const moe_config* c, bool train = false) {
  Layout L{};
  L.train = train;
  L.rp = route_plan(c);
  L.gp = gemm_plan(c);
  if (!train && L.gp.shape == kGemmDmaLarge) {
    // the forward's 256-row tiles take up to one more 32-row block per wave
    // row: a group's last rows, when they are that few, join its previous
    // tile; the K split's partial tiles grow by those rows
    L.gp.extra = kDmaLarge.WM * 32;
    L.gp.kpart_floats = int64_t(kDmaLarge.SPLIT) * (kDmaLarge.BM + L.gp.extra) *
                        std::max(kDmaLarge.BNU, kDmaLarge.BND);
  }
  const int64_t T = c->T, E = c->n_experts, k = L.rp.k;
  const bool ec = expert_choice(c);
  L.ec_C = ec ? ec_capacity(c) : 0;
  L.ec_W = ec ? static_cast<int>(ceil_div(T, 32)) : 0;
  L.rows_max = routed_rows_max(c) + (c->shared_d_ff > 0 ? T : 0);
  const size_t elt = c->dtype == MOE_BF16 ? 2 : 4;
  const int64_t ldh = std::max(c->d_ff, c->shared_d_ff);
  const int64_t nb = L.rp.nb;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + std::max<size_t>(bytes, 1), kAlign);
    return at;
  };
  L.part = take(sizeof(float) * L.rp.S * T * E);
  L.stat = take(sizeof(double) * nb * E);
  L.hist = take(sizeof(int32_t) * nb * E);
  L.base = take(sizeof(int32_t) * nb * E);
  L.topk_idx = take(sizeof(int32_t) * T * k);
  L.topk_w = take(sizeof(float) * T * k);
  L.counts = take(sizeof(int32_t) * E);
  L.kept = take(sizeof(int32_t) * E);
  L.offsets = take(sizeof(int32_t) * (E + 2));
  L.row_token = take(sizeof(int32_t) * L.rows_max);
  L.row_slot = take(sizeof(int32_t) * (ec ? 0 : L.rows_max));
  L.inv = take(sizeof(int32_t) * (ec ? 0 : T * k));
  L.tiles = take(sizeof(RowTile) * L.gp.tiles_max);
  L.ntiles = take(sizeof(int32_t) * (2 + kSplitSlots));  // count, split counters, heavy count
  L.row_gate = take(sizeof(float) * L.rows_max);
  L.probsT = take(sizeof(float) * (ec ? E * T : 0));
  L.sel = take(sizeof(uint32_t) * E * L.ec_W);
  L.pre = take(sizeof(int32_t) * E * L.ec_W);
  L.H = take(elt * L.rows_max * ldh);
  L.y_rows = take(sizeof(float) * L.rows_max * c->d_model);
  L.kpart = take(sizeof(float) * L.gp.kpart_floats);
  if (train) {
    const int64_t d = c->d_model, F = c->d_ff, Fs = c->shared_d_ff;
    const int64_t G = E + (Fs > 0 ? 1 : 0);
    L.Z = take(elt * L.rows_max * ldh);
    L.probs = take(sizeof(float) * (ec ? 0 : T * E));  // expert choice keeps probsT
    // gate gradients: one per (token, slot), or per routed row under expert choice
    L.dg = take(sizeof(float) * (ec ? L.rows_max : T * k));
    L.dl = take(sizeof(float) * T * E);
    L.aux_dp = take(sizeof(float) * E);
    // router weight gradient: enough token chunks for ~512 blocks
    const int64_t col_blocks = ceil_div(d + 1, 256 * 8) * ceil_div(E, 8);  // 8 columns a thread
    L.wg_split = static_cast<int>(std::max<int64_t>(
        1, std::min<int64_t>(ceil_div(512, col_blocks), ceil_div(std::max<int64_t>(T, 1), 64))));
    L.wg_chunk = ceil_div(std::max<int64_t>(T, 1), L.wg_split);
    L.wg_part = take(sizeof(float) * L.wg_split * E * (d + 1));
    L.poff = take(sizeof(int32_t) * (G + 1));
    L.Rp = static_cast<int64_t>(align_up(L.rows_max + 64 * G, 64));
    L.ZT = take(elt * ldh * L.Rp);
    L.HT = take(elt * ldh * L.Rp);
    L.XT = take(elt * d * L.Rp);
    L.DT = take(elt * d * L.Rp);
    L.bsum = take(sizeof(float) * (L.Rp / 64) * std::max<int64_t>(ldh, d));
  }
  L.total = o;
  return L;
}

inline char* at(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

moe_status check_ws(const Layout& L, void* ws, size_t ws_bytes) {
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) || ws_bytes < L.total)
    return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

moe_status check_weights(const moe_config* c, const moe_weights* w) {
  if (!w || !w->Wg || !w->W1 || !w->W2) return MOE_ERR_INVALID_ARG;
  if (!aligned16(w->Wg) || !aligned16(w->W1) || !aligned16(w->W2)) return MOE_ERR_INVALID_ARG;
  if (c->shared_d_ff > 0) {
    if (!w->Ws1 || !w->Ws2 || !aligned16(w->Ws1) || !aligned16(w->Ws2)) return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

moe_status run_ffn(const moe_config* c, const Layout& L, const void* x, const moe_weights* w,
                   const int32_t* offsets, const int32_t* row_token, const int32_t* row_slot,
                   const float* topk_w, float* y_rows, void* ws, hipStream_t st,
                   bool tiles_ready = false, int pass = kPassForward) {
  FfnArgs f{};
  f.T = c->T;
  f.d = c->d_model;
  f.F = c->d_ff;
  f.E = c->n_experts;
  f.k = c->top_k;
  f.Fs = c->shared_d_ff;
  f.act = c->act;
  f.dtype = c->dtype;
  f.x = x;
  f.W1 = w->W1;
  f.b1 = w->b1;
  f.W2 = w->W2;
  f.b2 = w->b2;
  f.Ws1 = w->Ws1;
  f.bs1 = w->bs1;
  f.Ws2 = w->Ws2;
  f.bs2 = w->bs2;
  f.offsets = offsets;
  f.row_token = row_token;
  f.row_slot = row_slot;
  f.topk_w = topk_w;
  f.H = at(ws, L.H);
  f.y_rows = y_rows;
  f.tiles = reinterpret_cast<RowTile*>(at(ws, L.tiles));
  f.ntiles = reinterpret_cast<int32_t*>(at(ws, L.ntiles));
  f.row_gate = reinterpret_cast<float*>(at(ws, L.row_gate));
  f.tiles_ready = tiles_ready ? 1 : 0;
  f.rows_max = L.rows_max;
  f.row_gates = expert_choice(c) ? 1 : 0;
  f.pass = pass;
  f.Z = pass == kPassForwardTrain ? at(ws, L.Z) : nullptr;
  f.kpart = L.gp.kpart_floats ? reinterpret_cast<float*>(at(ws, L.kpart)) : nullptr;
  f.ksem = f.ntiles + 1;
  return hip_status(launch_ffn(L.gp, f, st));
}

// Expert-choice layer: the router writes the probabilities expert-major, each
// expert selects its C tokens, the expert MLPs run over the E * C rows (+ the
// shared expert's T), and the combine walks the selection bitmaps.
moe_status forward_expert_choice(const moe_config* c, const Layout& L, const moe_weights* w,
                                 const void* x, void* y, const moe_stats& o, void* ws,
                                 hipStream_t st) {
  moe_status s;
  float* probsT = reinterpret_cast<float*>(at(ws, L.probsT));
  double* stat_part = reinterpret_cast<double*>(at(ws, L.stat));
  // the gate's top-1 and histogram go to scratch; only probsT and stat_part are used
  if ((s = hip_status(launch_router(L.rp, x, c->dtype, w->Wg, w->bg,
                                    reinterpret_cast<float*>(at(ws, L.part)),
                                    reinterpret_cast<int32_t*>(at(ws, L.topk_idx)),
                                    reinterpret_cast<float*>(at(ws, L.topk_w)), probsT, stat_part,
                                    reinterpret_cast<int32_t*>(at(ws, L.hist)), nullptr, nullptr,
                                    st))) != MOE_OK)
    return s;
  EcArgs a{};
  a.T = c->T;
  a.E = c->n_experts;
  a.Ce = static_cast<int>(L.ec_C);
  a.W = L.ec_W;
  a.shared = c->shared_d_ff > 0;
  a.BM = L.gp.BM;
  a.extra = L.gp.extra;
  a.nb = L.rp.nb;
  a.row_token = reinterpret_cast<int32_t*>(at(ws, L.row_token));
  a.offsets = reinterpret_cast<int32_t*>(at(ws, L.offsets));
  a.counts = o.counts;
  a.kept = o.kept;
  a.row_gate = reinterpret_cast<float*>(at(ws, L.row_gate));
  a.sel = reinterpret_cast<uint32_t*>(at(ws, L.sel));
  a.pre = reinterpret_cast<int32_t*>(at(ws, L.pre));
  a.tiles = reinterpret_cast<RowTile*>(at(ws, L.tiles));
  a.ntiles = reinterpret_cast<int32_t*>(at(ws, L.ntiles));
  a.stat_part = stat_part;
  a.mean_prob = o.mean_prob;
  a.balance = o.balance;
  a.cv2 = o.cv2;
  a.ec_idx = o.ec_idx;
  a.ec_w = o.ec_w;
  if ((s = hip_status(launch_expert_choice(a, probsT, st))) != MOE_OK) return s;
  if (c->T == 0) return MOE_OK;
  float* y_rows = reinterpret_cast<float*>(at(ws, L.y_rows));
  if ((s = run_ffn(c, L, x, w, a.offsets, a.row_token, nullptr, nullptr, y_rows, ws, st, true,
                   L.train ? kPassForwardTrain : kPassForward)) != MOE_OK)
    return s;
  return hip_status(launch_combine_ec(c->T, c->d_model, c->n_experts, a.Ce, a.shared, c->dtype,
                                      y_rows, a.sel, a.pre, y, st));
}

// Token-choice layer (train: also keeps the softmax and the pre-activations
// for moe_backward).
moe_status forward_token(const moe_config* cfg, const Layout& L, const moe_weights* w,
                         const void* x, void* y, const moe_stats& o, void* ws, hipStream_t st) {
  moe_status s;
  // training keeps the routing in the workspace (copied out when asked for)
  int32_t* topk_idx = o.topk_idx && !L.train ? o.topk_idx
                                             : reinterpret_cast<int32_t*>(at(ws, L.topk_idx));
  float* topk_w = o.topk_w && !L.train ? o.topk_w : reinterpret_cast<float*>(at(ws, L.topk_w));
  int32_t* counts = o.counts ? o.counts : reinterpret_cast<int32_t*>(at(ws, L.counts));
  int32_t* kept = o.kept ? o.kept : reinterpret_cast<int32_t*>(at(ws, L.kept));
  int32_t* offsets = reinterpret_cast<int32_t*>(at(ws, L.offsets));
  int32_t* row_token = reinterpret_cast<int32_t*>(at(ws, L.row_token));
  int32_t* row_slot = reinterpret_cast<int32_t*>(at(ws, L.row_slot));
  int32_t* inv = reinterpret_cast<int32_t*>(at(ws, L.inv));
  int32_t* hist = reinterpret_cast<int32_t*>(at(ws, L.hist));
  float* y_rows = reinterpret_cast<float*>(at(ws, L.y_rows));

  double* stat_part = reinterpret_cast<double*>(at(ws, L.stat));
  // up to kDispatchLdsBases histogram entries: the whole dispatch (and the load
  // statistics) in one launch
  const bool one = dispatch_fused(L.rp.nb, cfg->n_experts);
  if ((s = hip_status(launch_router(L.rp, x, cfg->dtype, w->Wg, w->bg,
                                    reinterpret_cast<float*>(at(ws, L.part)), topk_idx, topk_w,
                                    L.train ? reinterpret_cast<float*>(at(ws, L.probs)) : nullptr,
                                    stat_part, hist, one ? nullptr : o.mean_prob,
                                    one ? nullptr : o.balance, st))) != MOE_OK)
    return s;
  if (L.train && cfg->T > 0) {
    const size_t n = static_cast<size_t>(cfg->T) * cfg->top_k * 4;
    if (o.topk_idx &&
        (s = hip_status(hipMemcpyAsync(o.topk_idx, topk_idx, n, hipMemcpyDeviceToDevice, st))) !=
            MOE_OK)
      return s;
    if (o.topk_w &&
        (s = hip_status(hipMemcpyAsync(o.topk_w, topk_w, n, hipMemcpyDeviceToDevice, st))) !=
            MOE_OK)
      return s;
  }
  // the gate kernel already wrote the per-block expert histogram
  if (one) {
    DispatchArgs d{};
    d.topk_idx = topk_idx;
    d.topk_w = topk_w;
    d.hist = hist;
    d.stat_part = stat_part;
    d.T = cfg->T;
    d.nb = L.rp.nb;
    d.E = cfg->n_experts;
    d.k = cfg->top_k;
    d.capacity = cfg->capacity;
    d.shared = cfg->shared_d_ff > 0;
    d.BM = L.gp.BM;
    d.extra = L.gp.extra;
    d.counts = counts;
    d.kept = kept;
    d.offsets = offsets;
    d.row_token = row_token;
    d.row_slot = row_slot;
    d.inv = inv;
    d.row_gate = reinterpret_cast<float*>(at(ws, L.row_gate));
    d.tiles = reinterpret_cast<RowTile*>(at(ws, L.tiles));
    d.ntiles = reinterpret_cast<int32_t*>(at(ws, L.ntiles));
    d.mean_prob = o.mean_prob;
    d.balance = o.balance;
    d.cv2 = o.cv2;
    if ((s = hip_status(launch_dispatch_blocks(d, st))) != MOE_OK) return s;
  } else if ((s = hip_status(launch_dispatch(cfg->T, cfg->n_experts, cfg->top_k, cfg->capacity,
                                             cfg->shared_d_ff > 0, L.rp.nb, topk_idx, false,
                                             hist, reinterpret_cast<int32_t*>(at(ws, L.base)),
                                             counts, kept, offsets, row_token, row_slot, inv,
                                             o.cv2, st))) != MOE_OK) {
    return s;
  }
  if (cfg->T == 0) return MOE_OK;
  if ((s = run_ffn(cfg, L, x, w, offsets, row_token, row_slot, topk_w, y_rows, ws, st, one,
                   L.train ? kPassForwardTrain : kPassForward)) != MOE_OK)
    return s;
  return hip_status(launch_combine(cfg->T, cfg->d_model, cfg->n_experts, cfg->top_k,
                                   cfg->shared_d_ff > 0, cfg->dtype, y_rows, inv, offsets, y, st));
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK) return 0;
  return layout(cfg).total;
}

moe_status moe_route(const moe_config* cfg, const void* x, const float* Wg, const float* bg,
                     int32_t* topk_idx, float* topk_w, float* probs, float* mean_prob,
                     float* balance, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (expert_choice(cfg)) return MOE_ERR_UNSUPPORTED;
  if (cfg->T > 0 && (!x || !Wg || !topk_idx || !topk_w)) return MOE_ERR_INVALID_ARG;
  if (cfg->T > 0 && (!aligned16(x) || !aligned16(Wg))) return MOE_ERR_INVALID_ARG;
  const Layout L = layout(cfg);
  if ((s = check_ws(L, ws, ws_bytes)) != MOE_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(launch_router(L.rp, x, cfg->dtype, Wg, bg, reinterpret_cast<float*>(at(ws, L.part)),
                                  topk_idx, topk_w, probs, reinterpret_cast<double*>(at(ws, L.stat)),
                                  reinterpret_cast<int32_t*>(at(ws, L.hist)), mean_prob, balance, st));
}

moe_status moe_dispatch(const moe_config* cfg, const int32_t* topk_idx, int32_t* counts,
                        int32_t* kept, int32_t* offsets, int32_t* row_token, int32_t* row_slot,
                        int32_t* inv, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (expert_choice(cfg)) return MOE_ERR_UNSUPPORTED;
  if (!counts || !kept || !offsets) return MOE_ERR_INVALID_ARG;
  if (cfg->T > 0 && (!topk_idx || !row_token || !row_slot || !inv)) return MOE_ERR_INVALID_ARG;
  const Layout L = layout(cfg);
  if ((s = check_ws(L, ws, ws_bytes)) != MOE_OK) return s;
  return hip_status(launch_dispatch(cfg->T, cfg->n_experts, cfg->top_k, cfg->capacity,
                                    cfg->shared_d_ff > 0, L.rp.nb, topk_idx, true,
                                    reinterpret_cast<int32_t*>(at(ws, L.hist)),
                                    reinterpret_cast<int32_t*>(at(ws, L.base)), counts, kept,
                                    offsets, row_token, row_slot, inv, nullptr,
                                    static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_ffn(const moe_config* cfg, const void* x, const moe_weights* w,
                          const int32_t* offsets, const int32_t* row_token,
                          const int32_t* row_slot, const float* topk_w, float* y_rows, void* ws,
                          size_t ws_bytes, void* stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  if ((s = check_weights(cfg, w)) != MOE_OK) return s;
  // expert choice: one gate per routed row, no slots
  if (!offsets || (cfg->T > 0 && (!x || !row_token || !topk_w || !y_rows)) ||
      (cfg->T > 0 && !expert_choice(cfg) && !row_slot))
    return MOE_ERR_INVALID_ARG;
  if (cfg->T > 0 && !aligned16(x)) return MOE_ERR_INVALID_ARG;
  const Layout L = layout(cfg);
  if ((s = check_ws(L, ws, ws_bytes)) != MOE_OK) return s;
  if (cfg->T == 0) return MOE_OK;
  return run_ffn(cfg, L, x, w, offsets, row_token, row_slot, topk_w, y_rows, ws,
                 static_cast<hipStream_t>(stream));
}

moe_status moe_combine(const moe_config* cfg, const float* y_rows, const int32_t* inv,
                       const int32_t* offsets, void* y, void* stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  if (expert_choice(cfg)) return MOE_ERR_UNSUPPORTED;
  if (cfg->T > 0 && (!y_rows || !inv || !offsets || !y)) return MOE_ERR_INVALID_ARG;
  if (cfg->T > 0 && (!aligned16(y_rows) || !aligned16(y))) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(cfg->T, cfg->d_model, cfg->n_experts, cfg->top_k,
                                   cfg->shared_d_ff > 0, cfg->dtype, y_rows, inv, offsets, y,
                                   static_cast<hipStream_t>(stream)));
}

moe_status moe_forward(const moe_config* cfg, const moe_weights* w, const void* x, void* y,
                       moe_stats* stats, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  if ((s = check_weights(cfg, w)) != MOE_OK) return s;
  if (cfg->T > 0 && (!x || !y || !aligned16(x) || !aligned16(y))) return MOE_ERR_INVALID_ARG;
  const Layout L = layout(cfg);
  if ((s = check_ws(L, ws, ws_bytes)) != MOE_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  moe_stats none{};
  const moe_stats& o = stats ? *stats : none;
  if (expert_choice(cfg)) {
    if (o.topk_idx || o.topk_w) return MOE_ERR_INVALID_ARG;
    return forward_expert_choice(cfg, L, w, x, y, o, ws, st);
  }
  if (o.ec_idx || o.ec_w) return MOE_ERR_INVALID_ARG;
  return forward_token(cfg, L, w, x, y, o, ws, st);
}

size_t moe_train_workspace_bytes(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK) return 0;
  return layout(cfg, true).total;
}

moe_status moe_forward_train(const moe_config* cfg, const moe_weights* w, const void* x, void* y,
                             moe_stats* stats, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  if ((s = check_weights(cfg, w)) != MOE_OK) return s;
  if (cfg->T > 0 && (!x || !y || !aligned16(x) || !aligned16(y))) return MOE_ERR_INVALID_ARG;
  const Layout L = layout(cfg, true);
  if ((s = check_ws(L, ws, ws_bytes)) != MOE_OK) return s;
  moe_stats none{};
  const moe_stats& o = stats ? *stats : none;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (expert_choice(cfg)) {
    if (o.topk_idx || o.topk_w) return MOE_ERR_INVALID_ARG;
    return forward_expert_choice(cfg, L, w, x, y, o, ws, st);
  }
  if (o.ec_idx || o.ec_w) return MOE_ERR_INVALID_ARG;
  return forward_token(cfg, L, w, x, y, o, ws, st);
}

moe_status moe_backward(const moe_config* cfg, const moe_weights* w, const void* x,
                        const void* dy, float aux_coef, moe_grads* grads, void* ws,
                        size_t ws_bytes, void* stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  if ((s = check_weights(cfg, w)) != MOE_OK) return s;
  if (!grads) return MOE_ERR_INVALID_ARG;
  const moe_grads& g = *grads;
  if (cfg->T > 0 && (!x || !dy || !aligned16(x) || !aligned16(dy))) return MOE_ERR_INVALID_ARG;
  if ((g.dx && !aligned16(g.dx)) || (g.dW1 && !aligned16(g.dW1)) ||
      (g.dW2 && !aligned16(g.dW2)) || (g.dWs1 && !aligned16(g.dWs1)) ||
      (g.dWs2 && !aligned16(g.dWs2)))
    return MOE_ERR_INVALID_ARG;
  if (cfg->shared_d_ff == 0 && (g.dWs1 || g.dbs1 || g.dWs2 || g.dbs2)) return MOE_ERR_INVALID_ARG;
  if (!(aux_coef == aux_coef)) return MOE_ERR_INVALID_ARG;  // NaN
  const Layout L = layout(cfg, true);
  if ((s = check_ws(L, ws, ws_bytes)) != MOE_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t T = cfg->T, d = cfg->d_model, F = cfg->d_ff, E = cfg->n_experts;
  const int64_t Fs = cfg->shared_d_ff;
  const size_t elt = cfg->dtype == MOE_BF16 ? 2 : 4;
  if (T == 0) {  // no tokens: every parameter gradient is zero
    // (every size is a whole number of 4-byte words: d, F and Fs are multiples of 8)
    const size_t e = static_cast<size_t>(E), dd = static_cast<size_t>(d);
    const size_t ff = static_cast<size_t>(F), fs = static_cast<size_t>(Fs);
    const struct {
      void* p;
      size_t n;
    } z[] = {{g.dWg, 4 * e * dd},        {g.dbg, 4 * e},         {g.dW1, elt * e * ff * dd},
             {g.db1, elt * e * ff},       {g.dW2, elt * e * dd * ff}, {g.db2, elt * e * dd},
             {g.dWs1, elt * fs * dd},     {g.dbs1, elt * fs},     {g.dWs2, elt * dd * fs},
             {g.dbs2, fs > 0 ? elt * dd : 0}};
    for (const auto& q : z)
      if (q.p && q.n && (s = hip_status(launch_zero(q.p, q.n, st))) != MOE_OK) return s;
    return MOE_OK;
  }
  BwdArgs b{};
  b.rows_avg = routed_rows_max(cfg) / std::max(1, cfg->n_experts);
  b.T = T;
  b.d = cfg->d_model;
  b.F = cfg->d_ff;
  b.E = cfg->n_experts;
  b.k = cfg->top_k;
  b.Fs = cfg->shared_d_ff;
  b.dtype = cfg->dtype;
  b.renorm = cfg->renormalize;
  b.nb = L.rp.nb;
  b.alpha = aux_coef;
  b.x = x;
  b.dy = dy;
  b.Wg = w->Wg;
  b.probs = reinterpret_cast<const float*>(at(ws, L.probs));
  b.ec = expert_choice(cfg) ? 1 : 0;
  b.Ce = static_cast<int>(L.ec_C);
  b.W = L.ec_W;
  b.sel = reinterpret_cast<const uint32_t*>(at(ws, L.sel));
  b.pre = reinterpret_cast<const int32_t*>(at(ws, L.pre));
  b.probsT = reinterpret_cast<const float*>(at(ws, L.probsT));
  b.topk_idx = reinterpret_cast<const int32_t*>(at(ws, L.topk_idx));
  b.topk_w = reinterpret_cast<const float*>(at(ws, L.topk_w));
  b.inv = reinterpret_cast<const int32_t*>(at(ws, L.inv));
  b.offsets = reinterpret_cast<const int32_t*>(at(ws, L.offsets));
  b.row_token = reinterpret_cast<const int32_t*>(at(ws, L.row_token));
  b.row_gate = reinterpret_cast<const float*>(at(ws, L.row_gate));
  b.stat_part = reinterpret_cast<const double*>(at(ws, L.stat));
  b.y_rows = reinterpret_cast<const float*>(at(ws, L.y_rows));
  b.dg = reinterpret_cast<float*>(at(ws, L.dg));
  b.dl = reinterpret_cast<float*>(at(ws, L.dl));
  b.aux_dp = reinterpret_cast<float*>(at(ws, L.aux_dp));
  b.wg_part = reinterpret_cast<float*>(at(ws, L.wg_part));
  b.wg_split = L.wg_split;
  b.wg_chunk = L.wg_chunk;
  b.dX = reinterpret_cast<const float*>(at(ws, L.y_rows));
  b.Z = at(ws, L.Z);
  b.H = at(ws, L.H);
  b.poff = reinterpret_cast<int32_t*>(at(ws, L.poff));
  b.Rp = L.Rp;
  b.ZT = at(ws, L.ZT);
  b.HT = at(ws, L.HT);
  b.XT = at(ws, L.XT);
  b.DT = at(ws, L.DT);
  b.bsum = reinterpret_cast<float*>(at(ws, L.bsum));
  b.dx = g.dx;
  b.dWg = g.dWg;
  b.dbg = g.dbg;
  b.dW1 = g.dW1;
  b.db1 = g.db1;
  b.dW2 = g.dW2;
  b.db2 = g.db2;
  b.dWs1 = g.dWs1;
  b.dbs1 = g.dbs1;
  b.dWs2 = g.dWs2;
  b.dbs2 = g.dbs2;
  // gate gradients read the forward's expert rows before the dgrad pass reuses them
  if ((s = hip_status(launch_backward(b, kBwdRouter, st))) != MOE_OK) return s;
  // input-gradient pass: dz (in place of z) and dz W1 per row (in place of y_rows)
  FfnArgs f{};
  f.T = T;
  f.d = cfg->d_model;
  f.F = cfg->d_ff;
  f.E = cfg->n_experts;
  f.k = cfg->top_k;
  f.Fs = cfg->shared_d_ff;
  f.act = cfg->act;
  f.dtype = cfg->dtype;
  f.x = dy;
  f.W1 = w->W2;  // read as [K = d, N = F]
  f.W2 = w->W1;  // read as [K = F, N = d]
  f.Ws1 = w->Ws2;
  f.Ws2 = w->Ws1;
  f.offsets = b.offsets;
  f.row_token = b.row_token;
  f.H = at(ws, L.Z);
  f.y_rows = reinterpret_cast<float*>(at(ws, L.y_rows));
  f.tiles = reinterpret_cast<RowTile*>(at(ws, L.tiles));
  f.ntiles = reinterpret_cast<int32_t*>(at(ws, L.ntiles));
  f.row_gate = reinterpret_cast<float*>(at(ws, L.row_gate));
  f.tiles_ready = 1;
  f.pass = kPassDgrad;
  f.kpart = L.gp.kpart_floats ? reinterpret_cast<float*>(at(ws, L.kpart)) : nullptr;
  f.ksem = f.ntiles + 1;
  if ((s = hip_status(launch_ffn(L.gp, f, st))) != MOE_OK) return s;
  if (g.dx && (s = hip_status(launch_backward(b, kBwdDx, st))) != MOE_OK) return s;
  if (g.dW1 || g.db1 || g.dW2 || g.db2 || g.dWs1 || g.dbs1 || g.dWs2 || g.dbs2)
    s = hip_status(launch_backward(b, kBwdExpertWeights, st));
  return s;
}

moe_status moe_forward_noalloc(const moe_config* cfg, const moe_weights* w, const void* x,
                               void* y, moe_stats* stats, void* stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  const size_t need = layout(cfg).total;
  if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  void* ws = nullptr;
  if ((s = noalloc_scratch(&ws)) != MOE_OK) return s;
  return moe_forward(cfg, w, x, y, stats, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_SCRATCH:
      return "moe_forward_noalloc: the layer needs more workspace than its static scratch "
             "(MOE_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

}  // extern "C"
