// Router: scores l = x W_g^T (+ b_g) in fp32, then softmax, top-k and
// renormalisation per token, plus the per-block partial sums the load
// statistics and the dispatch histogram are built from.
//
// Pages: botmartz "Mixture of Experts (MoE) and Mixtral", "Expert Routing"
// (router nn.Linear, softmax, topk, renormalise); roadtointelligence "Mixture
// of Experts", router formula Softmax(TopK(x W_g)) and "Tiny example";
// botmartz "Load Balancing" (mean router probability per expert).
#include "kernels.h"

namespace moe {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Scores.  Block = 4 waves; tile = 64 tokens x TE experts (TE = 16 or 64) over
// one K chunk.  Each wave owns 16 tokens and all TE experts of the tile
// (TE / 16 fp32 MFMA 16x16x4 accumulators).  The next K step is loaded into
// registers while the current one is multiplied.  Partial sums of chunk s go
// to part[s][T][E]; the gate kernel adds the chunks in order s = 0, 1, ...
// so the result is deterministic.
// ---------------------------------------------------------------------------
constexpr int kRtM = 64, kRtK = 32;

template <typename XT>
struct XLoad;
template <>
struct XLoad<bf16> {  // 8 bf16 per 16-byte chunk, 4 chunks per 32-wide row
  static constexpr int kPer = 8;
};
template <>
struct XLoad<float> {  // 4 floats per chunk, 8 chunks per row
  static constexpr int kPer = 4;
};

template <typename XT, int TE>
__global__ __launch_bounds__(256) void router_scores_kernel(const XT* __restrict__ x,
                                                            const float* __restrict__ Wg,
                                                            int64_t T, int d, int E, int kchunk,
                                                            float* __restrict__ part) {
  constexpr int XP = XLoad<XT>::kPer;
  constexpr int XCH = kRtM * kRtK / XP;  // x chunks per stage
  constexpr int WCH = TE * kRtK / 4;     // W chunks (float4) per stage
  constexpr int XPT = (XCH + 255) / 256, WPT = (WCH + 255) / 256;
  constexpr int NB = TE / 16;
  __shared__ float xs[kRtM][kRtK + 1];
  __shared__ float ws[TE][kRtK + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRtM;
  const int e0 = blockIdx.y * TE;
  const int s = blockIdx.z;
  const int kb = s * kchunk;
  const int ke = min(d, kb + kchunk);

  float xr[XPT][XP];
  float wr[WPT][4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int c = tid + i * 256;
      const int r = c / (kRtK / XP), kc = (c % (kRtK / XP)) * XP;
      const int64_t t = t0 + r;
      const int k = k0 + kc;
      const bool ok = c < XCH && t < T && k < ke;  // ke and k are multiples of 8
      if constexpr (XP == 8) {
        uint4 u = ok ? *reinterpret_cast<const uint4*>(x + t * d + k) : make_uint4(0, 0, 0, 0);
        const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          xr[i][2 * q] = __uint_as_float(w4[q] << 16);
          xr[i][2 * q + 1] = __uint_as_float(w4[q] & 0xffff0000u);
        }
      } else {
        float4 f = ok ? *reinterpret_cast<const float4*>(x + t * d + k) : make_float4(0, 0, 0, 0);
        xr[i][0] = f.x;
        xr[i][1] = f.y;
        xr[i][2] = f.z;
        xr[i][3] = f.w;
      }
    }
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int c = tid + i * 256;
      const int r = c / (kRtK / 4), kc = (c % (kRtK / 4)) * 4;
      const int e = e0 + r;
      const int k = k0 + kc;
      const bool ok = c < WCH && e < E && k < ke;
      float4 f = ok ? *reinterpret_cast<const float4*>(Wg + static_cast<int64_t>(e) * d + k)
                    : make_float4(0, 0, 0, 0);
      wr[i][0] = f.x;
      wr[i][1] = f.y;
      wr[i][2] = f.z;
      wr[i][3] = f.w;
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int c = tid + i * 256;
      if (c < XCH) {
        const int r = c / (kRtK / XP), kc = (c % (kRtK / XP)) * XP;
#pragma unroll
        for (int q = 0; q < XP; ++q) xs[r][kc + q] = xr[i][q];
      }
    }
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int c = tid + i * 256;
      if (c < WCH) {
        const int r = c / (kRtK / 4), kc = (c % (kRtK / 4)) * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) ws[r][kc + q] = wr[i][q];
      }
    }
  };

  f32x4 acc[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  gload(kb);
  for (int k0 = kb; k0 < ke; k0 += kRtK) {
    __syncthreads();
    sstore();
    __syncthreads();
    if (k0 + kRtK < ke) gload(k0 + kRtK);
#pragma unroll
    for (int kk = 0; kk < kRtK; kk += 4) {
      const float a = xs[wave * 16 + (lane & 15)][kk + (lane >> 4)];
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const float b = ws[n * 16 + (lane & 15)][kk + (lane >> 4)];
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[n], 0, 0, 0);
      }
    }
  }
  // acc[n][j] holds token row (lane>>4)*4 + j of the wave, expert column lane&15.
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const int e = e0 + n * 16 + (lane & 15);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t t = t0 + wave * 16 + (lane >> 4) * 4 + j;
      if (t < T && e < E) part[(static_cast<int64_t>(s) * T + t) * E + e] = acc[n][j];
    }
  }
}

// ---------------------------------------------------------------------------
// Gate.  One block handles kGateTokens tokens with 8 waves of 8 tokens each.
// A token's E scores are spread over LPT lanes (LPT = min(64, next pow2 of E)),
// VPL values per lane, expert e = s + v * LPT for lane sub-index s.  Max, sum,
// and each of the k argmax rounds are xor-shuffle trees inside the LPT group,
// so every lane of the group ends with identical values.  Ties pick the lower
// expert index.  Per-block sums of the probabilities (fp64) are reduced in a
// fixed order; the per-block count of (token, slot) pairs per expert uses LDS
// integer atomics, whose result does not depend on their order.
// ---------------------------------------------------------------------------
// Sum of the score chunks in chunk order, written over chunk 0.
__global__ __launch_bounds__(256) void router_reduce_kernel(float* __restrict__ part, int S,
                                                            int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  float z = part[i];
  for (int sp = 1; sp < S; ++sp) z += part[static_cast<int64_t>(sp) * n + i];
  part[i] = z;
}

template <int VPL, int kGateWaves>
__global__ __launch_bounds__(kGateWaves * 64) void router_gate_kernel(
    const float* __restrict__ logit, const float* __restrict__ bg, int64_t T, int E, int k,
    int renorm, int lpt, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ probs, double* __restrict__ stat_part, int32_t* __restrict__ hist) {
  constexpr int kGateTPW = kGateTokens / kGateWaves;  // tokens per wave
  __shared__ double red_d[4][kMaxExperts];
  __shared__ int32_t hcnt[kMaxExperts];
  __shared__ float selp_s[kGateWaves][64];
  __shared__ int32_t sele_s[kGateWaves][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = lane & (lpt - 1);
  const int grp = lane / lpt;
  const int tpw = kWave / lpt;  // tokens per wave step
  const int64_t blk = blockIdx.x;
  for (int e = tid; e < E; e += kGateWaves * 64) hcnt[e] = 0;
  __syncthreads();

  double sacc[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) sacc[v] = 0.0;

  const int iters = (kGateTPW + tpw - 1) / tpw;
  for (int it = 0; it < iters; ++it) {
    const int local = it * tpw + grp;
    const int64_t t = blk * kGateTokens + wave * kGateTPW + local;
    const bool vt = local < kGateTPW && t < T;
    float l[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = s + v * lpt;
      float z = -INFINITY;
      if (vt && e < E) {
        z = logit[t * E + e];
        if (bg) z += bg[e];
      }
      l[v] = z;
    }
    float m = l[0];
#pragma unroll
    for (int v = 1; v < VPL; ++v) m = fmaxf(m, l[v]);
    for (int o = lpt >> 1; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    float pz[VPL];
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      pz[v] = (l[v] == -INFINITY) ? 0.f : expf(l[v] - m);
      sum += pz[v];
    }
    for (int o = lpt >> 1; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = s + v * lpt;
      const float p = pz[v] / sum;
      if (vt && e < E) {
        if (probs) probs[t * E + e] = p;
        sacc[v] += static_cast<double>(p);
      }
    }

    // top-k: k rounds of a group argmax over the not-yet-taken experts
    uint32_t taken = 0;
    float selsum = 0.f;
    for (int i = 0; i < k; ++i) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int e = s + v * lpt;
        if (e < E && !((taken >> v) & 1u) && (l[v] > bv || (l[v] == bv && e < be))) {
          bv = l[v];
          be = e;
        }
      }
      for (int o = lpt >> 1; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oe = __shfl_xor(be, o);
        if (ov > bv || (ov == bv && oe < be)) {
          bv = ov;
          be = oe;
        }
      }
      if ((be & (lpt - 1)) == s) {
        const int v = be / lpt;
#pragma unroll
        for (int vv = 0; vv < VPL; ++vv)
          if (vv == v) taken |= 1u << vv;
        if (vt) atomicAdd(&hcnt[be], 1);
      }
      const float p = expf(bv - m) / sum;  // same value the owner lane computed
      selsum += p;
      if (s == 0) {
        selp_s[wave][grp * k + i] = p;
        sele_s[wave][grp * k + i] = be;
      }
    }
    __syncthreads();
    if (vt && s < k) {
      const float p = selp_s[wave][grp * k + s];
      topk_idx[t * k + s] = sele_s[wave][grp * k + s];
      topk_w[t * k + s] = renorm ? p / selsum : p;
    }
    __syncthreads();
  }

  // reduce across the token groups of the wave (lanes with the same s), then
  // across waves in a fixed order: slot w % 4 accumulates waves w % 4, w % 4 + 4,
  // ... in wave order, then the four slots are added in order
#pragma unroll
  for (int v = 0; v < VPL; ++v)
    for (int o = lpt; o < kWave; o <<= 1) sacc[v] += __shfl_xor(sacc[v], o);
  for (int half = 0; half < kGateWaves / 4; ++half) {
    if (grp == 0 && (wave >> 2) == half) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int e = s + v * lpt;
        if (e < E) red_d[wave & 3][e] = half ? red_d[wave & 3][e] + sacc[v] : sacc[v];
      }
    }
    __syncthreads();
  }
  for (int e = tid; e < E; e += kGateWaves * 64) {
    stat_part[blk * E + e] = ((red_d[0][e] + red_d[1][e]) + red_d[2][e]) + red_d[3][e];
    hist[blk * E + e] = hcnt[e];
  }
}

// mean_prob[e] = (sum over blocks, in block order) / T; balance = unbiased
// variance of mean_prob over experts.  fp64 inside, fp32 out.
__global__ __launch_bounds__(1024) void router_stats_kernel(const double* __restrict__ stat_part,
                                                            int nb, int E, int64_t T,
                                                            float* __restrict__ mean_prob,
                                                            float* __restrict__ balance) {
  __shared__ double mp[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    double acc = 0.0;
    for (int b = 0; b < nb; ++b) acc += stat_part[static_cast<int64_t>(b) * E + e];
    const double v = acc / static_cast<double>(T);  // T = 0 gives NaN
    mp[e] = v;
    if (mean_prob) mean_prob[e] = static_cast<float>(v);
  }
  __syncthreads();
  if (threadIdx.x == 0 && balance) {
    double mean = 0.0;
    for (int e = 0; e < E; ++e) mean += mp[e];
    mean /= static_cast<double>(E);
    double var = 0.0;
    for (int e = 0; e < E; ++e) var += (mp[e] - mean) * (mp[e] - mean);
    balance[0] = static_cast<float>(var / static_cast<double>(E - 1));  // E = 1 gives NaN
  }
}

// ------------------------------------------------------------------ launches
hipError_t launch_router(const RoutePlan& p, const void* x, int dtype, const float* Wg,
                         const float* bg, float* part, int32_t* topk_idx, float* topk_w,
                         float* probs, double* stat_part, int32_t* hist, float* mean_prob,
                         float* balance, hipStream_t st) {
  if (p.T > 0) {
    const int TE = p.E <= 16 ? 16 : 64;
    dim3 g1(static_cast<unsigned>(ceil_div(p.T, kRtM)), static_cast<unsigned>(ceil_div(p.E, TE)),
            static_cast<unsigned>(p.S));
#define MOE_SCORES(XT, TEV)                                                                  \
  router_scores_kernel<XT, TEV><<<g1, 256, 0, st>>>(static_cast<const XT*>(x), Wg, p.T, p.d, \
                                                    p.E, p.kchunk, part)
    if (dtype == MOE_BF16) {
      if (TE == 16) MOE_SCORES(bf16, 16); else MOE_SCORES(bf16, 64);
    } else {
      if (TE == 16) MOE_SCORES(float, 16); else MOE_SCORES(float, 64);
    }
#undef MOE_SCORES
    const unsigned nb = static_cast<unsigned>(p.nb);
    if (p.S > 1) {
      const int64_t n = p.T * p.E;
      router_reduce_kernel<<<static_cast<unsigned>(ceil_div(n, 256)), 256, 0, st>>>(part, p.S, n);
    }
#define MOE_GATE(V, W)                                                                      \
  router_gate_kernel<V, W><<<nb, W * 64, 0, st>>>(part, bg, p.T, p.E, p.k, p.renorm, p.lpt, \
                                                  topk_idx, topk_w, probs, stat_part, hist)
    switch (p.vpl) {
      case 1: MOE_GATE(1, 16); break;
      case 2: MOE_GATE(2, 16); break;
      case 4: MOE_GATE(4, 16); break;
      case 8: MOE_GATE(8, 8); break;
      default: MOE_GATE(16, 8); break;
    }
#undef MOE_GATE
  }
  if (mean_prob || balance)
    router_stats_kernel<<<1, 1024, 0, st>>>(stat_part, p.nb, p.E, p.T, mean_prob, balance);
  return hipGetLastError();
}

}  // namespace moe
