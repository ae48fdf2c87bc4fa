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
// Scores.  Block = 4 waves; tile = 64 tokens x 64 experts over one K chunk.
// Each wave owns 16 tokens and all 64 experts of the tile: 4 fp32 MFMA
// 16x16x4 accumulators.  Partial sums of chunk s go to part[s][T][E]; the gate
// kernel adds the chunks in order s = 0, 1, ... so the result is deterministic.
// ---------------------------------------------------------------------------
constexpr int kRtM = 64, kRtE = 64, kRtK = 32;

template <typename XT>
__global__ __launch_bounds__(256) void router_scores_kernel(const XT* __restrict__ x,
                                                            const float* __restrict__ Wg,
                                                            int64_t T, int d, int E, int kchunk,
                                                            float* __restrict__ part) {
  __shared__ float xs[kRtM][kRtK + 1];
  __shared__ float ws[kRtE][kRtK + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRtM;
  const int e0 = blockIdx.y * kRtE;
  const int s = blockIdx.z;
  const int kb = s * kchunk;
  const int ke = min(d, kb + kchunk);
  f32x4 acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = kb; k0 < ke; k0 += kRtK) {
#pragma unroll
    for (int i = tid; i < kRtM * kRtK; i += 256) {
      const int r = i / kRtK, c = i % kRtK;
      const int k = k0 + c;
      const int64_t t = t0 + r;
      xs[r][c] = (t < T && k < ke) ? to_f32(x[t * d + k]) : 0.f;
      const int e = e0 + r;
      ws[r][c] = (e < E && k < ke) ? Wg[static_cast<int64_t>(e) * d + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kRtK; kk += 4) {
      const float a = xs[wave * 16 + (lane & 15)][kk + (lane >> 4)];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const float b = ws[n * 16 + (lane & 15)][kk + (lane >> 4)];
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[n], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // acc[n][j] holds token row (lane>>4)*4 + j of the wave, expert column lane&15.
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int e = e0 + n * 16 + (lane & 15);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t t = t0 + wave * 16 + (lane >> 4) * 4 + j;
      if (t < T && e < E) part[(static_cast<int64_t>(s) * T + t) * E + e] = acc[n][j];
    }
  }
}

// ---------------------------------------------------------------------------
// Gate.  One block handles kGateTokens tokens with 4 waves of 16 tokens each.
// A token's E scores are spread over LPT lanes (LPT = min(64, next pow2 of E)),
// VPL values per lane, expert e = s + v * LPT for lane sub-index s.  Max, sum,
// and each of the k argmax rounds are xor-shuffle trees inside the LPT group,
// so every lane of the group ends with identical values.  Ties pick the lower
// expert index.  Per-block sums of the probabilities (fp64) and the count of
// (token, slot) pairs per expert are reduced in a fixed order: no atomics.
// ---------------------------------------------------------------------------
template <int VPL>
__global__ __launch_bounds__(256) void router_gate_kernel(
    const float* __restrict__ part, int S, const float* __restrict__ bg, int64_t T, int E, int k,
    int renorm, int lpt, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ probs, double* __restrict__ stat_part, int32_t* __restrict__ hist) {
  __shared__ double red_d[4][kMaxExperts];
  __shared__ int32_t red_i[4][kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = lane & (lpt - 1);
  const int grp = lane / lpt;
  const int tpw = kWave / lpt;  // tokens per wave step
  const int64_t blk = blockIdx.x;

  double sacc[VPL];
  int cnt[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    sacc[v] = 0.0;
    cnt[v] = 0;
  }

  const int iters = (16 + tpw - 1) / tpw;  // each wave owns 16 tokens
  for (int it = 0; it < iters; ++it) {
    const int local = it * tpw + grp;
    const int64_t t = blk * kGateTokens + wave * 16 + local;
    const bool vt = local < 16 && t < T;
    float l[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = s + v * lpt;
      float z = -INFINITY;
      if (vt && e < E) {
        z = part[t * E + e];
        for (int sp = 1; sp < S; ++sp) z += part[(static_cast<int64_t>(sp) * T + t) * E + e];
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
    float selp[kMaxTopK];
    int sele[kMaxTopK];
#pragma unroll
    for (int i = 0; i < kMaxTopK; ++i) {
      if (i < k) {
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
            if (vv == v) {
              taken |= 1u << vv;
              if (vt) cnt[vv] += 1;
            }
        }
        const float p = expf(bv - m) / sum;  // same value the owner lane computed
        selp[i] = p;
        sele[i] = be;
        selsum += p;
      }
    }
    if (vt && s == 0) {
#pragma unroll
      for (int i = 0; i < kMaxTopK; ++i)
        if (i < k) {
          topk_idx[t * k + i] = sele[i];
          topk_w[t * k + i] = renorm ? selp[i] / selsum : selp[i];
        }
    }
  }

  // reduce across the token groups of the wave (lanes with the same s)
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    for (int o = lpt; o < kWave; o <<= 1) {
      sacc[v] += __shfl_xor(sacc[v], o);
      cnt[v] += __shfl_xor(cnt[v], o);
    }
  }
  if (grp == 0) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = s + v * lpt;
      if (e < E) {
        red_d[wave][e] = sacc[v];
        red_i[wave][e] = cnt[v];
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    stat_part[blk * E + e] = ((red_d[0][e] + red_d[1][e]) + red_d[2][e]) + red_d[3][e];
    hist[blk * E + e] = red_i[0][e] + red_i[1][e] + red_i[2][e] + red_i[3][e];
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
    dim3 g1(static_cast<unsigned>(ceil_div(p.T, kRtM)), static_cast<unsigned>(ceil_div(p.E, kRtE)),
            static_cast<unsigned>(p.S));
    if (dtype == MOE_BF16)
      router_scores_kernel<bf16><<<g1, 256, 0, st>>>(static_cast<const bf16*>(x), Wg, p.T, p.d, p.E,
                                                     p.kchunk, part);
    else
      router_scores_kernel<float><<<g1, 256, 0, st>>>(static_cast<const float*>(x), Wg, p.T, p.d,
                                                      p.E, p.kchunk, part);
    const unsigned nb = static_cast<unsigned>(p.nb);
#define MOE_GATE(V)                                                                            \
  router_gate_kernel<V><<<nb, 256, 0, st>>>(part, p.S, bg, p.T, p.E, p.k, p.renorm, p.lpt,     \
                                            topk_idx, topk_w, probs, stat_part, hist)
    switch (p.vpl) {
      case 1: MOE_GATE(1); break;
      case 2: MOE_GATE(2); break;
      case 4: MOE_GATE(4); break;
      case 8: MOE_GATE(8); break;
      default: MOE_GATE(16); break;
    }
#undef MOE_GATE
  }
  if (mean_prob || balance)
    router_stats_kernel<<<1, 1024, 0, st>>>(stat_part, p.nb, p.E, p.T, mean_prob, balance);
  return hipGetLastError();
}

}  // namespace moe
