// Router: scores l = x W_g^T (+ b_g) in fp32, then softmax, top-k and
// renormalisation per token, plus the per-block partial sums the load
// statistics and the dispatch histogram are built from.
//
// Pages: botmartz "Mixture of Experts (MoE) and Mixtral", "Expert Routing"
// (router nn.Linear, softmax, topk, renormalise); roadtointelligence "Mixture
// of Experts", router formula Softmax(TopK(x W_g)) and "Tiny example";
// botmartz "Load Balancing" (mean router probability per expert).
#include "kernels.h"
#include "router_tile.h"
#include "block_ops.h"

namespace moe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kRtM = 64, kRtK = 32;
constexpr int kRw = 16;  // waves per block of the bf16 score kernel and of the gate

// ---------------------------------------------------------------------------
// Butterfly exchange inside a group of lanes.  Levels 1 and 2 swap lanes of a
// quad, levels 4 and 8 mirror a half row / a row (DPP, no LDS traffic); 16 and
// 32 cross rows.  For an all-reduce with a commutative combine, a mirror
// partner is as good as the xor partner: after the previous levels every lane
// of the smaller group already holds that group's result.
// ---------------------------------------------------------------------------
template <int O>
__device__ __forceinline__ int xchg(int v) {
  if constexpr (O == 1) return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  else if constexpr (O == 2) return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  else if constexpr (O == 4) return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
  else if constexpr (O == 8) return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
  else return __shfl_xor(v, O);
}
template <int O>
__device__ __forceinline__ float xchg(float v) {
  return __int_as_float(xchg<O>(__float_as_int(v)));
}

template <int LPT, int O = 1>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (O < LPT) return group_max<LPT, O * 2>(fmaxf(v, xchg<O>(v)));
  else return v;
}
template <int LPT, int O = 1>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (O < LPT) return group_sum<LPT, O * 2>(v + xchg<O>(v));
  else return v;
}
// larger value wins; equal values go to the lower expert index
template <int LPT, int O = 1>
__device__ __forceinline__ void group_argmax(float& bv, int& be) {
  if constexpr (O < LPT) {
    const float ov = xchg<O>(bv);
    const int oe = xchg<O>(be);
    if (ov > bv || (ov == bv && oe < be)) {
      bv = ov;
      be = oe;
    }
    group_argmax<LPT, O * 2>(bv, be);
  }
}

// ---------------------------------------------------------------------------
// Gate of one block of kGateTokens tokens, kRw waves of kGateTokens / kRw
// tokens.  A token's E scores are spread over LPT lanes (16, or 64 for E > 256),
// VPL consecutive experts per lane: lane sub-index s holds experts s * VPL + v,
// so the scores of a lane load as vectors.  Max, sum and each of the k argmax
// rounds are all-reduces inside the LPT group, so every lane of the group ends
// with identical values and lane s keeps the selections of rounds s, s + LPT,
// ...  Ties pick the lower expert index.  Per-block sums of the probabilities
// (fp64) are reduced in a fixed order; the per-block count of (token, slot)
// pairs per expert uses LDS integer atomics, whose result does not depend on
// their order.  `load(tl, e0, l)` fills l[v] with the raw score (bias excluded)
// of local token tl and expert e0 + v (entries past E are ignored).
// ---------------------------------------------------------------------------
template <int EM>
struct GateSmem {  // EM: largest expert count the block handles
  double red_d[4][EM];
  int32_t hcnt[EM];
};

template <int LPT, int VPL, int EM, class Load>
__device__ __forceinline__ void gate_block(Load load, GateSmem<EM>& sm, int64_t blk,
                                           const float* __restrict__ bg, int64_t T, int E,
                                           int k, int renorm, int32_t* __restrict__ topk_idx,
                                           float* __restrict__ topk_w, float* __restrict__ probs,
                                           int64_t ps_t, int64_t ps_e,
                                           double* __restrict__ stat_part,
                                           int32_t* __restrict__ hist) {
  constexpr int TPW = kGateTokens / kRw;  // tokens per wave
  constexpr int TPS = kWave / LPT;        // tokens per wave step
  constexpr int ITERS = (TPW + TPS - 1) / TPS;
  constexpr int NSL = (kMaxTopK + LPT - 1) / LPT;  // output slots per lane
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = lane & (LPT - 1);
  const int grp = lane / LPT;
  const int e0 = s * VPL;
  for (int e = tid; e < E; e += kRw * 64) sm.hcnt[e] = 0;
  __syncthreads();

  double sacc[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) sacc[v] = 0.0;

#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int local = it * TPS + grp;
    const int tl = wave * TPW + local;
    const int64_t t = blk * kGateTokens + tl;
    const bool vt = local < TPW && t < T;
    float l[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) l[v] = -INFINITY;
    if (vt && e0 < E) load(tl, e0, l);
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = e0 + v;
      if (vt && e < E) {
        if (bg) l[v] += bg[e];
      } else {
        l[v] = -INFINITY;
      }
    }
    float m = l[0];
#pragma unroll
    for (int v = 1; v < VPL; ++v) m = fmaxf(m, l[v]);
    m = group_max<LPT>(m);
    float pz[VPL];
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      pz[v] = (l[v] == -INFINITY) ? 0.f : expf(l[v] - m);
      sum += pz[v];
    }
    sum = group_sum<LPT>(sum);
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = e0 + v;
      const float p = pz[v] / sum;
      if (vt && e < E) {
        if (probs) probs[t * ps_t + e * ps_e] = p;
        sacc[v] += static_cast<double>(p);
      }
    }

    // top-k: k rounds of a group argmax over the not-yet-taken experts
    uint32_t taken = 0;
    float selsum = 0.f;
    float myp[NSL];
    int mye[NSL];
#pragma unroll
    for (int j = 0; j < NSL; ++j) {
      myp[j] = 0.f;
      mye[j] = 0;
    }
    for (int i = 0; i < k; ++i) {
      float bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        // ascending v: on equal scores the lower expert stays
        if (!((taken >> v) & 1u) && l[v] > bv) {
          bv = l[v];
          be = e0 + v;
        }
      }
      group_argmax<LPT>(bv, be);
      if (be / VPL == s) {
        const int v = be % VPL;
#pragma unroll
        for (int vv = 0; vv < VPL; ++vv)
          if (vv == v) taken |= 1u << vv;
        if (vt) atomicAdd(&sm.hcnt[be], 1);
      }
      const float p = expf(bv - m) / sum;  // same value the owner lane computed
      selsum += p;
#pragma unroll
      for (int j = 0; j < NSL; ++j)
        if (i == s + j * LPT) {
          myp[j] = p;
          mye[j] = be;
        }
    }
#pragma unroll
    for (int j = 0; j < NSL; ++j) {
      const int slot = s + j * LPT;
      if (vt && slot < k) {
        topk_idx[t * k + slot] = mye[j];
        topk_w[t * k + slot] = renorm ? myp[j] / selsum : myp[j];
      }
    }
  }

  // reduce across the token groups of the wave (lanes with the same s), then
  // across waves in a fixed order: slot w % 4 accumulates waves w % 4, w % 4 + 4,
  // ... in wave order, then the slots are added in order
#pragma unroll
  for (int v = 0; v < VPL; ++v)
    for (int o = LPT; o < kWave; o <<= 1) sacc[v] += __shfl_xor(sacc[v], o);
  for (int round = 0; round < kRw / 4; ++round) {
    if (grp == 0 && (wave >> 2) == round) {
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int e = e0 + v;
        if (e < E) sm.red_d[wave & 3][e] = round ? sm.red_d[wave & 3][e] + sacc[v] : sacc[v];
      }
    }
    __syncthreads();
  }
  for (int e = tid; e < E; e += kRw * 64) {
    const double tot = ((sm.red_d[0][e] + sm.red_d[1][e]) + sm.red_d[2][e]) + sm.red_d[3][e];
    stat_part[blk * E + e] = tot;
    hist[blk * E + e] = sm.hcnt[e];
  }
}

// ---------------------------------------------------------------------------
// Scores, fp32 x.  Block = 4 waves; tile = 64 tokens x TE experts (TE = 16 or
// 64) over one K chunk; each wave owns 16 tokens (fp32 MFMA 16x16x4).  The
// next K step is loaded into registers while the current one is multiplied.
// Partial sums of chunk s go to part[s][T][E].
// ---------------------------------------------------------------------------
template <int TE>
__global__ __launch_bounds__(256) void router_scores_f32_kernel(const float* __restrict__ x,
                                                                const float* __restrict__ Wg,
                                                                int64_t T, int d, int E,
                                                                int kchunk,
                                                                float* __restrict__ part) {
  constexpr int XCH = kRtM * kRtK / 4;  // x float4 chunks per stage
  constexpr int WCH = TE * kRtK / 4;    // W float4 chunks per stage
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

  float4 xr[XPT], wr[WPT];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int c = tid + i * 256;
      const int r = c / (kRtK / 4), kc = (c % (kRtK / 4)) * 4;
      const int64_t t = t0 + r;
      const int kk = k0 + kc;
      xr[i] = (c < XCH && t < T && kk < ke) ? *reinterpret_cast<const float4*>(x + t * d + kk)
                                           : make_float4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int c = tid + i * 256;
      const int r = c / (kRtK / 4), kc = (c % (kRtK / 4)) * 4;
      const int e = e0 + r;
      const int kk = k0 + kc;
      wr[i] = (c < WCH && e < E && kk < ke)
                  ? *reinterpret_cast<const float4*>(Wg + static_cast<int64_t>(e) * d + kk)
                  : make_float4(0, 0, 0, 0);
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int c = tid + i * 256;
      if (c < XCH) {
        const int r = c / (kRtK / 4), kc = (c % (kRtK / 4)) * 4;
        xs[r][kc] = xr[i].x;
        xs[r][kc + 1] = xr[i].y;
        xs[r][kc + 2] = xr[i].z;
        xs[r][kc + 3] = xr[i].w;
      }
    }
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int c = tid + i * 256;
      if (c < WCH) {
        const int r = c / (kRtK / 4), kc = (c % (kRtK / 4)) * 4;
        ws[r][kc] = wr[i].x;
        ws[r][kc + 1] = wr[i].y;
        ws[r][kc + 2] = wr[i].z;
        ws[r][kc + 3] = wr[i].w;
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
// Scores, bf16 x, on bf16 MFMA with fp32 accumulation.  Each fp32 router weight
// is cut into three bf16 parts whose sum is exactly w: hi = w with the low 16
// bits cleared, mid = the same cut of r = w - hi, lo = r - mid (at most 8
// significant bits left, so it is a bf16 value; weights in the normal range).
// x is exactly bf16, so every product x * part is exact in fp32 and the score
// sum_k x w = S(hi) + S(mid + lo) is accumulated in fp32: the precision of an
// fp32 dot product.
//
// Block = 16 waves over 64 tokens x TE experts (TE = 16, 32 or 64) and one K chunk.
// Wave w takes expert block w % (TE / 16) and K slice w / (TE / 16): the chunk's
// 32-wide K steps are dealt round-robin to the slices.  A wave multiplies all
// four 16-token row blocks with its 16 experts (v_mfma_f32_16x16x32_bf16: lane l
// supplies row l % 16, k = (l / 16) * 8 + 0..7), loading its x and W fragments
// straight from global memory, two K steps in flight.  The slices' partial
// tiles are added in slice order through LDS.  With FUSE (one chunk, E <= TE)
// the gate runs in the same block on those scores; otherwise chunk s goes to
// part[s][T][E].
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t hi16x2(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);  // a.hi16 | b.hi16 << 16
}

template <int TE, bool FUSE, int LPT, int VPL>
__global__ __launch_bounds__(kRw * 64) void router_scores_bf16_kernel(
    const bf16* __restrict__ x, const float* __restrict__ Wg, const float* __restrict__ bg,
    int64_t T, int d, int E, int kchunk, float* __restrict__ part, int k, int renorm,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, float* __restrict__ probs,
    int64_t ps_t, int64_t ps_e, double* __restrict__ stat_part, int32_t* __restrict__ hist) {
  constexpr int NE = TE / 16;   // expert blocks
  constexpr int QK = kRw / NE;  // K slices
  constexpr int G = 2;          // K steps in flight per wave
  __shared__ float red[kRw][kRtM * 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int eb = wave % NE, q = wave / NE;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kRtM;
  const int e = blockIdx.y * TE + eb * 16 + (lane & 15);
  const int kb = blockIdx.z * kchunk;
  const int ke = min(d, kb + kchunk);
  const int nks = (ke - kb + 31) / 32;
  const int kl = (lane >> 4) * 8;

  const bf16* xr[4];
  bool rv[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int64_t t = t0 + rb * 16 + (lane & 15);
    rv[rb] = t < T;
    xr[rb] = x + (rv[rb] ? t : 0) * d + kl;
  }
  const bool ev = e < E;
  const float* wrow = Wg + static_cast<int64_t>(ev ? e : 0) * d + kl;

  f32x4 ah[4], al[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    ah[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    al[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int j0 = q; j0 < nks; j0 += G * QK) {
    uint4 a[G][4];
    float4 w[G][2];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int k0 = kb + (j0 + g * QK) * 32 + kl;
      const bool kv = (j0 + g * QK) < nks && k0 < ke;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        a[g][rb] = (kv && rv[rb]) ? *reinterpret_cast<const uint4*>(xr[rb] + (k0 - kl))
                                  : make_uint4(0, 0, 0, 0);
      w[g][0] = (kv && ev) ? *reinterpret_cast<const float4*>(wrow + (k0 - kl))
                           : make_float4(0, 0, 0, 0);
      w[g][1] = (kv && ev) ? *reinterpret_cast<const float4*>(wrow + (k0 - kl) + 4)
                           : make_float4(0, 0, 0, 0);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float wv[8] = {w[g][0].x, w[g][0].y, w[g][0].z, w[g][0].w,
                           w[g][1].x, w[g][1].y, w[g][1].z, w[g][1].w};
      uint32_t hb[8], mb[8], lb[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        hb[i] = __float_as_uint(wv[i]);
        const float r1 = wv[i] - __uint_as_float(hb[i] & 0xffff0000u);
        mb[i] = __float_as_uint(r1);
        lb[i] = __float_as_uint(r1 - __uint_as_float(mb[i] & 0xffff0000u));
      }
      uint4 bh, bm, bl;
      bh = make_uint4(hi16x2(hb[0], hb[1]), hi16x2(hb[2], hb[3]), hi16x2(hb[4], hb[5]),
                      hi16x2(hb[6], hb[7]));
      bm = make_uint4(hi16x2(mb[0], mb[1]), hi16x2(mb[2], mb[3]), hi16x2(mb[4], mb[5]),
                      hi16x2(mb[6], mb[7]));
      bl = make_uint4(hi16x2(lb[0], lb[1]), hi16x2(lb[2], lb[3]), hi16x2(lb[4], lb[5]),
                      hi16x2(lb[6], lb[7]));
      const bf16x8_t fh = __builtin_bit_cast(bf16x8_t, bh);
      const bf16x8_t fm = __builtin_bit_cast(bf16x8_t, bm);
      const bf16x8_t fl = __builtin_bit_cast(bf16x8_t, bl);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const bf16x8_t fa = __builtin_bit_cast(bf16x8_t, a[g][rb]);
        ah[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fh, ah[rb], 0, 0, 0);
      }
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const bf16x8_t fa = __builtin_bit_cast(bf16x8_t, a[g][rb]);
        al[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fm, al[rb], 0, 0, 0);
      }
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const bf16x8_t fa = __builtin_bit_cast(bf16x8_t, a[g][rb]);
        al[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fl, al[rb], 0, 0, 0);
      }
    }
  }
  // C layout: ah[rb][j] is token row rb*16 + (lane>>4)*4 + j, expert column lane&15
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      red[wave][(rb * 16 + (lane >> 4) * 4 + j) * 16 + (lane & 15)] = ah[rb][j] + al[rb][j];
  __syncthreads();
  // add the K slices in slice order; the sum lands in slice 0's tile
  for (int i = tid; i < NE * kRtM * 16; i += kRw * 64) {
    const int b = i / (kRtM * 16), off = i % (kRtM * 16);
    float z = red[b][off];
#pragma unroll
    for (int qq = 1; qq < QK; ++qq) z += red[b + qq * NE][off];
    red[b][off] = z;
  }
  __syncthreads();
  if constexpr (FUSE) {
    __shared__ GateSmem<TE> gsm;
    // VPL divides 16: a lane's experts sit in one 16-expert column block
    gate_block<LPT, VPL>(
        [&](int tl, int ee0, float (&l)[VPL]) {
          const float* src = &red[ee0 >> 4][tl * 16 + (ee0 & 15)];
#pragma unroll
          for (int v = 0; v < VPL; ++v) l[v] = src[v];
        },
        gsm, blockIdx.x, bg, T, E, k, renorm, topk_idx, topk_w, probs, ps_t, ps_e, stat_part,
        hist);
  } else {
    for (int i = tid; i < kRtM * TE; i += kRw * 64) {
      const int tl = i / TE, el = i % TE;
      const int64_t t = t0 + tl;
      const int ee = blockIdx.y * TE + el;
      if (t < T && ee < E)
        part[(static_cast<int64_t>(blockIdx.z) * T + t) * E + ee] =
            red[el >> 4][tl * 16 + (el & 15)];
    }
  }
}

// Gate over scores held as S chunk partials part[s][T][E]; the chunks are
// added in chunk order.
template <int LPT, int VPL>
__global__ __launch_bounds__(kRw * 64) void router_gate_kernel(
    const float* __restrict__ part, int S, const float* __restrict__ bg, int64_t T, int E, int k,
    int renorm, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ probs, int64_t ps_t, int64_t ps_e, double* __restrict__ stat_part,
    int32_t* __restrict__ hist) {
  __shared__ GateSmem<kMaxExperts> gsm;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kGateTokens;
  const int64_t n = T * E;
  gate_block<LPT, VPL>(
      [&](int tl, int ee0, float (&l)[VPL]) {
        const int64_t i = (t0 + tl) * E + ee0;
        if (VPL % 4 == 0 && (E & 3) == 0 && ee0 + VPL <= E) {
          // whole lane in range and 16-byte aligned: vector loads, chunks in order
#pragma unroll
          for (int v = 0; v < VPL; v += 4) {
            const float4 z = *reinterpret_cast<const float4*>(part + i + v);
            l[v] = z.x;
            l[v + 1] = z.y;
            l[v + 2] = z.z;
            l[v + 3] = z.w;
          }
#pragma unroll 4
          for (int sp = 1; sp < S; ++sp) {
#pragma unroll
            for (int v = 0; v < VPL; v += 4) {
              const float4 z = *reinterpret_cast<const float4*>(part + sp * n + i + v);
              l[v] += z.x;
              l[v + 1] += z.y;
              l[v + 2] += z.z;
              l[v + 3] += z.w;
            }
          }
        } else {
#pragma unroll
          for (int v = 0; v < VPL; ++v) {
            if (ee0 + v < E) {
              float z = part[i + v];
#pragma unroll 4
              for (int sp = 1; sp < S; ++sp) z += part[sp * n + i + v];
              l[v] = z;
            }
          }
        }
      },
      gsm, blockIdx.x, bg, T, E, k, renorm, topk_idx, topk_w, probs, ps_t, ps_e, stat_part, hist);
}

// Load statistics from the per-block probability sums, one block.
__global__ __launch_bounds__(1024) void router_stats_kernel(const double* __restrict__ stat_part,
                                                            int nb, int E, int64_t T,
                                                            float* __restrict__ mean_prob,
                                                            float* __restrict__ balance) {
  __shared__ double wsd[kMaxExperts / 64];
  load_stats(stat_part, nb, E, T, mean_prob, balance, wsd);
}

// ------------------------------------------------------------------ launches
// Fused score + gate kernels: TE = 16 (E <= 16), 32 (E <= 32, VPL 2) or 64 (E <= 64,
// VPL 2 or 4).
#define MOE_FUSED(TE_, VPL_)                                                                    \
  router_scores_bf16_kernel<TE_, true, 16, VPL_><<<g1, kRw * 64, 0, st>>>(                     \
      static_cast<const bf16*>(x), Wg, bg, p.T, p.d, p.E, p.kchunk, part, p.k, p.renorm,       \
      topk_idx, topk_w, probs, p.ps_t, p.ps_e, stat_part, hist)

hipError_t launch_router(const RoutePlan& p, const void* x, int dtype, const float* Wg,
                         const float* bg, float* part, int32_t* topk_idx, float* topk_w,
                         float* probs, double* stat_part, int32_t* hist, float* mean_prob,
                         float* balance, hipStream_t st) {
  if (p.T > 0) {
    const int TE = router_tile(p.E, dtype);
    dim3 g1(static_cast<unsigned>(ceil_div(p.T, kRtM)), static_cast<unsigned>(ceil_div(p.E, TE)),
            static_cast<unsigned>(p.S));
    if (p.fused) {
      // one block holds every score of its 64 tokens: the gate runs in place
      if (TE == 16) MOE_FUSED(16, 1);
      else if (TE == 32) MOE_FUSED(32, 2);
      else if (p.vpl <= 2) MOE_FUSED(64, 2);
      else MOE_FUSED(64, 4);
    } else {
      if (dtype == MOE_BF16) {
        if (TE == 16)
          router_scores_bf16_kernel<16, false, 16, 1><<<g1, kRw * 64, 0, st>>>(
              static_cast<const bf16*>(x), Wg, bg, p.T, p.d, p.E, p.kchunk, part, p.k,
              p.renorm, topk_idx, topk_w, probs, p.ps_t, p.ps_e, stat_part, hist);
        else if (TE == 32)
          router_scores_bf16_kernel<32, false, 16, 1><<<g1, kRw * 64, 0, st>>>(
              static_cast<const bf16*>(x), Wg, bg, p.T, p.d, p.E, p.kchunk, part, p.k,
              p.renorm, topk_idx, topk_w, probs, p.ps_t, p.ps_e, stat_part, hist);
        else
          router_scores_bf16_kernel<64, false, 16, 1><<<g1, kRw * 64, 0, st>>>(
              static_cast<const bf16*>(x), Wg, bg, p.T, p.d, p.E, p.kchunk, part, p.k,
              p.renorm, topk_idx, topk_w, probs, p.ps_t, p.ps_e, stat_part, hist);
      } else {
        if (TE == 16)
          router_scores_f32_kernel<16><<<g1, 256, 0, st>>>(static_cast<const float*>(x), Wg,
                                                            p.T, p.d, p.E, p.kchunk, part);
        else
          router_scores_f32_kernel<64><<<g1, 256, 0, st>>>(static_cast<const float*>(x), Wg,
                                                            p.T, p.d, p.E, p.kchunk, part);
      }
      const unsigned nb = static_cast<unsigned>(p.nb);
#define MOE_GATE(L, V)                                                                         \
  router_gate_kernel<L, V><<<nb, kRw * 64, 0, st>>>(part, p.S, bg, p.T, p.E, p.k, p.renorm,    \
                                                    topk_idx, topk_w, probs, p.ps_t, p.ps_e,     \
                                                    stat_part, hist)
      if (p.lpt == 16) {
        switch (p.vpl) {
          case 1: MOE_GATE(16, 1); break;
          case 2: MOE_GATE(16, 2); break;
          case 4: MOE_GATE(16, 4); break;
          case 8: MOE_GATE(16, 8); break;
          default: MOE_GATE(16, 16); break;
        }
      } else {
        if (p.vpl <= 8) MOE_GATE(64, 8);
        else MOE_GATE(64, 16);
      }
#undef MOE_GATE
    }
  }
  if (mean_prob || balance)
    router_stats_kernel<<<1, 1024, 0, st>>>(stat_part, p.nb, p.E, p.T, mean_prob, balance);
  return hipGetLastError();
}
#undef MOE_FUSED

}  // namespace moe
