// Backward pass of the layer: gradients of
//   L = sum_t <dy_t, y_t> + alpha * balance
// with the top-k selection and the capacity drops fixed (the training side of
// the layer: botmartz "Load Balancing: The Hidden Challenge", total loss = task
// loss + 0.01 * balance loss; roadtointelligence "Keeping the experts busy";
// matteuscruz "Load balancing").
//
// Per kept (token, slot) row r of expert e with gate g, pre-activation z and
// hidden h = act(z) (both kept by the training forward), and the shared rows
// (gate 1):
//   dz_r   = g (dy_t W2[e]) * act'(z)        input-gradient GEMM pass (gemm.hip)
//   dX_r   = dz_r W1[e]                       same pass, second GEMM
//   dx_t   = sum over t's rows of dX_r + sum_e dl[t, e] W_g[e]       dx_kernel
//   dW1[e] = sum_r dz_r^T x_t,  dW2[e] = sum_r (g dy_t)^T h_r        wgrad_kernel
//   db1[e] = sum_r dz_r,        db2[e] = sum_r g dy_t                transposes + seg_finish_kernel
//   dg     = <dy_t, o_r> = <dy_t, y_rows[r]> / g                     gate_grad_kernel
//   dp     = renormalisation backward of dg, plus the balance term,
//   dl     = p (dp - <p, dp>)                                       router_bwd_kernel
//   dW_g   = dl^T x, db_g = sum_t dl                                 router_wgrad_*
// Expert choice is the same with gates p[t, e], no renormalisation, and each
// token's rows found in the selection bitmaps (ec_router_bwd_kernel,
// ec_dx_kernel).
//
// The input-gradient pass reads the expert weights in their stored layout
// (the grouped GEMM's transposed-B path).  The weight-gradient GEMMs contract
// over an expert's rows, so their operands are transposed with each expert's
// rows padded to a multiple of 64 columns (gather_transpose_kernel; padding
// columns are zero, so every group's K is a whole number of K steps).
#include "kernels.h"
#include "block_ops.h"
#include "mfma.h"

namespace moe {

namespace {

// Sum over the 64 lanes of a wave (xor tree, every lane gets the total).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Padded column offsets of the G row groups: poff[g + 1] = poff[g] + the
// group's rows rounded up to 64.
__global__ __launch_bounds__(kMaxExperts) void poff_kernel(const int32_t* __restrict__ offsets,
                                                           int G, int32_t* __restrict__ poff) {
  __shared__ int32_t wsum[kMaxExperts / 64];
  const int g = threadIdx.x;
  const int w = g < G ? (offsets[g + 1] - offsets[g] + 63) / 64 * 64 : 0;
  int total;
  const int start = block_excl_scan(w, wsum, total);
  if (g < G) poff[g] = start;
  if (g == 0) poff[G] = total;
}

// out[c][poff[g] + j] = scale * src[row][c] for the j-th row of group g (row =
// row_token[offsets[g] + j] when gathering, else offsets[g] + j; scale =
// row_gate of that grouped row when given, else 1); zero in the padding
// columns.  A block covers 64 padded columns (inside one group, as every group
// spans a multiple of 64) and 64 values of c, moved as 16-byte chunks through
// a padded LDS tile (the padding keeps the column reads on distinct banks).
// C and lds are multiples of the chunk width.  With psum, also the sum over
// the block's 64 rows of each c: psum[col0 / 64][c] (rows 16 q .. 16 q + 15
// added in order by quarter q, then the quarters in order), for the bias
// gradients (seg_finish_kernel).
template <typename T>
__global__ __launch_bounds__(256) void gather_transpose_kernel(
    const T* __restrict__ src, int64_t lds, int C, const int32_t* __restrict__ row_token,
    const float* __restrict__ row_gate, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ poff, int G, T* __restrict__ out, int64_t ldo,
    float* __restrict__ psum) {
  constexpr int V = 16 / sizeof(T), CPR = 64 / V, LDT = 64 + V;
  __shared__ __align__(16) T tile[64 * LDT];
  __shared__ float qsum[4][64];
  const int col0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  if (col0 >= poff[G]) return;
  int lo = 0, hi = G;  // poff[lo] <= col0 < poff[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (poff[mid] <= col0) lo = mid;
    else hi = mid;
  }
  const int j0 = col0 - poff[lo], base = offsets[lo], rows = offsets[lo + 1] - base;
  union Chunk {
    uint4 u;
    T e[V];
  };
  for (int q = threadIdx.x; q < 64 * CPR; q += 256) {
    const int i = q / CPR, ch = q % CPR;  // tile row i = padded column col0 + i
    const int j = j0 + i, c = c0 + ch * V;
    Chunk v;
    v.u = make_uint4(0, 0, 0, 0);
    if (j < rows && c < C) {
      const int r = base + j;
      const int64_t srow = row_token ? row_token[r] : r;
      v.u = *reinterpret_cast<const uint4*>(src + srow * lds + c);
      if (row_gate) {
        const float g = row_gate[r];
#pragma unroll
        for (int e = 0; e < V; ++e) v.e[e] = from_f32<T>(g * to_f32<T>(v.e[e]));
      }
    }
    *reinterpret_cast<uint4*>(&tile[i * LDT + ch * V]) = v.u;
  }
  __syncthreads();
  if (psum) {
    const int cc = threadIdx.x & 63, qq = threadIdx.x >> 6;
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) sq += to_f32<T>(tile[(qq * 16 + i) * LDT + cc]);
    qsum[qq][cc] = sq;
    __syncthreads();
    if (threadIdx.x < 64 && c0 + cc < C)
      psum[static_cast<int64_t>(col0 / 64) * C + c0 + cc] =
          ((qsum[0][cc] + qsum[1][cc]) + qsum[2][cc]) + qsum[3][cc];
  }
  for (int q = threadIdx.x; q < 64 * CPR; q += 256) {
    const int cc = q / CPR, ch = q % CPR;  // output row c0 + cc, columns col0 + ch V ..
    const int c = c0 + cc;
    if (c >= C) continue;
    Chunk w;
#pragma unroll
    for (int e = 0; e < V; ++e) w.e[e] = tile[(ch * V + e) * LDT + cc];
    *reinterpret_cast<uint4*>(out + static_cast<int64_t>(c) * ldo + col0 + ch * V) = w.u;
  }
}

// Bias gradients from the transpose's block sums: out_g[c] = sum over group
// g's 64-row blocks (poff[g] / 64 .. poff[g + 1] / 64) of psum[block][c], in
// block order (routed groups g < E write out + g * C, the shared group out_sh,
// with Cs values).  ldp = the row length of psum.
template <typename T>
__global__ __launch_bounds__(256) void seg_finish_kernel(const float* __restrict__ psum, int ldp,
                                                         const int32_t* __restrict__ poff, int E,
                                                         int C, int Cs, T* __restrict__ out,
                                                         T* __restrict__ out_sh) {
  const int g = blockIdx.y, c = blockIdx.x * 256 + threadIdx.x;
  const int Cg = g < E ? C : Cs;
  T* o = g < E ? (out ? out + static_cast<int64_t>(g) * C : nullptr) : out_sh;
  if (c >= Cg || !o) return;
  float s = 0.f;
  for (int blk = poff[g] / 64; blk < poff[g + 1] / 64; ++blk)
    s += psum[static_cast<int64_t>(blk) * ldp + c];
  o[c] = from_f32<T>(s);
}

struct WgradArgs {
  const void* A;  // [M, lda]: group g's K columns start at poff[g0 + gi]
  int64_t lda;
  const void* B;  // [N, ldb]
  int64_t ldb;
  const int32_t* poff;
  int g0;         // first group of this launch
  int M, N, tiles_m, tiles_n;
  void* C;        // [groups, M, N]
};

// C_gi[m][n] = sum over group g0 + gi's K columns of A[m][k] B[n][k]: the
// weight gradients, contracting over the rows each expert received.  Every
// group's K is a multiple of 64 (zero padded); K = 0 writes zeros.  Register-
// staged tiles with a padded LDS row; MFMA 32x32.
template <typename T, int BM, int BN, int BK, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64) void wgrad_kernel(WgradArgs a) {
  using M = Mfma<T>;
  constexpr int NT = WM * WN * 64;
  constexpr int CH = 16 / sizeof(T);
  constexpr int LDK = BK + CH;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MI = WTM / 32, NI = WTN / 32;
  constexpr int CPR = BK / CH;
  constexpr int ACH = BM * CPR / NT, BCH = BN * CPR / NT;
  static_assert(ACH >= 1 && BCH >= 1 && BM * CPR % NT == 0 && BN * CPR % NT == 0, "loader");
  __shared__ __align__(16) T smem[(BM + BN) * LDK];
  T* As = smem;
  T* Bs = smem + BM * LDK;

  const int per = a.tiles_m * a.tiles_n;
  const int gi = blockIdx.x / per, rem = blockIdx.x % per;
  const int mt = rem / a.tiles_n, nt = rem % a.tiles_n;
  const int g = a.g0 + gi;
  const int k0 = a.poff[g], K = a.poff[g + 1] - k0;
  const int m0 = mt * BM, n0 = nt * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  const T* asrc[ACH];
  int aoff[ACH], akc[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int c = tid + i * NT, r = c / CPR;
    akc[i] = (c % CPR) * CH;
    aoff[i] = r * LDK + akc[i];
    asrc[i] = m0 + r < a.M ? static_cast<const T*>(a.A) + static_cast<int64_t>(m0 + r) * a.lda + k0
                           : nullptr;
  }
  const T* bsrc[BCH];
  int boff[BCH], bkc[BCH];
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int c = tid + i * NT, r = c / CPR;
    bkc[i] = (c % CPR) * CH;
    boff[i] = r * LDK + bkc[i];
    bsrc[i] = n0 + r < a.N ? static_cast<const T*>(a.B) + static_cast<int64_t>(n0 + r) * a.ldb + k0
                           : nullptr;
  }
  uint4 ra[ACH], rb[BCH];
  auto gload = [&](int kk0) {
#pragma unroll
    for (int i = 0; i < ACH; ++i)
      ra[i] = asrc[i] ? *reinterpret_cast<const uint4*>(asrc[i] + kk0 + akc[i])
                      : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < BCH; ++i)
      rb[i] = bsrc[i] ? *reinterpret_cast<const uint4*>(bsrc[i] + kk0 + bkc[i])
                      : make_uint4(0, 0, 0, 0);
  };
  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  if (K > 0) gload(0);
  for (int kk0 = 0; kk0 < K; kk0 += BK) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ACH; ++i) *reinterpret_cast<uint4*>(&As[aoff[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < BCH; ++i) *reinterpret_cast<uint4*>(&Bs[boff[i]]) = rb[i];
    __syncthreads();
    if (kk0 + BK < K) gload(kk0 + BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += M::kStep) {
      const int kl = kk + (lane >> 5) * M::kVec;
      typename M::frag fa[MI], fb[NI];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        fa[i] = M::load(&As[(wm * WTM + i * 32 + (lane & 31)) * LDK + kl]);
#pragma unroll
      for (int j = 0; j < NI; ++j)
        fb[j] = M::load(&Bs[(wn * WTN + j * 32 + (lane & 31)) * LDK + kl]);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = M::op(fa[i], fb[j], acc[i][j]);
    }
  }
  // Epilogue through LDS: each wave writes its WTM x WTN block (in T) to its own
  // region of the (now free) tile buffers, then stores whole 16-byte chunks of
  // output rows, so a wave's stores cover full 128-byte lines.
  constexpr int V = 16 / sizeof(T), LDW = WTN + V;
  static_assert(WM * WN * WTM * LDW <= (BM + BN) * LDK, "epilogue staging fits the tile buffers");
  __syncthreads();  // every wave is done with As / Bs
  T* stage = smem + wave * WTM * LDW;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
        stage[r * LDW + j * 32 + (lane & 31)] = from_f32<T>(acc[i][j][q]);
      }
  __syncthreads();
  T* Cg = static_cast<T*>(a.C) + static_cast<int64_t>(gi) * a.M * a.N;
  constexpr int CPRW = WTN / V;  // chunks per wave row
  for (int q = lane; q < WTM * CPRW; q += 64) {
    const int r = q / CPRW, ch = q % CPRW;
    const int m = m0 + wm * WTM + r, n = n0 + wn * WTN + ch * V;
    if (m < a.M && n < a.N)
      *reinterpret_cast<uint4*>(Cg + static_cast<int64_t>(m) * a.N + n) =
          *reinterpret_cast<const uint4*>(stage + r * LDW + ch * V);
  }
}

// dg[t * k + i] = <dy_t, y_rows[r]> / gate_r for the pair's row r = inv[t * k + i]
// (the expert output before gating); 0 for a dropped pair or a zero gate.
// Without inv (expert choice) the pairs are the rows themselves: dg[r] for
// token row_token[r].  One wave per pair.
template <typename T>
__global__ __launch_bounds__(256) void gate_grad_kernel(const T* __restrict__ dy,
                                                        const float* __restrict__ y_rows,
                                                        const int32_t* __restrict__ inv,
                                                        const int32_t* __restrict__ row_token,
                                                        const float* __restrict__ row_gate,
                                                        int64_t pairs, int k, int d,
                                                        float* __restrict__ dg) {
  const int64_t pair = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (pair >= pairs) return;
  const int r = inv ? inv[pair] : static_cast<int>(pair);
  const int64_t t = inv ? pair / k : row_token[r];
  float s = 0.f;
  if (r >= 0) {
    const float* yr = y_rows + static_cast<int64_t>(r) * d;
    const T* dyt = dy + t * d;
    for (int c = lane * 4; c < d; c += 256) {
      const float4 v = *reinterpret_cast<const float4*>(yr + c);
      s += v.x * to_f32<T>(dyt[c]) + v.y * to_f32<T>(dyt[c + 1]) + v.z * to_f32<T>(dyt[c + 2]) +
           v.w * to_f32<T>(dyt[c + 3]);
    }
  }
  s = wave_sum(s);
  if (lane == 0) {
    const float g = r >= 0 ? row_gate[r] : 0.f;
    dg[pair] = g != 0.f ? s / g : 0.f;
  }
}

// aux_dp[e] = alpha * 2 (m_e - mean m) / ((E - 1) T): the balance term's
// gradient with respect to each token's probability of expert e, m_e the mean
// probability (from the gate's fp64 per-block sums); 0 when alpha = 0 or E = 1.
__global__ __launch_bounds__(kMaxExperts) void aux_prep_kernel(const double* __restrict__ stat_part,
                                                               int nb, int E, int64_t T,
                                                               float alpha,
                                                               float* __restrict__ aux_dp) {
  __shared__ double wsd[kMaxExperts / 64];
  __shared__ double rsum[kMaxExperts];
  const int e = threadIdx.x;
  // thread (c, e') adds expert e' over range c of the blocks; thread e then
  // adds its ranges in order (fp64 throughout)
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
  double m = 0.0;
  if (e < E) {
    for (int c = 0; c < chunks; ++c) m += rsum[e * chunks + c];
    m /= static_cast<double>(T);
  }
  const double mbar = block_sum_d(m, wsd) / E;
  if (e < E)
    aux_dp[e] = (E > 1 && alpha != 0.f)
                    ? static_cast<float>(alpha * 2.0 * (m - mbar) / ((E - 1) * static_cast<double>(T)))
                    : 0.f;
}

// One 64-lane block per token: dp over the experts (renormalisation backward of
// the gate gradients on the k chosen experts, plus aux_dp), then the softmax
// backward dl = p (dp - <p, dp>).
__global__ __launch_bounds__(64) void router_bwd_kernel(const float* __restrict__ probs,
                                                        const int32_t* __restrict__ topk_idx,
                                                        const float* __restrict__ topk_w,
                                                        const float* __restrict__ dg,
                                                        const float* __restrict__ aux_dp, int E,
                                                        int k, int renorm, float* __restrict__ dl) {
  __shared__ float dp[kMaxExperts];
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x;
  const float* p = probs + t * E;
  for (int e = lane; e < E; e += 64) dp[e] = aux_dp[e];
  int ei = 0;
  float pi = 0.f, gi = 0.f, dgi = 0.f;
  if (lane < k) {
    ei = topk_idx[t * k + lane];
    pi = p[ei];
    gi = topk_w[t * k + lane];
    dgi = dg[t * k + lane];
  }
  const float S = wave_sum(pi), dot = wave_sum(dgi * gi);
  __syncthreads();
  if (lane < k) dp[ei] += renorm ? (dgi - dot) / S : dgi;  // the k experts are distinct
  __syncthreads();
  float s = 0.f;
  for (int e = lane; e < E; e += 64) s += p[e] * dp[e];
  s = wave_sum(s);
  for (int e = lane; e < E; e += 64) dl[t * E + e] = p[e] * (dp[e] - s);
}

// Expert choice, one 64-lane block per token: dp[e] = the gate gradient of the
// row where expert e took the token (from the selection bitmap; 0 if it did
// not take it) + aux_dp[e], then dl = p (dp - <p, dp>) with p read from the
// expert-major softmax.
__global__ __launch_bounds__(64) void ec_router_bwd_kernel(const float* __restrict__ probsT,
                                                           const uint32_t* __restrict__ sel,
                                                           const int32_t* __restrict__ pre,
                                                           const float* __restrict__ dgr,
                                                           const float* __restrict__ aux_dp,
                                                           int64_t Tn, int E, int W, int Ce,
                                                           float* __restrict__ dl) {
  __shared__ float dp[kMaxExperts];
  __shared__ float pp[kMaxExperts];
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t w = t >> 5;
  const uint32_t bit = 1u << (t & 31);
  float s = 0.f;
  for (int e = lane; e < E; e += 64) {
    const float p = probsT[static_cast<int64_t>(e) * Tn + t];
    float g = aux_dp[e];
    const uint32_t m = sel[static_cast<int64_t>(e) * W + w];
    if (m & bit)
      g += dgr[static_cast<int64_t>(e) * Ce + pre[static_cast<int64_t>(e) * W + w] +
               __popc(m & (bit - 1u))];
    dp[e] = g;
    pp[e] = p;
    s += p * g;
  }
  s = wave_sum(s);
  for (int e = lane; e < E; e += 64) dl[t * E + e] = pp[e] * (dp[e] - s);
}

// Partial router weight gradients: part[s][e][j] = sum over the tokens of
// chunk s of dl[t][e] * x[t][j] (x[t][d] = 1 gives the bias), tokens in order.
// A thread owns 8 consecutive columns and 8 experts: one 16-byte x load and
// the block's 8 dl values feed 64 products per token.
template <typename T>
__global__ __launch_bounds__(256) void router_wgrad_part_kernel(const T* __restrict__ x,
                                                                const float* __restrict__ dl,
                                                                int64_t Tn, int d, int E,
                                                                int64_t chunk,
                                                                float* __restrict__ part) {
  constexpr int V = 16 / sizeof(T);  // x elements per 16-byte load
  static_assert(V <= 8, "columns per thread");
  constexpr int NC = 8;              // columns per thread (two loads for fp32)
  const int j0 = (blockIdx.x * 256 + threadIdx.x) * NC;
  const int e0 = blockIdx.y * 8;
  const int64_t s = blockIdx.z, t0 = s * chunk, t1 = min(Tn, t0 + chunk);
  if (j0 > d) return;
  float acc[8][NC];
#pragma unroll
  for (int q = 0; q < 8; ++q)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[q][c] = 0.f;
  auto load_x = [&](int64_t t, float (&xv)[NC]) {
    if (j0 < d) {  // d is a multiple of 8: the chunk lies inside the row
#pragma unroll
      for (int h = 0; h < NC / V; ++h) {
        const uint4 u = *reinterpret_cast<const uint4*>(x + t * d + j0 + h * V);
        const T* v = reinterpret_cast<const T*>(&u);
#pragma unroll
        for (int c = 0; c < V; ++c) xv[h * V + c] = to_f32<T>(v[c]);
      }
    } else {  // j0 == d: the bias column, then nothing
#pragma unroll
      for (int c = 0; c < NC; ++c) xv[c] = c == 0 ? 1.f : 0.f;
    }
  };
  // four tokens' loads go out together (one memory latency per four tokens);
  // the products are still added token by token
  constexpr int U = 4;
  // all eight experts present and their dl rows 16-byte aligned (E % 4 == 0)
  const bool full8 = e0 + 8 <= E && E % 4 == 0;
  int64_t t = t0;
  for (; t + U <= t1; t += U) {
    float xv[U][NC], g[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) load_x(t + u, xv[u]);
    if (full8) {  // block-uniform: one 8-value scalar load per token
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float4* p = reinterpret_cast<const float4*>(dl + (t + u) * E + e0);
        const float4 a = p[0], b = p[1];
        g[u][0] = a.x, g[u][1] = a.y, g[u][2] = a.z, g[u][3] = a.w;
        g[u][4] = b.x, g[u][5] = b.y, g[u][6] = b.z, g[u][7] = b.w;
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int q = 0; q < 8; ++q) g[u][q] = e0 + q < E ? dl[(t + u) * E + e0 + q] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int c = 0; c < NC; ++c) acc[q][c] += g[u][q] * xv[u][c];
  }
  for (; t < t1; ++t) {
    float xv[NC];
    load_x(t, xv);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float g = e0 + q < E ? dl[t * E + e0 + q] : 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[q][c] += g * xv[c];
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q)
#pragma unroll
    for (int c = 0; c < NC; ++c)
      if (e0 + q < E && j0 + c <= d) part[(s * E + e0 + q) * (d + 1) + j0 + c] = acc[q][c];
}

// dWg[e][j] (j < d) and dbg[e] (j = d) = sum over the chunks, in chunk order.
__global__ __launch_bounds__(256) void router_wgrad_sum_kernel(const float* __restrict__ part,
                                                               int S, int d, int E,
                                                               float* __restrict__ dWg,
                                                               float* __restrict__ dbg) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t n = static_cast<int64_t>(E) * (d + 1);
  if (i >= n) return;
  float v = 0.f;
  for (int s = 0; s < S; ++s) v += part[s * n + i];
  const int e = static_cast<int>(i / (d + 1)), j = static_cast<int>(i % (d + 1));
  if (j < d) {
    if (dWg) dWg[static_cast<int64_t>(e) * d + j] = v;
  } else if (dbg) {
    dbg[e] = v;
  }
}

// dx[t] = sum over t's kept slots of dX[inv[t, i]] (+ the shared row) +
// sum_e dl[t][e] W_g[e].  Eight tokens per block share the W_g loads; a thread
// owns 4 columns.
constexpr int kDxTokens = 8;
template <typename T>
__global__ __launch_bounds__(256) void dx_kernel(const float* __restrict__ dX,
                                                 const int32_t* __restrict__ inv,
                                                 const int32_t* __restrict__ offsets,
                                                 const float* __restrict__ dl,
                                                 const float* __restrict__ Wg, int64_t Tn, int d,
                                                 int E, int k, int shared, T* __restrict__ dx) {
  __shared__ float sdl[kDxTokens][kMaxExperts];
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kDxTokens;
  for (int i = threadIdx.x; i < kDxTokens * E; i += 256) {
    const int tt = i / E, e = i % E;
    sdl[tt][e] = t0 + tt < Tn ? dl[(t0 + tt) * E + e] : 0.f;
  }
  __syncthreads();
  const int c = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (c >= d) return;
  float4 acc[kDxTokens];
#pragma unroll
  for (int tt = 0; tt < kDxTokens; ++tt) acc[tt] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int e = 0; e < E; ++e) {
    const float4 w = *reinterpret_cast<const float4*>(Wg + static_cast<int64_t>(e) * d + c);
#pragma unroll
    for (int tt = 0; tt < kDxTokens; ++tt) {
      const float l = sdl[tt][e];
      acc[tt].x += l * w.x;
      acc[tt].y += l * w.y;
      acc[tt].z += l * w.z;
      acc[tt].w += l * w.w;
    }
  }
  const int rs0 = shared ? offsets[E] : 0;
  for (int tt = 0; tt < kDxTokens; ++tt) {
    const int64_t t = t0 + tt;
    if (t >= Tn) break;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i = 0; i < k; ++i) {
      const int r = inv[t * k + i];
      if (r < 0) continue;
      const float4 u = *reinterpret_cast<const float4*>(dX + static_cast<int64_t>(r) * d + c);
      v.x += u.x;
      v.y += u.y;
      v.z += u.z;
      v.w += u.w;
    }
    if (shared) {
      const float4 u = *reinterpret_cast<const float4*>(dX + (rs0 + t) * d + c);
      v.x += u.x;
      v.y += u.y;
      v.z += u.z;
      v.w += u.w;
    }
    v.x += acc[tt].x;
    v.y += acc[tt].y;
    v.z += acc[tt].z;
    v.w += acc[tt].w;
    store4<T>(dx + t * d + c, v);
  }
}

// Expert choice: dx[t] = sum over the experts that took t, in expert order, of
// dX rows (+ the shared row) + sum_e dl[t][e] W_g[e].  Eight tokens per block:
// each token's rows are found in the selection bitmaps and compacted into LDS
// in expert order (ballots), then summed as in dx_kernel.
template <typename T>
__global__ __launch_bounds__(256) void ec_dx_kernel(const float* __restrict__ dX,
                                                    const uint32_t* __restrict__ sel,
                                                    const int32_t* __restrict__ pre, int W,
                                                    int Ce, const float* __restrict__ dl,
                                                    const float* __restrict__ Wg, int64_t Tn,
                                                    int d, int E, int shared,
                                                    T* __restrict__ dx) {
  __shared__ float sdl[kDxTokens][kMaxExperts];
  __shared__ int32_t rows[kDxTokens][kMaxExperts];
  __shared__ int32_t nrow[kDxTokens];
  __shared__ int32_t wcnt[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kDxTokens;
  for (int i = tid; i < kDxTokens * E; i += 256) {
    const int tt = i / E, e = i % E;
    sdl[tt][e] = t0 + tt < Tn ? dl[(t0 + tt) * E + e] : 0.f;
  }
  for (int tt = 0; tt < kDxTokens; ++tt) {
    const int64_t t = t0 + tt;
    const int64_t w = t >> 5;
    const uint32_t bit = 1u << (t & 31);
    int n = 0;
    for (int e0 = 0; e0 < E; e0 += 256) {
      const int e = e0 + tid;
      int row = -1;
      if (t < Tn && e < E) {
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
      if (row >= 0) rows[tt][off + __popcll(b & ((uint64_t(1) << lane) - 1))] = row;
      n += tot;
      __syncthreads();
    }
    if (tid == 0) nrow[tt] = n;
  }
  __syncthreads();
  const int c = (blockIdx.y * 256 + tid) * 4;
  if (c >= d) return;
  float4 acc[kDxTokens];
#pragma unroll
  for (int tt = 0; tt < kDxTokens; ++tt) acc[tt] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int e = 0; e < E; ++e) {
    const float4 wv = *reinterpret_cast<const float4*>(Wg + static_cast<int64_t>(e) * d + c);
#pragma unroll
    for (int tt = 0; tt < kDxTokens; ++tt) {
      const float l = sdl[tt][e];
      acc[tt].x += l * wv.x;
      acc[tt].y += l * wv.y;
      acc[tt].z += l * wv.z;
      acc[tt].w += l * wv.w;
    }
  }
  const int64_t rs0 = static_cast<int64_t>(E) * Ce;
  for (int tt = 0; tt < kDxTokens; ++tt) {
    const int64_t t = t0 + tt;
    if (t >= Tn) break;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i = 0; i < nrow[tt]; ++i) {
      const float4 u =
          *reinterpret_cast<const float4*>(dX + static_cast<int64_t>(rows[tt][i]) * d + c);
      v.x += u.x;
      v.y += u.y;
      v.z += u.z;
      v.w += u.w;
    }
    if (shared) {
      const float4 u = *reinterpret_cast<const float4*>(dX + (rs0 + t) * d + c);
      v.x += u.x;
      v.y += u.y;
      v.z += u.z;
      v.w += u.w;
    }
    v.x += acc[tt].x;
    v.y += acc[tt].y;
    v.z += acc[tt].z;
    v.w += acc[tt].w;
    store4<T>(dx + t * d + c, v);
  }
}

// Zero fill (used where a gradient is zero by definition, e.g. T = 0).
__global__ __launch_bounds__(256) void zero_kernel(uint32_t* __restrict__ p, int64_t words) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < words;
       i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0u;
}

template <typename T>
void run_wgrad(const WgradArgs& w, int groups, int64_t rows_avg, hipStream_t st) {
  if (groups <= 0 || w.M <= 0 || w.N <= 0) return;
  if constexpr (sizeof(T) == 2) {
    // bf16: the LDS-DMA GEMM with each group's K range (the padded rows are
    // multiples of 64 whatever the layer's tier).  Tiles cover the weights,
    // M x N per group: 256 x 256 when they fill at least two rounds of one
    // block per CU (256 x 128 with two 4-wave blocks per CU when a group has
    // at most 64 rows: its tiles are almost all epilogue writes), else
    // 128 x 128.  Chosen from measurements: with 64 < rows per expert < 256 (a
    // few K steps per tile) wgrad_kernel below, four resident blocks per CU,
    // overlaps the short K loops better.
    const WgradGemm g{w.A, w.lda, w.B, w.ldb, w.poff, w.g0, groups, w.M, w.N, w.C};
    const int64_t large = int64_t(groups) * ceil_div(w.M, 256) * ceil_div(w.N, 256);
    const int shape = large < 512 ? kGemmDmaMid : rows_avg <= 64 ? kGemmDmaSmall : kGemmDmaLarge;
    if ((rows_avg >= 256 || rows_avg <= 64) && wgrad_dma_fits(shape, g)) {
      (void)launch_wgrad_dma(shape, g, st);
      return;
    }
  }
  constexpr bool B16 = sizeof(T) == 2;
  constexpr int BM = B16 ? 128 : 64, BN = B16 ? 128 : 64, BK = B16 ? 64 : 32;
  WgradArgs a = w;
  a.tiles_m = static_cast<int>(ceil_div(a.M, BM));
  a.tiles_n = static_cast<int>(ceil_div(a.N, BN));
  const int64_t blocks = static_cast<int64_t>(groups) * a.tiles_m * a.tiles_n;
  wgrad_kernel<T, BM, BN, BK, 2, 2><<<static_cast<unsigned>(blocks), 256, 0, st>>>(a);
}

template <typename T>
void run_bwd(const BwdArgs& b, int part, hipStream_t st) {
  const int ldh = b.F > b.Fs ? b.F : b.Fs;
  const int G = b.E + (b.Fs > 0 ? 1 : 0);
  if (part == kBwdRouter) {
    const int64_t pairs = b.ec ? static_cast<int64_t>(b.E) * b.Ce : b.T * b.k;
    if (pairs > 0)
      gate_grad_kernel<T><<<static_cast<unsigned>(ceil_div(pairs, 4)), 256, 0, st>>>(
          static_cast<const T*>(b.dy), b.y_rows, b.ec ? nullptr : b.inv, b.row_token, b.row_gate,
          pairs, b.k, b.d, b.dg);
    aux_prep_kernel<<<1, kMaxExperts, 0, st>>>(b.stat_part, b.nb, b.E, b.T, b.alpha, b.aux_dp);
    if (b.ec)
      ec_router_bwd_kernel<<<static_cast<unsigned>(b.T), 64, 0, st>>>(
          b.probsT, b.sel, b.pre, b.dg, b.aux_dp, b.T, b.E, b.W, b.Ce, b.dl);
    else
      router_bwd_kernel<<<static_cast<unsigned>(b.T), 64, 0, st>>>(
          b.probs, b.topk_idx, b.topk_w, b.dg, b.aux_dp, b.E, b.k, b.renorm, b.dl);
    if (b.dWg || b.dbg) {
      const dim3 grid(static_cast<unsigned>(ceil_div(b.d + 1, 256 * 8)),
                      static_cast<unsigned>(ceil_div(b.E, 8)), static_cast<unsigned>(b.wg_split));
      router_wgrad_part_kernel<T><<<grid, 256, 0, st>>>(static_cast<const T*>(b.x), b.dl, b.T,
                                                        b.d, b.E, b.wg_chunk, b.wg_part);
      const int64_t n = static_cast<int64_t>(b.E) * (b.d + 1);
      router_wgrad_sum_kernel<<<static_cast<unsigned>(ceil_div(n, 256)), 256, 0, st>>>(
          b.wg_part, b.wg_split, b.d, b.E, b.dWg, b.dbg);
    }
    return;
  }
  if (part == kBwdDx) {
    const dim3 grid(static_cast<unsigned>(ceil_div(b.T, kDxTokens)),
                    static_cast<unsigned>(ceil_div(b.d, 1024)));
    if (b.ec)
      ec_dx_kernel<T><<<grid, 256, 0, st>>>(b.dX, b.sel, b.pre, b.W, b.Ce, b.dl, b.Wg, b.T, b.d,
                                            b.E, b.Fs > 0, static_cast<T*>(b.dx));
    else
      dx_kernel<T><<<grid, 256, 0, st>>>(b.dX, b.inv, b.offsets, b.dl, b.Wg, b.T, b.d, b.E, b.k,
                                         b.Fs > 0, static_cast<T*>(b.dx));
    return;
  }
  // kBwdExpertWeights: transposed operands, weight GEMMs, bias sums
  poff_kernel<<<1, kMaxExperts, 0, st>>>(b.offsets, G, b.poff);
  const unsigned pcols = static_cast<unsigned>(b.Rp / 64);
  auto gt = [&](const void* src, int64_t lds, int C, const int32_t* rt, const float* gate,
                void* out, float* psum) {
    const dim3 grid(pcols, static_cast<unsigned>(ceil_div(C, 64)));
    gather_transpose_kernel<T><<<grid, 256, 0, st>>>(static_cast<const T*>(src), lds, C, rt, gate,
                                                     b.offsets, b.poff, G,
                                                     static_cast<T*>(out), b.Rp, psum);
  };
  // bias gradients: the transposes' 64-row block sums, added per group
  auto finish = [&](int C, int Cout, int Cs, void* out, void* out_sh) {
    const int cmax = Cout > Cs ? Cout : Cs;
    seg_finish_kernel<T><<<dim3(static_cast<unsigned>(ceil_div(cmax, 256)), G), 256, 0, st>>>(
        b.bsum, C, b.poff, b.E, Cout, Cs, static_cast<T*>(out), static_cast<T*>(out_sh));
  };
  const bool w1 = b.dW1 || b.dWs1 || b.db1 || b.dbs1;
  const bool w2 = b.dW2 || b.dWs2 || b.db2 || b.dbs2;
  const bool s1 = b.db1 || b.dbs1, s2 = b.db2 || b.dbs2;
  if (w1) {
    gt(b.Z, ldh, ldh, nullptr, nullptr, b.ZT, s1 ? b.bsum : nullptr);  // dz^T
    if (s1) finish(ldh, b.F, b.Fs, b.db1, b.dbs1);
    if (b.dW1 || b.dWs1) gt(b.x, b.d, b.d, b.row_token, nullptr, b.XT, nullptr);  // x rows^T
  }
  if (w2) {
    gt(b.dy, b.d, b.d, b.row_token, b.row_gate, b.DT, s2 ? b.bsum : nullptr);  // (gate dy)^T
    if (s2) finish(b.d, b.d, b.d, b.db2, b.dbs2);
    if (b.dW2 || b.dWs2) gt(b.H, ldh, ldh, nullptr, nullptr, b.HT, nullptr);  // h^T
  }
  WgradArgs w{};
  w.poff = b.poff;
  if (b.dW1) {  // dW1[e] [F, d] = dz^T x
    w.A = b.ZT, w.lda = b.Rp, w.B = b.XT, w.ldb = b.Rp, w.g0 = 0, w.M = b.F, w.N = b.d;
    w.C = b.dW1;
    run_wgrad<T>(w, b.E, b.rows_avg, st);
  }
  if (b.dWs1 && b.Fs > 0) {
    w.A = b.ZT, w.lda = b.Rp, w.B = b.XT, w.ldb = b.Rp, w.g0 = b.E, w.M = b.Fs, w.N = b.d;
    w.C = b.dWs1;
    run_wgrad<T>(w, 1, b.T, st);
  }
  if (b.dW2) {  // dW2[e] [d, F] = (gate dy)^T h
    w.A = b.DT, w.lda = b.Rp, w.B = b.HT, w.ldb = b.Rp, w.g0 = 0, w.M = b.d, w.N = b.F;
    w.C = b.dW2;
    run_wgrad<T>(w, b.E, b.rows_avg, st);
  }
  if (b.dWs2 && b.Fs > 0) {
    w.A = b.DT, w.lda = b.Rp, w.B = b.HT, w.ldb = b.Rp, w.g0 = b.E, w.M = b.d, w.N = b.Fs;
    w.C = b.dWs2;
    run_wgrad<T>(w, 1, b.T, st);
  }
}

}  // namespace

hipError_t launch_backward(const BwdArgs& b, int part, hipStream_t st) {
  if (b.dtype == MOE_BF16) run_bwd<bf16>(b, part, st);
  else run_bwd<float>(b, part, st);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st) {
  const int64_t words = static_cast<int64_t>(bytes / 4);
  if (words > 0)
    zero_kernel<<<static_cast<unsigned>(std::min<int64_t>(ceil_div(words, 256), 4096)), 256, 0,
                  st>>>(static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace moe
