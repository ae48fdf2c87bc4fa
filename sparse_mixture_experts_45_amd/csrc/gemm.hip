// Grouped expert GEMMs on MFMA: the up-projection with bias and activation
// fused into its epilogue, and the down-projection with bias and the gate
// weight fused into its epilogue.
//
// Pages: botmartz "Expert Routing" (expert = Linear(d, 4d), GELU,
// Linear(4d, d); output accumulates prob * expert(x)); codingnowai "Code"
// (Linear(d, d_ff), ReLU, Linear(d_ff, d)); roadtointelligence "Total versus
// active parameters" (one always-on shared expert).
//
// Both products are C[m, n] = sum_k A[m, k] B[n, k]: A rows are token rows
// (gathered from x through row_token for the up-projection, contiguous rows
// of H for the down-projection) and B rows are nn.Linear weight rows, so both
// operands are K-contiguous and feed MFMA fragments with 16-byte LDS reads.
//
// Work list: row tiles (group, first row, rows) built on the device from the
// dispatch offsets, times N tiles.  The grid is sized from an upper bound on
// the row-tile count known on the host; blocks past the real count exit.
#include "kernels.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename T>
struct Mfma;

// v_mfma_f32_32x32x16_bf16: lane l supplies row (l % 32), k = (l / 32) * 8 + 0..7
template <>
struct Mfma<bf16> {
  static constexpr int kStep = 16;
  static constexpr int kVec = 8;
  typedef bf16x8_t frag;
  static __device__ __forceinline__ frag load(const bf16* p) {
    return *reinterpret_cast<const bf16x8_t*>(p);
  }
  static __device__ __forceinline__ f32x16 op(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

// v_mfma_f32_32x32x2f32: lane l supplies row (l % 32), k = l / 32
template <>
struct Mfma<float> {
  static constexpr int kStep = 2;
  static constexpr int kVec = 1;
  typedef float frag;
  static __device__ __forceinline__ frag load(const float* p) { return *p; }
  static __device__ __forceinline__ f32x16 op(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752440f));
}

struct GemmArgs {
  const RowTile* tiles;
  const int32_t* ntiles;
  int E;                 // group E is the shared expert
  const void* A;         // up: x [T, K]; down: H [rows, lda]
  int64_t lda;
  const int32_t* row_token;
  const int32_t* row_slot;
  const float* topk_w;
  int k;
  const void* W;         // routed weights [E, N, K]
  const void* Wsh;       // shared weights [Ns, Ks]
  const void* bias;      // routed [E, N] or NULL
  const void* bias_sh;   // shared [Ns] or NULL
  int N, K, Ns, Ks;
  int n_tiles_n;         // N tiles per row tile (over max(N, Ns))
  void* out;             // up: H (T) ; down: y_rows (float)
  int64_t ldo;
  int act;
};

template <typename T, int BM, int BN, int BK, int WM, int WN, bool UP>
__global__ __launch_bounds__(WM* WN * 64) void grouped_gemm_kernel(GemmArgs a) {
  using M = Mfma<T>;
  constexpr int NT = WM * WN * 64;
  constexpr int CH = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int LDK = BK + CH;        // padded LDS row (breaks bank conflicts)
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MI = WTM / 32, NI = WTN / 32;
  constexpr int CPR = BK / CH;        // chunks per tile row
  constexpr int ACH = BM * CPR / NT;
  constexpr int BCH = BN * CPR / NT;
  static_assert(MI >= 1 && NI >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(ACH >= 1 && BCH >= 1 && BM * CPR % NT == 0 && BN * CPR % NT == 0, "loader");

  __shared__ __align__(16) T As[BM * LDK];
  __shared__ __align__(16) T Bs[BN * LDK];
  __shared__ float gate_s[BM];

  const int bid = blockIdx.x;
  const int rt = bid / a.n_tiles_n;
  const int nt = bid - rt * a.n_tiles_n;
  if (rt >= *a.ntiles) return;
  const RowTile tile = a.tiles[rt];
  const int g = tile.group;
  const bool sh = (g == a.E);
  const int N = sh ? a.Ns : a.N;
  const int K = sh ? a.Ks : a.K;
  const int n0 = nt * BN;
  if (n0 >= N) return;
  const T* Bw = static_cast<const T*>(sh ? a.Wsh : a.W) + (sh ? 0 : static_cast<int64_t>(g) * N * K);
  const T* bias = static_cast<const T*>(sh ? a.bias_sh : a.bias);
  if (bias && !sh) bias += static_cast<int64_t>(g) * N;
  const int row0 = tile.row0, rows = tile.rows;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  if (!UP) {
    for (int m = tid; m < BM; m += NT) {
      float gv = 0.f;
      if (m < rows) {
        const int r = row0 + m;
        gv = sh ? 1.0f : a.topk_w[static_cast<int64_t>(a.row_token[r]) * a.k + a.row_slot[r]];
      }
      gate_s[m] = gv;
    }
  }

  // per-thread 16-byte chunks of the A and B tiles
  const T* asrc[ACH];
  int aoff[ACH], akc[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int c = tid + i * NT;
    const int r = c / CPR;
    akc[i] = (c % CPR) * CH;
    aoff[i] = r * LDK + akc[i];
    asrc[i] = nullptr;
    if (r < rows) {
      const int64_t arow = UP ? static_cast<int64_t>(a.row_token[row0 + r]) : (row0 + r);
      asrc[i] = static_cast<const T*>(a.A) + arow * a.lda;
    }
  }
  const T* bsrc[BCH];
  int boff[BCH], bkc[BCH];
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int c = tid + i * NT;
    const int r = c / CPR;
    bkc[i] = (c % CPR) * CH;
    boff[i] = r * LDK + bkc[i];
    bsrc[i] = (n0 + r < N) ? Bw + static_cast<int64_t>(n0 + r) * K : nullptr;
  }

  uint4 ra[ACH], rb[BCH];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int kk = k0 + akc[i];
      ra[i] = (asrc[i] && kk < K) ? *reinterpret_cast<const uint4*>(asrc[i] + kk)
                                  : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int kk = k0 + bkc[i];
      rb[i] = (bsrc[i] && kk < K) ? *reinterpret_cast<const uint4*>(bsrc[i] + kk)
                                  : make_uint4(0, 0, 0, 0);
    }
  };

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  gload(0);
  for (int k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < ACH; ++i) *reinterpret_cast<uint4*>(&As[aoff[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < BCH; ++i) *reinterpret_cast<uint4*>(&Bs[boff[i]]) = rb[i];
    __syncthreads();
    if (k0 + BK < K) gload(k0 + BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += M::kStep) {
      const int kl = kk + (lane >> 5) * M::kVec;
      typename M::frag fa[MI], fb[NI];
#pragma unroll
      for (int i = 0; i < MI; ++i) fa[i] = M::load(&As[(wm * WTM + i * 32 + (lane & 31)) * LDK + kl]);
#pragma unroll
      for (int j = 0; j < NI; ++j) fb[j] = M::load(&Bs[(wn * WTN + j * 32 + (lane & 31)) * LDK + kl]);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = M::op(fa[i], fb[j], acc[i][j]);
    }
  }

  // epilogue: acc[i][j][q] is row (q/4)*8 + (lane/32)*4 + q%4, column lane%32 of the 32x32 block
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int n = n0 + wn * WTN + j * 32 + (lane & 31);
    if (n >= N) continue;
    const float bv = bias ? to_f32(bias[n]) : 0.f;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = wm * WTM + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
        if (m >= rows) continue;
        const float z = acc[i][j][q] + bv;
        const int64_t o = static_cast<int64_t>(row0 + m) * a.ldo + n;
        if (UP) {
          const float h = (a.act == MOE_ACT_RELU) ? fmaxf(z, 0.f) : gelu_erf(z);
          static_cast<T*>(a.out)[o] = from_f32<T>(h);
        } else {
          static_cast<float*>(a.out)[o] = gate_s[m] * z;
        }
      }
    }
  }
}

// Row tiles of BM rows per group, groups in order, from the dispatch offsets.
__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offsets,
                                                           int G, int BM,
                                                           RowTile* __restrict__ tiles,
                                                           int32_t* __restrict__ ntiles) {
  __shared__ int32_t sc[2][kMaxExperts + 1];
  const int g = threadIdx.x;
  int rows = 0, m = 0;
  if (g < G) {
    rows = offsets[g + 1] - offsets[g];
    m = (rows + BM - 1) / BM;
  }
  int src = 0;
  sc[0][g] = m;
  if (g == 0) sc[0][kMaxExperts] = 0;
  __syncthreads();
  for (int o = 1; o < kMaxExperts; o <<= 1) {
    const int v = sc[src][g] + (g >= o ? sc[src][g - o] : 0);
    sc[src ^ 1][g] = v;
    src ^= 1;
    __syncthreads();
  }
  const int start = sc[src][g] - m;
  if (g < G) {
    const int r0 = offsets[g];
    for (int j = 0; j < m; ++j) {
      RowTile t;
      t.group = g;
      t.row0 = r0 + j * BM;
      t.rows = min(BM, rows - j * BM);
      t.pad = 0;
      tiles[start + j] = t;
    }
  }
  if (g == kMaxExperts - 1) ntiles[0] = sc[src][g];
}

template <typename T, int BM, int BNU, int BND, int BK, int WM, int WN>
static void run_ffn(const GemmPlan& gp, const FfnArgs& f, hipStream_t st) {
  const int G = f.E + (f.Fs > 0 ? 1 : 0);
  build_tiles_kernel<<<1, kMaxExperts, 0, st>>>(f.offsets, G, BM, f.tiles, f.ntiles);
  const int64_t ldh = f.F > f.Fs ? f.F : f.Fs;

  GemmArgs u{};
  u.tiles = f.tiles;
  u.ntiles = f.ntiles;
  u.E = f.E;
  u.A = f.x;
  u.lda = f.d;
  u.row_token = f.row_token;
  u.row_slot = f.row_slot;
  u.topk_w = f.topk_w;
  u.k = f.k;
  u.W = f.W1;
  u.Wsh = f.Ws1;
  u.bias = f.b1;
  u.bias_sh = f.bs1;
  u.N = f.F;
  u.K = f.d;
  u.Ns = f.Fs;
  u.Ks = f.d;
  u.n_tiles_n = static_cast<int>(ceil_div(ldh, BNU));
  u.out = f.H;
  u.ldo = ldh;
  u.act = f.act;
  const int64_t gu = gp.tiles_max * u.n_tiles_n;
  if (gu > 0)
    grouped_gemm_kernel<T, BM, BNU, BK, WM, WN, true><<<static_cast<unsigned>(gu), WM * WN * 64, 0, st>>>(u);

  GemmArgs dn = u;
  dn.A = f.H;
  dn.lda = ldh;
  dn.W = f.W2;
  dn.Wsh = f.Ws2;
  dn.bias = f.b2;
  dn.bias_sh = f.bs2;
  dn.N = f.d;
  dn.K = f.F;
  dn.Ns = f.d;
  dn.Ks = f.Fs;
  dn.n_tiles_n = static_cast<int>(ceil_div(f.d, BND));
  dn.out = f.y_rows;
  dn.ldo = f.d;
  const int64_t gd = gp.tiles_max * dn.n_tiles_n;
  if (gd > 0)
    grouped_gemm_kernel<T, BM, BND, BK, WM, WN, false><<<static_cast<unsigned>(gd), WM * WN * 64, 0, st>>>(dn);
}

hipError_t launch_ffn(const GemmPlan& gp, const FfnArgs& f, hipStream_t st) {
  switch (gp.shape) {
    case kGemmF32: run_ffn<float, 64, 64, 64, 32, 2, 2>(gp, f, st); break;
    case kGemmBf16Large: run_ffn<bf16, 128, 128, 128, 64, 2, 2>(gp, f, st); break;
    case kGemmBf16Mid: run_ffn<bf16, 64, 128, 128, 64, 1, 4>(gp, f, st); break;
    default: run_ffn<bf16, 32, 128, 128, 64, 1, 4>(gp, f, st); break;
  }
  return hipGetLastError();
}

}  // namespace moe
