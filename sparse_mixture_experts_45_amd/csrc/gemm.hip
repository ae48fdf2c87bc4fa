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
//
// Tile order.  Workgroup i is dispatched to XCD i % 8, and each XCD has its own
// L2.  Block ids are remapped so each XCD walks a contiguous range of the
// tile list, and the list is ordered group by group, in bands of kBand N tiles
// with the group's row tiles fastest: the blocks that run together on one XCD
// share the same weight columns and the same token rows.
#include <type_traits>

#include "kernels.h"
#include "block_ops.h"
#include "mfma.h"

namespace moe {

constexpr int kXcd = 8;
constexpr int kBand = 8;

// erf by Abramowitz & Stegun, Handbook of Mathematical Functions, eq. 7.1.26:
// erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),
// t = 1 / (1 + p x) for x >= 0, odd in x; absolute error <= 1.5e-7.
__device__ __forceinline__ float erf_as(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * ax);  // 1 ulp: far below the 1.5e-7 bound
  const float poly =
      t * (0.254829592f +
           t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  const float e = 1.0f - poly * __expf(-ax * ax);
  return copysignf(e, x);
}

// GELU, exact (erf) form: 0.5 z (1 + erf(z / sqrt 2))
__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.0f + erf_as(z * 0.70710678118654752440f));
}

// its derivative: Phi(z) + z phi(z) = 0.5 (1 + erf(z / sqrt 2)) + z exp(-z^2 / 2) / sqrt(2 pi)
__device__ __forceinline__ float gelu_erf_grad(float z) {
  return 0.5f * (1.0f + erf_as(z * 0.70710678118654752440f)) +
         z * 0.39894228040143267794f * __expf(-0.5f * z * z);
}

// What a grouped-GEMM launch computes (C = A B^T over row tiles):
//   kUp       A = x rows gathered by row_token; out (layer dtype) = act(C + b1)
//   kUpTrain  as kUp, and the pre-activation C + b1 also to aux (same layout)
//   kDown     A = contiguous rows; out (fp32) = gate * (C + b2), gate = row_gate
//             of the row (1 when row_gate is null)
//   kDz       A = upstream-gradient rows gathered by row_token; out holds the
//             pre-activation z on entry and gets gate * C * act'(z) (in place)
//   kWgrad    weight gradients: A [M, lda] and B [N, ldb] (transposed grouped
//             activations), group g's K columns poff[g0 + g] .. poff[g0 + g + 1];
//             out [groups, M, N] (layer dtype) = C, no bias, no gate, no tile list
enum GemmMode { kUp = 0, kDown = 1, kDz = 2, kUpTrain = 3, kWgrad = 4 };
template <int MODE>
struct ModeOf {
  static constexpr bool gather = MODE != kDown && MODE != kWgrad;
  static constexpr bool gated = MODE == kDown || MODE == kDz;
  static constexpr bool out_f32 = MODE == kDown;
  static constexpr bool fwd_act = MODE == kUp || MODE == kUpTrain;
};

struct GemmArgs {
  const RowTile* tiles;
  const int32_t* ntiles;
  int E;                 // group E is the shared expert
  const void* A;         // up: x [T, K]; down: H [rows, lda]
  int64_t lda;
  const int32_t* row_token;
  const float* row_gate;  // gate of each row (1 for shared rows), built with the tile list
  const void* W;         // routed weights [E, N, K]
  const void* Wsh;       // shared weights [Ns, Ks]
  const void* bias;      // routed [E, N] or NULL
  const void* bias_sh;   // shared [Ns] or NULL
  int N, K, Ns, Ks;
  int n_tiles_n;         // N tiles per row tile (over max(N, Ns))
  void* out;             // up: H (T) ; down: y_rows (float); dz: z in, dz out (T)
  void* aux;             // up (train): the pre-activations (T), same layout as out
  int64_t ldo;
  int act;
  // K split of the tiles of a last, partly filled round (LDS-DMA kernel, one
  // tile per block): kpart null or smax < 2 turns it off
  float* kpart;   // partial tiles, BM * BN fp32 each
  int32_t* ksem;  // one arrival counter per split tile, zero between launches
  int slots;      // resident blocks of the launch (at most the partial tiles reserved)
  int smax;       // parts per tile, at most
  // kWgrad only (E = groups, W = B, out = C [groups, M, N], ldo = N)
  const int32_t* poff;
  int g0, M, tiles_m;
  int64_t ldb;
};

// Whole tiles and split tiles of a launch over `total` tiles: the tiles of a
// last round that fills at most half of the `slots` resident blocks are cut
// into S = min(smax, slots / R) parts (R = those tiles); D tiles run whole.
// Blocks 0 .. D-1 take whole tiles; block D + i S + s takes part s of tile
// D + i.  Every block computes the same plan from the same tile count.
__device__ __forceinline__ void split_plan(int total, int slots, int smax, int* D, int* R,
                                           int* S) {
  *D = total;
  *R = 0;
  *S = 1;
  if (smax < 2 || slots <= 0 || total <= 0) return;
  const int rem = total % slots;
  if (rem == 0) return;
  const int s = min(smax, slots / rem);
  if (s < 2) return;
  *D = total - rem;
  *R = rem;
  *S = s;
}

// XCD i % 8 runs the blocks with id i (in id order); block ids are remapped so
// each XCD walks tiles of [0, total) that share weight columns and token rows
// in its L2.  Contiguous (CHUNKED false): each XCD walks one contiguous range.
// CHUNKED: each XCD walks chunks of kChunk consecutive tiles, chunk c on XCD
// c % 8; the tiles an XCD runs at once (one per CU) come from one chunk, and
// every XCD draws chunks from the whole list, so a group whose tiles cost more
// (heavy tiles) is not left to one XCD.  A last partial round of chunks is cut
// into one contiguous range per XCD.
constexpr int kChunk = 32;
template <bool CHUNKED>
__device__ __forceinline__ int xcd_order(int pid, int total) {
  const int full = CHUNKED ? total / (kXcd * kChunk) * (kXcd * kChunk) : 0;
  if (pid < full) {
    const int x = pid % kXcd, local = pid / kXcd;
    return (local / kChunk * kXcd + x) * kChunk + local % kChunk;  // bijection onto [0, full)
  }
  const int rest = total - full, p = pid - full;
  const int q = rest / kXcd, r = rest % kXcd;
  const int x = p % kXcd, local = p / kXcd;
  return full + x * q + min(x, r) + local;  // bijection onto [full, total)
}

// Tile id -> (row tile, n tile).  The first H row tiles of the list are heavy
// (more rows than the tile height, at most one per group): their H * NT tiles
// come first, each row tile's N tiles in a row, so the longest tiles start in
// the first round and a CU gets at most one of them while there are fewer than
// the CUs.  The other tiles follow group by group.
template <bool CHUNKED = false>
__device__ __forceinline__ void decode_tile(const GemmArgs& a, int pid, int total, int H,
                                            int* rt, int* nt) {
  const int NT = a.n_tiles_n;
  int v = xcd_order<CHUNKED>(pid, total);
  if (v < H * NT) {
    *rt = v / NT;
    *nt = v % NT;
    return;
  }
  v -= H * NT;  // index among the other tiles, whose row tiles start at H
  const RowTile& t = a.tiles[H + v / NT];
  const int m = t.count;
  const int ve = v - (t.first - H) * NT;     // index inside the group
  const int band = ve / (m * kBand);
  const int rem = ve - band * m * kBand;
  *nt = band * kBand + rem / m;
  *rt = t.first + rem % m;
}

// ---------------------------------------------------------------------------
// Generic kernel: any K that is a multiple of 8 (bf16) or 4 (fp32); tiles are
// staged through registers with zero fill beyond K and beyond the tile rows.
// ---------------------------------------------------------------------------
template <typename T, int BM, int BN, int BK, int WM, int WN, int MODE, bool BT>
__global__ __launch_bounds__(WM* WN * 64) void grouped_gemm_kernel(GemmArgs a) {
  using M = Mfma<T>;
  using MD = ModeOf<MODE>;
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

  const int total = *a.ntiles * a.n_tiles_n;
  if (static_cast<int>(blockIdx.x) >= total) return;
  int rt, nt;
  decode_tile(a, blockIdx.x, total, 0, &rt, &nt);
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

  if constexpr (MD::gated) {
    for (int m = tid; m < BM; m += NT) {
      gate_s[m] = m < rows ? (a.row_gate ? a.row_gate[row0 + m] : 1.f) : 0.f;
    }
  }

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
      const int64_t arow = MD::gather ? static_cast<int64_t>(a.row_token[row0 + r]) : (row0 + r);
      asrc[i] = static_cast<const T*>(a.A) + arow * a.lda;
    }
  }
  const T* bsrc[BCH];
  int boff[BCH], bkc[BCH];
#pragma unroll
  for (int i = 0; i < BCH; ++i) {
    const int c = tid + i * NT;
    if constexpr (BT) {
      // B stored [K, N]: chunk c is row k = c / (BN / CH), columns n0 + (c % (BN / CH)) CH ..;
      // its values go to LDS transposed, Bs[n][k]
      const int kr = c / (BN / CH), nc = (c % (BN / CH)) * CH;
      bkc[i] = kr;
      boff[i] = nc * LDK + kr;
      bsrc[i] = (n0 + nc < N) ? Bw + static_cast<int64_t>(kr) * N + n0 + nc : nullptr;
    } else {
      const int r = c / CPR;
      bkc[i] = (c % CPR) * CH;
      boff[i] = r * LDK + bkc[i];
      bsrc[i] = (n0 + r < N) ? Bw + static_cast<int64_t>(n0 + r) * K : nullptr;
    }
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
      if constexpr (BT)
        rb[i] = (bsrc[i] && kk < K)
                    ? *reinterpret_cast<const uint4*>(bsrc[i] + static_cast<int64_t>(k0) * N)
                    : make_uint4(0, 0, 0, 0);
      else
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
    for (int i = 0; i < BCH; ++i) {
      if constexpr (BT) {
        union {
          uint4 u;
          T e[CH];
        } v;
        v.u = rb[i];
#pragma unroll
        for (int e = 0; e < CH; ++e) Bs[boff[i] + e * LDK] = v.e[e];
      } else {
        *reinterpret_cast<uint4*>(&Bs[boff[i]]) = rb[i];
      }
    }
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
      // kDz: the 16 pre-activations are loaded before any result is stored
      // (a load after a possibly aliasing store waits out a memory latency)
      float zr[MODE == kDz ? 16 : 1];
      if constexpr (MODE == kDz) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int m = wm * WTM + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
          // rows past the tile read its last row (no branch); unused
          zr[q] = to_f32<T>(
              static_cast<const T*>(a.out)[static_cast<int64_t>(row0 + min(m, rows - 1)) * a.ldo + n]);
        }
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = wm * WTM + i * 32 + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
        if (m >= rows) continue;
        const float z = acc[i][j][q] + bv;
        const int64_t o = static_cast<int64_t>(row0 + m) * a.ldo + n;
        if constexpr (MD::fwd_act) {
          const float h = (a.act == MOE_ACT_RELU) ? fmaxf(z, 0.f) : gelu_erf(z);
          static_cast<T*>(a.out)[o] = from_f32<T>(h);
          if constexpr (MODE == kUpTrain) static_cast<T*>(a.aux)[o] = from_f32<T>(z);
        } else if constexpr (MODE == kDz) {
          const float pre = zr[q];
          const float da = (a.act == MOE_ACT_RELU) ? (pre > 0.f ? 1.f : 0.f) : gelu_erf_grad(pre);
          static_cast<T*>(a.out)[o] = from_f32<T>(gate_s[m] * z * da);
        } else {
          static_cast<float*>(a.out)[o] = gate_s[m] * z;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 kernel for K a multiple of BK (32 or 64).  Tiles go from global memory
// straight into LDS with global_load_lds_dwordx4 (no register staging) through
// a ring of NS stages, so NS - 1 K steps are in flight while one is
// multiplied; one barrier per K step.  An LDS tile row holds BK bf16 (64 or
// 128 bytes, 4 or 8 sixteen-byte chunks) with the chunk index XORed with a
// function of the row (swz below), so the rows an MFMA fragment read touches
// per chunk land in different banks.  Each wave instruction fills 1 KB of consecutive
// tile rows; lane L writes chunk slot L % CPR of row L / CPR and fetches the
// global chunk that belongs there.  Rows past the tile (or past N) are fetched
// from a clamped valid row and their results are never stored.
// ---------------------------------------------------------------------------

// 16 bytes from global memory to LDS; the wave's 64 lanes fill 1 KB starting at
// the wave-uniform address `lds` (lane L at lds + 16 L).  CPOL: the load's
// cache-policy bits (0, or kCpolNT for data read once).
constexpr int kCpolNT = 2;  // gfx950 `nt`: non-temporal
template <int CPOL = 0>
__device__ __forceinline__ void lds_dma16(const void* g, char* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, CPOL);
}

// Chunk swizzle of tile row r.  gfx950 LDS has 64 four-byte banks (256 bytes
// per bank cycle) and services a 16-byte-per-lane read 16 lanes at a time; the
// 16 lanes of a fragment read hit 16 consecutive tile rows at the same logical
// chunk.  With 128-byte rows two rows share a bank line, so rows r and r + 2k
// must land on different chunks: chunk ^ ((r / 2) % 8).  With 64-byte rows four
// rows share a bank line: chunk ^ ((r / 4) % 4).
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  return CPR == 8 ? ((r >> 1) & 7) : ((r >> 2) & 3);
}

// Chunk swizzle of a [BK, BN] (K-major) B tile row k: the transposing reads of
// one 16-lane group touch 4 consecutive rows at the same chunk pair, so row k
// moves its chunks by 4 (k % 4) positions (4 rows x 2 chunks x 2 column halves
// = 16 distinct chunk positions, one pass of the 64 banks).
__device__ __forceinline__ int swzt(int k) { return (k & 3) << 2; }

typedef short i16x4 __attribute__((ext_vector_type(4)));
// ds_read_b64_tr_b16: within each group of 16 lanes, the four 16-bit values
// the lanes address (lane i: 4 values at its address) are redistributed so
// that lane j gets value j of the group's rows: lane i = 4 r + q addressing
// row r, columns 4 q .. 4 q + 3 hands lane j the column-j value of rows 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(const_cast<char*>(p)));
}

// s_waitcnt with vmcnt = n and the other counters left alone (gfx9 encoding)
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most min(pending, P) stages of JPW loads each are still in
// flight (pending <= 0: none); the loads issued before them have then landed.
template <int NS, int JPW, int P = NS - 2>
__device__ __forceinline__ void wait_stages(int pending) {
  if constexpr (P <= 0) {
    wait_vmcnt<0>();
  } else {
    if (pending >= P) wait_vmcnt<P * JPW>();
    else wait_stages<NS, JPW, P - 1>(pending);
  }
}

// Scheduling hints for N k16 steps: each step's NM MFMAs (0x008) with the NR
// fragment reads (0x100: DS reads) of the following step spread between them.
template <int S, int N, int NR, int NM>
__device__ __forceinline__ void sched_steps() {
  if constexpr (S < N) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, NM / NR > 0 ? NM / NR : 1, 0);
    }
    if constexpr (NM > NR && NM % NR != 0) __builtin_amdgcn_sched_group_barrier(0x008, NM % NR, 0);
    sched_steps<S + 1, N, NR, NM>();
  }
}

// Persistent kernel: one block per CU slot walks tiles t = blockIdx.x,
// blockIdx.x + gridDim.x, ...  While tile t is multiplied, the metadata of the
// next tile (its token rows, its gates) is already loaded; after the K loop
// the next tile's first stages are issued before tile t's epilogue runs, so
// load latency hides under the epilogue instead of idling the CU.
//
// Heavy tiles (XR = 1): a row tile may hold up to BM + 32 WM rows, the rows
// past BM forming one more 32-row block per wave row (rows BM + 32 wm ..).
// The tile list merges an expert's last few rows (at most 32 WM) into its
// previous tile instead of giving them a tile of their own; tiles of at most
// BM rows skip the extra block's loads and MFMAs.
template <int BM, int BN, int BK, int NS, int WM, int WN, int OCC, int PERSIST, int MODE,
          bool BT, int XR = 0, int NTB = 0>
__global__ __launch_bounds__(WM* WN * 64, OCC) void grouped_gemm_dma_kernel(GemmArgs a) {
  using MD = ModeOf<MODE>;
  // BT: the group's B is stored [K, N] (row k holds N contiguous values), as
  // the input-gradient pass reads the expert weights; its tile sits in LDS as
  // BK rows of BN values and MFMA fragments come from transposing LDS reads.
  static_assert(!BT || BN >= 128, "transposed B tile: at least 16 chunks per row");
  static_assert(MODE != kWgrad || (!PERSIST && !BT), "weight gradients: one tile per block");
  constexpr int NW = WM * WN;
  constexpr int NT = NW * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MI = WTM / 32, NI = WTN / 32;
  constexpr int BMX = BM + XR * WM * 32;   // A rows a tile can hold
  constexpr int MIX = MI + XR;             // row blocks per wave, the extra one included
  constexpr int RB = BK * 2;               // bytes per LDS tile row
  constexpr int CPR = BK / 8;              // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;            // rows per wave instruction
  constexpr int ROWS = BMX + BN;           // A rows then B rows
  constexpr int JPW = ROWS / RPI / NW;     // load instructions per wave per stage
  constexpr int STAGE = ROWS * RB;         // bytes
  constexpr int KS = BK / 16;              // k16 MFMA steps per stage
  constexpr int GPT = (BMX + NT - 1) / NT;  // gates per thread
  static_assert(ROWS % (RPI * NW) == 0 && MI >= 1 && NI >= 1, "tile shape");
  // the extra rows take whole load instructions; heavy tiles skip none of them
  // and lighter ones skip all, which the vmcnt waits of a 2-stage ring (all
  // vmcnt(0)) do not count
  static_assert(XR == 0 || (NS == 2 && (XR * WM * 32) % (RPI * NW) == 0 && !BT &&
                            MODE != kWgrad && !PERSIST),
                "heavy tiles: 2-stage ring, forward modes, one tile per block");
  static_assert(BK == 32 || BK == 64, "BK");
  static_assert(NS >= 2 && JPW * (NS - 2) < 64, "stages");

  extern __shared__ __align__(16) char smem[];
  __shared__ float gate_s[2][BMX];
  __shared__ int split_last;

  const int total = MODE == kWgrad ? a.E * a.tiles_m * a.n_tiles_n : *a.ntiles * a.n_tiles_n;
  // heavy row tiles lead the list (only lists built for heavy-tile kernels have any)
  const int nheavy = XR > 0 ? a.ntiles[kSplitSlots + 1] : 0;
  int D = total, R = 0, S = 1;
  if constexpr (!PERSIST) split_plan(total, a.slots, a.smax, &D, &R, &S);
  int t = blockIdx.x;
  if (t >= D + R * S) return;
  int part = -1;  // K part of a split tile, or -1 for a whole tile
  if (t >= D) {
    part = (t - D) % S;
    t = D + (t - D) / S;
  }

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane / CPR;  // row inside a load instruction's rows
  int aoffs[MIX], boffs[NI];
  const int lrow = lane & 31;
  // A row of row block i of this wave (the extra block: BM + 32 wm ..)
  auto arow_blk = [&](int i) { return i < MI ? wm * WTM + i * 32 : BM + wm * 32; };
#pragma unroll
  for (int i = 0; i < MIX; ++i) aoffs[i] = (arow_blk(i) + lrow) * RB;
#pragma unroll
  for (int j = 0; j < NI; ++j) boffs[j] = (BMX + wn * WTN + j * 32 + lrow) * RB;
  const int rsw = swz<CPR>(lrow);  // the same for every fragment row of this lane
  // BT fragment reads: lane l takes rows 8 (l / 32) + (l % 16) / 4 (+ 4 for the
  // second read) and 4 columns from 16 ((l / 16) % 2) + 4 (l % 4) of its
  // 32-column block; btoffs[j] is the byte offset (k16 step 0, first read)
  int btoffs[NI];
  if constexpr (BT) {
    const int trow = 8 * (lane >> 5) + ((lane & 15) >> 2);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int col = wn * WTN + j * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      btoffs[j] = BMX * RB + trow * (BN * 2) + (((col >> 3) ^ swzt(trow)) << 4) + (col & 7) * 2;
    }
  }

  struct Tile {
    int row0, rows, n0, N, K;
    const bf16* bw;    // weight rows of this group
    const bf16* bias;  // bias of this group, or null
    int ldb;           // elements between B rows (K, or ldb for kWgrad)
    int64_t aoff;      // bytes from A to the tile's first row (contiguous A) and
                       // first K column (kWgrad); A offsets below are relative
    int64_t ooff;      // output elements before the group's matrix (kWgrad)
  };
  // Tile fields are the same for the whole block: readfirstlane keeps them in
  // scalar registers (the vector register budget is tight).
  auto decode = [&](int tt) {
    Tile c;
    if constexpr (MODE == kWgrad) {
      // group-major, row tiles fastest: neighbouring blocks share B's column tile
      const int per = a.tiles_m * a.n_tiles_n;
      const int v = xcd_order<false>(tt, total);
      const int g = v / per, rr = v - g * per;
      const int nt = rr / a.tiles_m, mt = rr - nt * a.tiles_m;
      const int k0 = __builtin_amdgcn_readfirstlane(a.poff[a.g0 + g]);
      const int k1 = __builtin_amdgcn_readfirstlane(a.poff[a.g0 + g + 1]);
      c.row0 = mt * BM;
      c.rows = min(BM, a.M - c.row0);
      c.n0 = nt * BN;
      c.N = a.N;
      c.K = k1 - k0;
      c.bw = static_cast<const bf16*>(a.W) + k0;
      c.bias = nullptr;
      c.ldb = static_cast<int>(a.ldb);
      c.aoff = (static_cast<int64_t>(c.row0) * a.lda + k0) * 2;
      c.ooff = static_cast<int64_t>(g) * a.M * a.N;
      return c;
    }
    int rt, nt;
    decode_tile<(XR > 0)>(a, tt, total, nheavy, &rt, &nt);  // heavy: chunks across XCDs
    rt = __builtin_amdgcn_readfirstlane(rt);
    nt = __builtin_amdgcn_readfirstlane(nt);
    const RowTile& rtile = a.tiles[rt];
    const int group = __builtin_amdgcn_readfirstlane(rtile.group);
    const bool sh = (group == a.E);
    c.row0 = __builtin_amdgcn_readfirstlane(rtile.row0);
    c.rows = __builtin_amdgcn_readfirstlane(rtile.rows);
    c.n0 = nt * BN;
    c.N = sh ? a.Ns : a.N;
    c.K = sh ? a.Ks : a.K;
    c.bw = static_cast<const bf16*>(sh ? a.Wsh : a.W) +
           (sh ? 0 : static_cast<int64_t>(group) * c.N * c.K);
    c.bias = static_cast<const bf16*>(sh ? a.bias_sh : a.bias);
    if (c.bias && !sh) c.bias += static_cast<int64_t>(group) * c.N;
    c.ldb = c.K;
    c.aoff = MD::gather ? 0 : static_cast<int64_t>(c.row0) * a.lda * 2;
    c.ooff = 0;
    return c;
  };
  // token row (gathered A) behind tile row r, or r itself for contiguous A
  // (whose tile base holds the first row): gathered A must span < 4 GiB, a
  // contiguous one only a tile
  auto arow_of = [&](const Tile& c, int r) -> int {
    const int rr = min(r, c.rows - 1);
    return MD::gather ? a.row_token[c.row0 + rr] : rr;
  };
  // Load instruction j of this wave fills tile rows (wave + j NW) RPI ...; the
  // first JA instructions hold A rows (the last JX of them the extra rows of
  // heavy tiles), the rest B rows.  Sources are kept as 32-bit byte offsets
  // from the tensor (A) or the group's weights (B).
  constexpr int JA = BMX / (RPI * NW);
  constexpr int JX = (BMX - BM) / (RPI * NW);
  static_assert(BM % (RPI * NW) == 0, "A rows per load instruction");
  auto a_off = [&](int j, int arow) -> uint32_t {
    const int r = (wave + j * NW) * RPI + lr;
    const int chunk = (lane % CPR) ^ swz<CPR>(r);
    return static_cast<uint32_t>(arow) * static_cast<uint32_t>(a.lda * 2) + chunk * 16;
  };
  auto b_off = [&](const Tile& c, int j) -> uint32_t {
    if constexpr (BT) {
      // this lane's 16 bytes of the B region: row kr, chunk position pos, which
      // holds global chunk pos ^ swzt(kr) (clamped to a valid column chunk)
      const int o = ((wave + j * NW) * RPI - BMX) * RB + lane * 16;
      const int kr = o / (BN * 2), pos = (o % (BN * 2)) >> 4;
      const int nn = min(c.n0 + ((pos ^ swzt(kr)) << 3), c.N - 8);
      return static_cast<uint32_t>(kr) * static_cast<uint32_t>(c.N * 2) + nn * 2;
    } else {
      const int r = (wave + j * NW) * RPI + lr;
      const int chunk = (lane % CPR) ^ swz<CPR>(r);
      const int nn = min(c.n0 + r - BMX, c.N - 1);
      return static_cast<uint32_t>(nn) * static_cast<uint32_t>(c.ldb * 2) + chunk * 16;
    }
  };
  auto gate_of = [&](const Tile& c, int m) -> float {
    return m < c.rows ? (a.row_gate ? a.row_gate[c.row0 + m] : 1.f) : 0.f;
  };

  Tile cur = decode(t);
  uint32_t src[JPW];
#pragma unroll
  for (int j = 0; j < JPW; ++j)
    src[j] = j < JA ? a_off(j, arow_of(cur, (wave + j * NW) * RPI + lr)) : b_off(cur, j);
  if constexpr (MD::gated) {
#pragma unroll
    for (int g = 0; g < GPT; ++g)
      if (tid + g * NT < BMX) gate_s[0][tid + g * NT] = gate_of(cur, tid + g * NT);
  }
  const char* abase = static_cast<const char*>(a.A) + cur.aoff;
  const char* bbase = reinterpret_cast<const char*>(cur.bw);
  // K steps of this block: [kb, kb + ksteps) of the tile's K / BK
  int kb = 0, ksteps = cur.K / BK;
  if (part >= 0) {
    kb = part * ksteps / S;
    ksteps = (part + 1) * ksteps / S - kb;
  }
  // bytes per k of B: 2 (K-contiguous rows) or one [K, N] row
  uint32_t bstep = BT ? static_cast<uint32_t>(cur.N) * 2 : 2;
  bool heavy = XR > 0 && cur.rows > BM;
  auto issue = [&](int stage, int k0) {
#pragma unroll
    for (int j = 0; j < JPW; ++j) {
      if (XR > 0 && !heavy && j >= JA - JX && j < JA) continue;
      char* dst = smem + stage * STAGE + (wave + j * NW) * RPI * RB;
      if (j < JA)
        lds_dma16(abase + src[j] + static_cast<uint32_t>(k0) * 2u, dst);
      else  // the weights (not the activations B holds in kWgrad)
        lds_dma16<NTB && MODE != kWgrad ? kCpolNT : 0>(
            bbase + src[j] + static_cast<uint32_t>(k0) * bstep, dst);
    }
  };
#pragma unroll
  for (int p = 0; p < NS - 1; ++p)
    if (p < ksteps) issue(p, (kb + p) * BK);

  int gb = 0;
  for (;;) {
    const int tn = t + gridDim.x;
    const bool has_next = PERSIST && tn < total;
    Tile nxt = cur;
    if (has_next) nxt = decode(tn);
    int ntok[JA];
    float ngate[GPT];
#pragma unroll
    for (int j = 0; j < JA; ++j) ntok[j] = 0;
#pragma unroll
    for (int g = 0; g < GPT; ++g) ngate[g] = 0.f;

    // The tile's K loop, K split and epilogue over MU row blocks per wave (MI,
    // or MIX for a heavy tile; each path keeps only its own accumulators).
    // Returns true when this block is done (a part of a split tile that did
    // not arrive last).
    auto body = [&](auto mu) -> bool {
      constexpr int MU = decltype(mu)::value;
      f32x16 acc[MU][NI];
#pragma unroll
      for (int i = 0; i < MU; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

      const int KT = ksteps;
        for (int kt = 0; kt < KT; ++kt) {
          // this lane's loads of stage kt have landed once at most the loads of the
          // later stages already issued (min(NS - 2, KT - 1 - kt) of them) are
          // pending; the first step of a tile waits for everything (the previous
          // tile's epilogue stores were issued after this tile's first stages)
          if (kt == 0) {
            wait_vmcnt<0>();
          } else {
            wait_stages<NS, JPW>(KT - 1 - kt);
          }
          // Every lane's loads of stage kt landed; every wave finished reading stage
          // kt - 1.  A plain s_barrier: a workgroup fence would also wait for the
          // later stages.
          __builtin_amdgcn_s_barrier();
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          if (kt == 0 && has_next) {
            // next tile's token rows and gates: loaded now, used after the K loop
#pragma unroll
            for (int j = 0; j < JA; ++j) ntok[j] = arow_of(nxt, (wave + j * NW) * RPI + lr);
            if constexpr (MD::gated) {
#pragma unroll
              for (int g = 0; g < GPT; ++g)
                if (tid + g * NT < BMX) ngate[g] = gate_of(nxt, tid + g * NT);
            }
          }
          if (kt + NS - 1 < KT) issue((kt + NS - 1) % NS, (kb + kt + NS - 1) * BK);
          const char* st = smem + (kt % NS) * STAGE;
          // fragments of k16 step s + 1 are read while the MFMAs of step s run
          bf16x8_t fa[2][MU], fb[2][NI];
          auto frags = [&](int s, int buf) {
            const int cb = ((2 * s + (lane >> 5)) ^ rsw) * 16;
#pragma unroll
            for (int i = 0; i < MU; ++i)
              fa[buf][i] = *reinterpret_cast<const bf16x8_t*>(st + aoffs[i] + cb);
            if constexpr (BT) {
#pragma unroll
              for (int j = 0; j < NI; ++j) {
                const char* p = st + btoffs[j] + s * 16 * (BN * 2);
                const i16x4 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 4 * (BN * 2));
                fb[buf][j] = __builtin_bit_cast(
                    bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
              }
            } else {
#pragma unroll
              for (int j = 0; j < NI; ++j)
                fb[buf][j] = *reinterpret_cast<const bf16x8_t*>(st + boffs[j] + cb);
            }
          };
          frags(0, 0);
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            if (s + 1 < KS) frags(s + 1, (s + 1) & 1);
#pragma unroll
            for (int i = 0; i < MU; ++i)
#pragma unroll
              for (int j = 0; j < NI; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s & 1][i], fb[s & 1][j],
                                                                    acc[i][j], 0, 0, 0);
          }
          // Instruction order for the scheduler: the first step's fragment reads,
          // then each step's MFMAs with the next step's reads spread between them.
          constexpr int NRD = MU + (BT ? 2 : 1) * NI;  // fragment reads per k16 step
          __builtin_amdgcn_sched_group_barrier(0x100, NRD, 0);
          sched_steps<0, KS - 1, NRD, MU * NI>();
          __builtin_amdgcn_sched_group_barrier(0x008, MU * NI, 0);
        }
      // Every wave is done reading this tile's stages (and every load of it has
      // landed: the last iteration waited for all of them).
      __builtin_amdgcn_s_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (!PERSIST && part >= 0) {
        // Park this part's accumulators in its slot, lane-major (one 16-byte
        // store per lane: 1 KiB per wave instruction).  The last part to arrive
        // adds the S slots in part order (its own from registers) and goes on to
        // the epilogue; the others are done.
        // a slot holds MIX row blocks (heavy or not, the parts of one tile agree)
        constexpr int F4S = MIX * NI * 4;  // float4 per lane of a slot
        const int u = static_cast<int>(blockIdx.x) - D, ti = u / S;
        float4* mine = reinterpret_cast<float4*>(a.kpart) + static_cast<int64_t>(u) * F4S * NT;
#pragma unroll
        for (int i = 0; i < MU; ++i)
#pragma unroll
          for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c)
              mine[((i * NI + j) * 4 + c) * NT + tid] =
                  make_float4(acc[i][j][4 * c], acc[i][j][4 * c + 1], acc[i][j][4 * c + 2],
                              acc[i][j][4 * c + 3]);
        // Each wave waits until its stores have reached the L2; the workgroup
        // barrier (with its workgroup-scope fences) orders every wave's stores
        // before thread 0's agent-scope release, which writes this XCD's L2 back,
        // and the arrival count; the last part invalidates its stale L2 lines
        // (agent-scope acquire) before any wave reads the other parts' slots.
        // One release per part and one acquire per tile: each is a whole-L2
        // operation, so no wave beyond the first does either.
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        wait_vmcnt<0>();
        __syncthreads();
        if (tid == 0) {
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
          // the write-back has completed before the arrival is counted (an
          // explicit wait: the compiler drops its own here, as its counter model
          // already saw vmcnt at zero)
          wait_vmcnt<0>();
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          const int before =
              __hip_atomic_fetch_add(a.ksem + ti, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          split_last = before == S - 1;
          if (before == S - 1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
        __syncthreads();
        if (!split_last) return true;
        const float4* slots0 =
            reinterpret_cast<const float4*>(a.kpart) + static_cast<int64_t>(ti) * S * F4S * NT;
#pragma unroll
        for (int i = 0; i < MU; ++i)
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            f32x16 sum;
#pragma unroll
            for (int q = 0; q < 16; ++q) sum[q] = 0.f;
            for (int p = 0; p < S; ++p) {
              if (p == part) {
#pragma unroll
                for (int q = 0; q < 16; ++q) sum[q] += acc[i][j][q];
              } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                  const float4 v =
                      slots0[(static_cast<int64_t>(p) * F4S + (i * NI + j) * 4 + c) * NT + tid];
                  sum[4 * c] += v.x;
                  sum[4 * c + 1] += v.y;
                  sum[4 * c + 2] += v.z;
                  sum[4 * c + 3] += v.w;
                }
              }
            }
            acc[i][j] = sum;
          }
        if (tid == 0) a.ksem[ti] = 0;  // ready for the next launch (kernel end orders it)
      }
      if (has_next) {
#pragma unroll
        for (int j = 0; j < JPW; ++j) src[j] = j < JA ? a_off(j, ntok[j]) : b_off(nxt, j);
        abase = static_cast<const char*>(a.A) + nxt.aoff;
        bbase = reinterpret_cast<const char*>(nxt.bw);
        bstep = BT ? static_cast<uint32_t>(nxt.N) * 2 : 2;
        const int KTn = nxt.K / BK;
#pragma unroll
        for (int p = 0; p < NS - 1; ++p)
          if (p < KTn) issue(p, p * BK);
        if constexpr (MD::gated) {
#pragma unroll
          for (int g = 0; g < GPT; ++g)
            if (tid + g * NT < BMX) gate_s[gb ^ 1][tid + g * NT] = ngate[g];
        }
      }

      // epilogue of tile t (gates of this tile are in gate_s[gb]).  Stores address
      // the tile from one uniform base with 32-bit offsets; a full tile takes the
      // path without bounds checks; the activation is chosen once per tile.
      float bv[NI];
      int ncol[NI];
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        ncol[j] = wn * WTN + j * 32 + (lane & 31);  // column inside the tile
        const int n = cur.n0 + ncol[j];
        bv[j] = (cur.bias && n < cur.N) ? bf16_to_f32(cur.bias[n].bits) : 0.f;
      }
      constexpr int OE = MD::out_f32 ? 4 : 2;  // output element bytes
      char* obase = static_cast<char*>(a.out) +
                    (cur.ooff + static_cast<int64_t>(cur.row0) * a.ldo + cur.n0) * OE;
      char* xbase = MODE == kUpTrain ? static_cast<char*>(a.aux) +
                                           (static_cast<int64_t>(cur.row0) * a.ldo + cur.n0) * OE
                                     : nullptr;
      const uint32_t ldo = static_cast<uint32_t>(a.ldo);
      // CHK: some rows or columns of the tile are missing; then rows are
      // checked per 32-row block, only in blocks that reach past the tile's rows.
      auto epilogue = [&](auto checked, auto relu) {
        constexpr bool CHK = decltype(checked)::value;
        constexpr bool RELU = decltype(relu)::value;
#pragma unroll
        for (int i = 0; i < MU; ++i) {
          const bool rchk = CHK && arow_blk(i) + 32 > cur.rows;
#pragma unroll
         for (int qh = 0; qh < 16; qh += 8) {
          // kDz: eight rows' pre-activations are loaded before any of their
          // results is stored (a load after a possibly aliasing store would wait
          // out a full memory latency)
          uint16_t zr[MODE == kDz ? 8 : 1][MODE == kDz ? NI : 1];
          if constexpr (MODE == kDz) {
#pragma unroll
            for (int qq = 0; qq < 8; ++qq) {
              const int q = qh + qq;
              // partial tiles read a clamped valid element (no branch); the
              // value is used only where the result is stored
              const int m = arow_blk(i) + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
              const uint32_t orow = static_cast<uint32_t>(rchk ? min(m, cur.rows - 1) : m) * ldo;
#pragma unroll
              for (int j = 0; j < NI; ++j) {
                const int nc = CHK ? min(ncol[j], cur.N - 1 - cur.n0) : ncol[j];
                zr[qq][j] = *reinterpret_cast<const uint16_t*>(
                    obase + (orow + static_cast<uint32_t>(nc)) * OE);
              }
            }
          }
#pragma unroll
          for (int q = qh; q < qh + 8; ++q) {
            const int m = arow_blk(i) + (q >> 2) * 8 + (lane >> 5) * 4 + (q & 3);
            if (rchk && m >= cur.rows) continue;
            const uint32_t orow = static_cast<uint32_t>(m) * ldo;
            const float g = MD::gated ? gate_s[gb][m] : 1.f;
#pragma unroll
            for (int j = 0; j < NI; ++j) {
              if (CHK && cur.n0 + ncol[j] >= cur.N) continue;
              const float z = acc[i][j][q] + bv[j];
              const uint32_t off = (orow + static_cast<uint32_t>(ncol[j])) * OE;
              if constexpr (MD::fwd_act) {
                const float h = RELU ? fmaxf(z, 0.f) : gelu_erf(z);
                *reinterpret_cast<uint16_t*>(obase + off) = f32_to_bf16(h);
                if constexpr (MODE == kUpTrain)
                  *reinterpret_cast<uint16_t*>(xbase + off) = f32_to_bf16(z);
              } else if constexpr (MODE == kDz) {
                const float pre = bf16_to_f32(zr[q - qh][j]);
                const float da = RELU ? (pre > 0.f ? 1.f : 0.f) : gelu_erf_grad(pre);
                *reinterpret_cast<uint16_t*>(obase + off) = f32_to_bf16(g * z * da);
              } else if constexpr (MODE == kWgrad) {
                *reinterpret_cast<uint16_t*>(obase + off) = f32_to_bf16(z);
              } else {
                *reinterpret_cast<float*>(obase + off) = g * z;
              }
            }
          }
         }
          // one 32-row block at a time: keeps the epilogue's temporaries few
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      // A tile whose columns all lie past its group's N (the shared expert's
      // narrower projection) stores nothing; the clamps of the partial-tile
      // path assume at least one valid column.
      const bool full = cur.rows == MU * 32 * WM && cur.n0 + BN <= cur.N;
      if (cur.n0 >= cur.N) {
      } else if ((MD::fwd_act || MODE == kDz) && a.act == MOE_ACT_RELU) {
        if (full) epilogue(std::false_type{}, std::true_type{});
        else epilogue(std::true_type{}, std::true_type{});
      } else {
        if (full) epilogue(std::false_type{}, std::false_type{});
        else epilogue(std::true_type{}, std::false_type{});
      }
      return false;
    };
    bool done;
    if constexpr (XR > 0) {
      done = heavy ? body(std::integral_constant<int, MIX>{})
                   : body(std::integral_constant<int, MI>{});
    } else {
      done = body(std::integral_constant<int, MI>{});
    }
    if (done) return;
    if (!has_next) break;
    cur = nxt;
    t = tn;
    ksteps = cur.K / BK;
    gb ^= 1;
  }
}

// Row tiles of BM rows per group, groups in order, from the dispatch offsets,
// and each row's gate: topk_w[token, slot] (k > 0) or topk_w[row] (k = 0,
// one gate per routed row); 1 for the shared expert's rows.
__global__ __launch_bounds__(1024) void build_tiles_kernel(const int32_t* __restrict__ offsets,
                                                           int G, int BM, int extra, int E, int k,
                                                           const int32_t* __restrict__ row_token,
                                                           const int32_t* __restrict__ row_slot,
                                                           const float* __restrict__ topk_w,
                                                           RowTile* __restrict__ tiles,
                                                           int32_t* __restrict__ ntiles,
                                                           float* __restrict__ row_gate) {
  // block 0 builds the tile list; every block fills the gates of its
  // kMaxExperts rows (the grid covers the host's bound on the row count)
  __shared__ int32_t wsum[kMaxExperts / 64];
  if (blockIdx.x == 0) build_tile_list(offsets, G, BM, extra, tiles, ntiles, wsum);
  const int routed = offsets[E], nrows = offsets[G];
  const int r = static_cast<int>(blockIdx.x) * kMaxExperts + static_cast<int>(threadIdx.x);
  if (r < nrows)
    row_gate[r] = r >= routed ? 1.0f
                  : k > 0     ? topk_w[static_cast<int64_t>(row_token[r]) * k + row_slot[r]]
                              : topk_w[r];
}

static GemmArgs up_args(const FfnArgs& f, int BN) {
  const int64_t ldh = f.F > f.Fs ? f.F : f.Fs;
  GemmArgs u{};
  u.tiles = f.tiles;
  u.ntiles = f.ntiles;
  u.E = f.E;
  u.A = f.x;
  u.lda = f.d;
  u.row_token = f.row_token;
  u.row_gate = f.row_gate;
  u.W = f.W1;
  u.Wsh = f.Ws1;
  u.bias = f.b1;
  u.bias_sh = f.bs1;
  u.N = f.F;
  u.K = f.d;
  u.Ns = f.Fs;
  u.Ks = f.d;
  u.n_tiles_n = static_cast<int>(ceil_div(ldh, BN));
  u.out = f.H;
  u.aux = f.Z;
  u.ldo = ldh;
  u.act = f.act;
  u.kpart = f.kpart;
  u.ksem = f.ksem;
  return u;
}

static GemmArgs down_args(const FfnArgs& f, int BN) {
  const int64_t ldh = f.F > f.Fs ? f.F : f.Fs;
  GemmArgs dn = up_args(f, BN);
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
  dn.n_tiles_n = static_cast<int>(ceil_div(f.d, BN));
  dn.out = f.y_rows;
  dn.ldo = f.d;
  // the input-gradient pass multiplies by no gate (the gate sits in dz)
  if (f.pass == kPassDgrad) dn.row_gate = nullptr;
  return dn;
}

template <typename T, int BM, int BNU, int BND, int BK, int WM, int WN, int M1, bool BT>
static void run_generic(const GemmPlan& gp, const FfnArgs& f, hipStream_t st) {
  const GemmArgs u = up_args(f, BNU);
  const int64_t gu = gp.tiles_max * u.n_tiles_n;
  if (gu > 0)
    grouped_gemm_kernel<T, BM, BNU, BK, WM, WN, M1, BT>
        <<<static_cast<unsigned>(gu), WM * WN * 64, 0, st>>>(u);
  const GemmArgs dn = down_args(f, BND);
  const int64_t gd = gp.tiles_max * dn.n_tiles_n;
  if (gd > 0)
    grouped_gemm_kernel<T, BM, BND, BK, WM, WN, kDown, BT>
        <<<static_cast<unsigned>(gd), WM * WN * 64, 0, st>>>(dn);
}

// Compute units of the current device (host query, no synchronisation).
static int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  return n;
}

// Persistent launch: as many blocks as can be resident, capped by the tile
// count; otherwise one block per tile, plus up to `slots` more for the K split
// of a last round (split: partial tiles reserved, 0 for none).
template <int BM, int BN, int BK, int NS, int WM, int WN, int OCC, int PERSIST, int MODE,
          bool BT, int XR = 0, int NTB = 0>
static void launch_dma(GemmArgs g, int64_t tiles, int split, hipStream_t st) {
  if (tiles <= 0) return;
  auto kern = grouped_gemm_dma_kernel<BM, BN, BK, NS, WM, WN, OCC, PERSIST, MODE, BT, XR, NTB>;
  const size_t lds = static_cast<size_t>(NS) * (BM + XR * WM * 32 + BN) * BK * 2;
  static int per_cu = [&] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, kern, WM * WN * 64, lds) != hipSuccess ||
        b < 1)
      b = 1;
    return b;
  }();
  g.slots = 0;
  g.smax = 1;
  if (!PERSIST && split > 0 && g.kpart && g.ksem) {
    // the shared expert's K counts too when there is one
    const bool sh = g.Ns > 0 && g.Ks > 0;
    const int kt_min = (sh ? std::min(g.K, g.Ks) : g.K) / BK;
    g.smax = std::min(kSplitMax, kt_min / kSplitMinSteps);
    g.slots = std::min(cu_count() * per_cu, split);
  }
  const int64_t grid = PERSIST ? std::min<int64_t>(tiles, static_cast<int64_t>(cu_count()) * per_cu)
                               : tiles + (g.smax > 1 ? g.slots : 0);
  kern<<<static_cast<unsigned>(grid), WM * WN * 64, lds, st>>>(g);
}

template <int BM, int BNU, int BND, int BK, int NS, int WM, int WN, int OCC, int PERSIST,
          int WMD, int WND, int SPLIT, int NTB, int M1, bool BT, int XR = 0>
static void run_dma(const GemmPlan& gp, const FfnArgs& f, hipStream_t st) {
  const GemmArgs u = up_args(f, BNU);
  launch_dma<BM, BNU, BK, NS, WM, WN, OCC, PERSIST, M1, BT, XR, NTB>(
      u, gp.tiles_max * u.n_tiles_n, SPLIT, st);
  const GemmArgs dn = down_args(f, BND);
  launch_dma<BM, BND, BK, NS, WMD, WND, OCC, PERSIST, kDown, BT, XR, NTB>(
      dn, gp.tiles_max * dn.n_tiles_n, SPLIT, st);
}

// The two GEMMs of one pass over the grouped rows; M1 is the first GEMM's mode,
// BT whether B is stored [K, N].
template <int M1, bool BT>
static void run_pass(const GemmPlan& gp, const FfnArgs& f, hipStream_t st) {
  switch (gp.shape) {
    case kGemmF32: run_generic<float, 64, 64, 64, 32, 2, 2, M1, BT>(gp, f, st); break;
    case kGemmBf16Large: run_generic<bf16, 128, 128, 128, 64, 2, 2, M1, BT>(gp, f, st); break;
    case kGemmBf16Mid: run_generic<bf16, 64, 128, 128, 64, 1, 4, M1, BT>(gp, f, st); break;
    case kGemmBf16Small: run_generic<bf16, 32, 128, 128, 64, 1, 4, M1, BT>(gp, f, st); break;
#define MOE_RUN_DMA(C)                                                                     \
  run_dma<C.BM, C.BNU, C.BND, C.BK, C.NS, C.WM, C.WN, C.OCC, C.PERSIST, C.WMD, C.WND, C.SPLIT, \
          C.NTB, M1, BT>(gp, f, st)
    case kGemmDmaLarge:
      // the forward's tile list may hold heavy tiles (rows past BM)
      if constexpr (M1 == kUp && !BT) {
        constexpr DmaCfg C = kDmaLarge;
        static_assert(C.WM == C.WMD && C.NS == 2 && !C.PERSIST, "heavy tiles");
        if (gp.extra > 0) {
          run_dma<C.BM, C.BNU, C.BND, C.BK, C.NS, C.WM, C.WN, C.OCC, C.PERSIST, C.WMD, C.WND,
                  C.SPLIT, C.NTB, M1, BT, 1>(gp, f, st);
          break;
        }
      }
      MOE_RUN_DMA(kDmaLarge);
      break;
    case kGemmDmaTall: MOE_RUN_DMA(kDmaTall); break;
    case kGemmDmaMid: MOE_RUN_DMA(kDmaMid); break;
    case kGemmDmaSmall: MOE_RUN_DMA(kDmaSmall); break;
    default: MOE_RUN_DMA(kDmaSkinny); break;
#undef MOE_RUN_DMA
  }
}

template <int BM, int BN, int BK, int NS, int WM, int WN, int OCC>
static void run_wgrad_dma(const WgradGemm& w, hipStream_t st) {
  GemmArgs g{};
  g.A = w.A;
  g.lda = w.lda;
  g.W = w.B;
  g.ldb = w.ldb;
  g.poff = w.poff;
  g.g0 = w.g0;
  g.E = w.groups;
  g.M = w.M;
  g.N = w.N;
  g.out = w.C;
  g.ldo = w.N;
  g.tiles_m = static_cast<int>(ceil_div(w.M, BM));
  g.n_tiles_n = static_cast<int>(ceil_div(w.N, BN));
  launch_dma<BM, BN, BK, NS, WM, WN, OCC, 0, kWgrad, false>(
      g, static_cast<int64_t>(w.groups) * g.tiles_m * g.n_tiles_n, 0, st);
}

bool wgrad_dma_fits(int shape, const WgradGemm& w) {
  if (shape != kGemmDmaLarge && shape != kGemmDmaMid && shape != kGemmDmaSmall) return false;
  // 16-byte LDS-DMA chunks along K; 32-bit byte offsets inside a row tile of
  // A (whose base is per tile) and inside B
  const bool k16 = w.lda % 8 == 0 && w.ldb % 8 == 0 &&
                   reinterpret_cast<uintptr_t>(w.A) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(w.B) % 16 == 0;
  return k16 && int64_t(kDmaLarge.BM) * w.lda * 2 < (int64_t(1) << 31) &&
         int64_t(w.N) * w.ldb * 2 < (int64_t(1) << 31) && int64_t(w.M) * w.N < (int64_t(1) << 31);
}

hipError_t launch_wgrad_dma(int shape, const WgradGemm& w, hipStream_t st) {
  if (w.groups <= 0 || w.M <= 0 || w.N <= 0) return hipSuccess;
  if (shape == kGemmDmaLarge) {
    constexpr DmaCfg C = kDmaLarge;
    run_wgrad_dma<C.BM, C.BNU, C.BK, C.NS, C.WM, C.WN, C.OCC>(w, st);
  } else if (shape == kGemmDmaSmall) {
    // groups of at most a few rows (one or two K steps): 256 x 128 tiles of 4
    // waves with 32-wide K steps, two blocks per CU, so one block's loads
    // overlap the other's epilogue writes
    run_wgrad_dma<256, 128, 32, 2, 2, 2, 2>(w, st);
  } else {
    constexpr DmaCfg C = kDmaMid;
    run_wgrad_dma<C.BM, C.BNU, C.BK, C.NS, C.WM, C.WN, C.OCC>(w, st);
  }
  return hipGetLastError();
}

hipError_t launch_ffn(const GemmPlan& gp, const FfnArgs& f, hipStream_t st) {
  const int G = f.E + (f.Fs > 0 ? 1 : 0);
  if (!f.tiles_ready)
    build_tiles_kernel<<<static_cast<unsigned>(std::max<int64_t>(1, ceil_div(f.rows_max,
                                                                              kMaxExperts))),
                         kMaxExperts, 0, st>>>(f.offsets, G, gp.BM,
                                                  f.pass == kPassForward ? gp.extra : 0, f.E,
                                                  f.row_gates ? 0 : f.k, f.row_token,
                                                  f.row_slot, f.topk_w, f.tiles, f.ntiles,
                                                  f.row_gate);
  switch (f.pass) {
    case kPassForward: run_pass<kUp, false>(gp, f, st); break;
    case kPassForwardTrain: run_pass<kUpTrain, false>(gp, f, st); break;
    default: run_pass<kDz, true>(gp, f, st); break;
  }
  return hipGetLastError();
}

}  // namespace moe
