// Grouped GEMM over the selected experts with a fused SiLU * weight epilogue,
// and the same tiled GEMM in a dense mode for the plain value projection.
//
// Grouped mode: for every expert e, the pairs routed to it (rows perm[
// expert_off[e] .. expert_off[e+1])) form the A operand by gathering token rows
// of x; the expert's [N, d] weight (nn.Linear layout, k contiguous) is the B
// operand.  z = x_t W_e^T is accumulated in fp32 on bf16 MFMA, then
// y = w[pair] * SiLU(z) is computed in fp32 and stored, rounded once to fp16,
// to the pair's own partial row
// (page "MoVA: routing the value vectors ...", section "Where the routing
// happens": SiLU on each expert's output, weighted by the routing weight).
// Each partial row is written by exactly one tile, so no atomics are needed;
// the k-way sum happens afterwards in a fixed slot order.
//
// Dense mode: one weight [N, d], A rows are the tokens in order, and the
// epilogue stores z rounded once to bf16 (the dense layers' plain v_proj,
// section "So what does it cost?").
//
// Block tile BM x BN (BM = 256 or 128, BN = 256), k steps of 64, 8 waves in a
// 2 x 4 grid, each wave owning a BM/2 x 64 sub-tile (BM/32 x 4 MFMA 16x16x32
// tiles).  Operand tiles go global -> LDS with direct (global_load_lds)
// 16-byte loads, double buffered: the loads of step k+1 are in flight while
// step k's MFMAs run, with one barrier per step.  A staged row holds 64 bf16
// (128 B) whose 16-byte chunks sit at chunk ^ (row & 7), so the MFMA fragment
// reads hit distinct banks; since a direct load writes 64 consecutive 16-byte
// slots, the swizzle is applied when choosing which global chunk each lane
// loads.
//
// A tile with at most BM/2 valid rows runs its lower waves through a copy of
// the k loop that only loads and synchronises (no MFMA work on empty rows).
//
// Work order: tile id -> (expert, n-tile, m-tile), m fastest, so tiles that
// share an expert's weight slab are adjacent.  Workgroups are dealt round
// robin over the 8 XCDs; block b runs tile (b % 8) * per_xcd + b / 8, giving
// each XCD one contiguous run of tiles (and its L2 the weights they share).
#include "common.h"
#include "kernels.h"

namespace mova {

constexpr int kBMGrouped = 256;  // M tile of the grouped (routed) mode
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int kThreads = 512;
constexpr int kRowBytes = BK * 2;  // 128 B per staged row
constexpr int kTileB = BN * kRowBytes;  // 32 KB
constexpr int kXcds = 8;
constexpr int kLoadsB = BN * kRowBytes / 1024 / (kThreads / 64);  // 4 direct loads per wave

template <int kBM>
struct Tile {
  static constexpr int kTileA = kBM * kRowBytes;                       // 32 or 16 KB
  static constexpr int kStage = kTileA + kTileB;                       // 64 or 48 KB per buffer
  static constexpr int kLoadsA = kBM * kRowBytes / 1024 / (kThreads / 64);  // 4 or 2
  static constexpr int kMI = kBM / 32;                                 // MFMA row tiles per wave
};

int gemm_block_m() { return kBMGrouped; }

int gemm_max_mtiles(int T, int k, int E) { return (int)(((long long)T * k) / kBMGrouped) + E; }

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ (row & 7)) << 4);
}

template <int kBM>
struct TileCtx {
  const char* a_src[Tile<kBM>::kLoadsA];  // per lane: (gathered) x row + its chunk
  const char* b_src[kLoadsB];             // per lane: weight row + its chunk
};

// Direct loads of one k step: A block j (rows 8j .. 8j+7) for j = wave * kLoadsA + i,
// B block j for j = wave * kLoadsB + i.
template <int kBM>
__device__ __forceinline__ void issue_loads(const TileCtx<kBM>& c, char* stage, int wave,
                                            int k_byte) {
#pragma unroll
  for (int i = 0; i < Tile<kBM>::kLoadsA; ++i)
    __builtin_amdgcn_global_load_lds((const void*)(c.a_src[i] + k_byte),
                                     (lds_void*)(stage + (wave * Tile<kBM>::kLoadsA + i) * 1024),
                                     16, 0, 0);
#pragma unroll
  for (int i = 0; i < kLoadsB; ++i)
    __builtin_amdgcn_global_load_lds(
        (const void*)(c.b_src[i] + k_byte),
        (lds_void*)(stage + Tile<kBM>::kTileA + (wave * kLoadsB + i) * 1024), 16, 0, 0);
}

// One k step (two 32-wide MFMA steps) of the wave's BM/2 x 64 sub-tile.
template <int kBM>
__device__ __forceinline__ void mma_step(f32x4 (&acc)[Tile<kBM>::kMI][4], const char* stage,
                                         int wm, int wn, int q, int r16) {
  constexpr int MI = Tile<kBM>::kMI;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int chunk = ks * 4 + q;
    Frag16 fa[MI], fb[4];
#pragma unroll
    for (int i = 0; i < MI; ++i) fa[i].u = load16(stage + swz(wm * (kBM / 2) + i * 16 + r16, chunk));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fb[j].u = load16(stage + Tile<kBM>::kTileA + swz(wn * 64 + j * 16 + r16, chunk));
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(fa[i].h, fb[j].h, acc[i][j]);
  }
}

// kDense = false: grouped mode (perm, topk_w, expert_off, tile_base, partial).
// kDense = true: dense mode over T token rows and one [N, d] weight (out).
template <int kBM, bool kDense>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ W,
    const int32_t* __restrict__ perm, const float* __restrict__ topk_w,
    const int32_t* __restrict__ expert_off, const int32_t* __restrict__ tile_base,
    f16_t* __restrict__ partial, bf16_t* __restrict__ out, int T, int d, int N, int E, int k) {
  using TL = Tile<kBM>;
  extern __shared__ __attribute__((aligned(1024))) char smem[];  // 2 stages
  __shared__ int tile_pair[kDense ? 1 : kBM];
  __shared__ float tile_w[kDense ? 1 : kBM];

  const int NT = ceil_div(N, BN);
  const int MTd = kDense ? ceil_div(T, kBM) : 0;
  const int total = kDense ? MTd * NT : tile_base[E] * NT;
  const int per_xcd = ceil_div(total, kXcds);
  const int local = blockIdx.x / kXcds;
  if (local >= per_xcd) return;
  const int wid = (blockIdx.x % kXcds) * per_xcd + local;
  if (wid >= total) return;

  int e = 0, nt, row0, rows;
  if (kDense) {
    nt = wid / MTd;
    row0 = (wid % MTd) * kBM;
    rows = min(kBM, T - row0);
  } else {
    // Expert owning this tile: the last e with tile_base[e] * NT <= wid.
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tile_base[mid] * NT <= wid) lo = mid; else hi = mid;
    }
    e = lo;
    const int me = tile_base[e + 1] - tile_base[e];
    const int rel = wid - tile_base[e] * NT;
    nt = rel / me;
    row0 = expert_off[e] + (rel % me) * kBM;
    rows = min(kBM, expert_off[e + 1] - row0);
  }
  const int n0 = nt * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int q = lane >> 4, r16 = lane & 15;

  if (!kDense) {
    for (int r = tid; r < kBM; r += kThreads) {
      const int pair = perm[row0 + min(r, rows - 1)];
      tile_pair[r] = pair;
      tile_w[r] = topk_w[pair];
    }
  }

  // Lane -> (row, chunk) of each direct load: LDS block j holds rows 8j .. 8j+7,
  // lane l lands in slot l, i.e. row 8j + l/8, physical chunk l%8, which holds
  // logical chunk (l%8) ^ (row & 7).  Rows past the tile's valid rows (or past
  // N) load a clamped row and are never stored.
  TileCtx<kBM> c;
#pragma unroll
  for (int i = 0; i < TL::kLoadsA; ++i) {
    const int row = (wave * TL::kLoadsA + i) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ (row & 7);
    const int rr = row0 + min(row, rows - 1);
    const int token = kDense ? rr : perm[rr] / k;
    c.a_src[i] = reinterpret_cast<const char*>(x + (size_t)token * d) + chunk * 16;
  }
#pragma unroll
  for (int i = 0; i < kLoadsB; ++i) {
    const int row = (wave * kLoadsB + i) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ (row & 7);
    const int n = min(n0 + row, N - 1);
    c.b_src[i] = reinterpret_cast<const char*>(W + ((size_t)e * N + n) * d) + chunk * 16;
  }

  f32x4 acc[TL::kMI][4];
#pragma unroll
  for (int i = 0; i < TL::kMI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KT = d / BK;
  issue_loads<kBM>(c, smem, wave, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const bool active = wm * (kBM / 2) < rows;  // wave-uniform
  if (active) {
    for (int kt = 0; kt < KT; ++kt) {
      char* cur = smem + (kt & 1) * TL::kStage;
      if (kt + 1 < KT)
        issue_loads<kBM>(c, smem + ((kt + 1) & 1) * TL::kStage, wave, (kt + 1) * kRowBytes);
      mma_step<kBM>(acc, cur, wm, wn, q, r16);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  } else {
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + 1 < KT)
        issue_loads<kBM>(c, smem + ((kt + 1) & 1) * TL::kStage, wave, (kt + 1) * kRowBytes);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    return;
  }

  // Epilogue.  Grouped: y = w * SiLU(z) into the pair's partial row (fp16).
  // Dense: z into the token's output row (bf16).
#pragma unroll
  for (int i = 0; i < TL::kMI; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = wm * (kBM / 2) + i * 16 + q * 4 + v;
      if (r < rows) {
        if (kDense) {
          bf16_t* dst = out + (size_t)(row0 + r) * N + n0 + wn * 64 + r16;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (n0 + wn * 64 + j * 16 + r16 < N) dst[j * 16] = (bf16_t)acc[i][j][v];
        } else {
          const int pair = tile_pair[r];
          const float wt = tile_w[r];
          f16_t* dst = partial + (size_t)pair * N + n0 + wn * 64 + r16;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (n0 + wn * 64 + j * 16 + r16 < N) dst[j * 16] = (f16_t)(wt * siluf(acc[i][j][v]));
        }
      }
    }
  }
}

template <int kBM, bool kDense>
hipError_t launch_tiles(const GemmArgs& a, long long tiles, hipStream_t stream) {
  auto kern = gemm_kernel<kBM, kDense>;
  constexpr int smem = 2 * Tile<kBM>::kStage;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute((const void*)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  const long long grid = ((tiles + kXcds - 1) / kXcds) * kXcds;
  kern<<<dim3((unsigned)grid), kThreads, smem, stream>>>(a.x, a.W, a.perm, a.topk_w, a.expert_off,
                                                         a.tile_base, a.partial, a.out, a.T, a.d,
                                                         a.N, a.E, a.k);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t stream) {
  const long long ub = (long long)gemm_max_mtiles(a.T, a.k, a.E) * ceil_div(a.N, BN);
  return launch_tiles<kBMGrouped, false>(a, ub, stream);
}

int dense_gemm_block_m(int T, int N) {
  // 256-row tiles once they fill the 256 CUs at least once; 128-row tiles
  // (twice the workgroups) below that.
  const long long tiles256 = (long long)ceil_div(T, 256) * ceil_div(N, BN);
  return tiles256 >= 256 ? 256 : 128;
}

hipError_t launch_dense_gemm(const GemmArgs& a, hipStream_t stream) {
  const int bm = dense_gemm_block_m(a.T, a.N);
  const long long tiles = (long long)ceil_div(a.T, bm) * ceil_div(a.N, BN);
  return bm == 256 ? launch_tiles<256, true>(a, tiles, stream)
                   : launch_tiles<128, true>(a, tiles, stream);
}

}  // namespace mova
