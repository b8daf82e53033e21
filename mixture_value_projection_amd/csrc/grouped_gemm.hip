// Grouped GEMM over the selected experts with a fused SiLU * weight epilogue.
//
// For every expert e, the pairs routed to it (rows perm[expert_off[e] ..
// expert_off[e+1])) form the A operand by gathering token rows of x; the
// expert's [N, d] weight (nn.Linear layout, k contiguous) is the B operand.
// z = x_t W_e^T is accumulated in fp32 on bf16 MFMA, then
// y = w[pair] * SiLU(z) is computed in fp32 and stored, rounded once to fp16,
// to the pair's own partial row
// (page "MoVA: routing the value vectors ...", section "Where the routing
// happens": SiLU on each expert's output, weighted by the routing weight).
// Each partial row is written by exactly one tile, so no atomics are needed;
// the k-way sum happens afterwards in a fixed slot order.
//
// Block tile BM x BN = 256 x 256, k steps of 64, 8 waves in a 2 x 4 grid, each
// wave owning a 128 x 64 sub-tile (8 x 4 MFMA 16x16x32 tiles).  Operand tiles
// go global -> LDS with direct (global_load_lds) 16-byte loads, double
// buffered: the loads of step k+1 are in flight while step k's MFMAs run, with
// one barrier per step.  A staged row holds 64 bf16 (128 B) whose 16-byte
// chunks sit at chunk ^ (row & 7), so the MFMA fragment reads hit distinct
// banks; since a direct load writes 64 consecutive 16-byte slots, the swizzle
// is applied when choosing which global chunk each lane loads.
//
// A tile with at most 128 valid rows runs its lower waves through a copy of
// the k loop that only loads and synchronises (no MFMA work on empty rows).
//
// Work order: tile id -> (expert, n-tile, m-tile), m fastest, so tiles that
// share an expert's weight slab are adjacent.  Workgroups are dealt round
// robin over the 8 XCDs; block b runs tile (b % 8) * per_xcd + b / 8, giving
// each XCD one contiguous run of tiles (and its L2 the weights they share).
#include "common.h"
#include "kernels.h"

namespace mova {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int kThreads = 512;
constexpr int kRowBytes = BK * 2;             // 128 B per staged row
constexpr int kTileA = BM * kRowBytes;        // 32 KB
constexpr int kTileB = BN * kRowBytes;        // 32 KB
constexpr int kStage = kTileA + kTileB;       // 64 KB per buffer
constexpr int kXcds = 8;
constexpr int kLoadsPerWave = BM * kRowBytes / 1024 / (kThreads / 64);  // 4 (A) and 4 (B)

int gemm_block_m() { return BM; }

int gemm_max_mtiles(int T, int k, int E) { return (int)(((long long)T * k) / BM) + E; }

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ (row & 7)) << 4);
}

struct TileCtx {
  const char* a_src[kLoadsPerWave];  // per lane: gathered x row + its chunk
  const char* b_src[kLoadsPerWave];  // per lane: weight row + its chunk
  int lds_block[kLoadsPerWave];      // wave-uniform LDS block (1 KB units)
};

__device__ __forceinline__ void issue_loads(const TileCtx& c, char* stage, int k_byte) {
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    __builtin_amdgcn_global_load_lds((const void*)(c.a_src[i] + k_byte),
                                     (lds_void*)(stage + c.lds_block[i] * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(c.b_src[i] + k_byte),
                                     (lds_void*)(stage + kTileA + c.lds_block[i] * 1024), 16, 0, 0);
  }
}

// One k step (two 32-wide MFMA steps) of the wave's 128 x 64 sub-tile.
__device__ __forceinline__ void mma_step(f32x4 (&acc)[8][4], const char* stage, int wm, int wn,
                                         int q, int r16) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int chunk = ks * 4 + q;
    Frag16 fa[8], fb[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) fa[i].u = load16(stage + swz(wm * 128 + i * 16 + r16, chunk));
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j].u = load16(stage + kTileA + swz(wn * 64 + j * 16 + r16, chunk));
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(fa[i].h, fb[j].h, acc[i][j]);
  }
}

__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ W,
    const int32_t* __restrict__ perm, const float* __restrict__ topk_w,
    const int32_t* __restrict__ expert_off, const int32_t* __restrict__ tile_base,
    f16_t* __restrict__ partial, int d, int N, int E, int k) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];  // 2 stages
  __shared__ int tile_pair[BM];
  __shared__ float tile_w[BM];

  const int NT = ceil_div(N, BN);
  const int total = tile_base[E] * NT;
  const int per_xcd = ceil_div(total, kXcds);
  const int local = blockIdx.x / kXcds;
  if (local >= per_xcd) return;
  const int wid = (blockIdx.x % kXcds) * per_xcd + local;
  if (wid >= total) return;

  // Expert owning this tile: the last e with tile_base[e] * NT <= wid.
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tile_base[mid] * NT <= wid) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int me = tile_base[e + 1] - tile_base[e];
  const int rel = wid - tile_base[e] * NT;
  const int nt = rel / me;
  const int mt = rel % me;
  const int row0 = expert_off[e] + mt * BM;
  const int rows = min(BM, expert_off[e + 1] - row0);
  const int n0 = nt * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int q = lane >> 4, r16 = lane & 15;

  for (int r = tid; r < BM; r += kThreads) {
    const int pair = perm[row0 + min(r, rows - 1)];
    tile_pair[r] = pair;
    tile_w[r] = topk_w[pair];
  }

  // Lane -> (row, chunk) of each direct load: LDS block j holds rows 8j .. 8j+7,
  // lane l lands in slot l, i.e. row 8j + l/8, physical chunk l%8, which holds
  // logical chunk (l%8) ^ (row & 7).
  TileCtx c;
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    const int j = wave * kLoadsPerWave + i;
    const int row = j * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ (row & 7);
    const int pair = perm[row0 + min(row, rows - 1)];
    c.a_src[i] = reinterpret_cast<const char*>(x + (size_t)(pair / k) * d) + chunk * 16;
    const int n = min(n0 + row, N - 1);
    c.b_src[i] = reinterpret_cast<const char*>(W + ((size_t)e * N + n) * d) + chunk * 16;
    c.lds_block[i] = j;
  }

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KT = d / BK;
  issue_loads(c, smem, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const bool active = wm * 128 < rows;  // wave-uniform
  if (active) {
    for (int kt = 0; kt < KT; ++kt) {
      char* cur = smem + (kt & 1) * kStage;
      if (kt + 1 < KT) issue_loads(c, smem + ((kt + 1) & 1) * kStage, (kt + 1) * kRowBytes);
      mma_step(acc, cur, wm, wn, q, r16);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  } else {
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + 1 < KT) issue_loads(c, smem + ((kt + 1) & 1) * kStage, (kt + 1) * kRowBytes);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    return;
  }

  // Epilogue: y = w * SiLU(z) into the pair's partial row.
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = wm * 128 + i * 16 + q * 4 + v;
      if (r < rows) {
        const int pair = tile_pair[r];
        const float wt = tile_w[r];
        f16_t* dst = partial + (size_t)pair * N + n0 + wn * 64 + r16;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (n0 + wn * 64 + j * 16 + r16 < N) dst[j * 16] = (f16_t)(wt * siluf(acc[i][j][v]));
        }
      }
    }
  }
}

hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute((const void*)grouped_gemm_kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kStage);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  const long long ub = (long long)gemm_max_mtiles(a.T, a.k, a.E) * ceil_div(a.N, BN);
  const long long grid = ((ub + kXcds - 1) / kXcds) * kXcds;
  grouped_gemm_kernel<<<dim3((unsigned)grid), kThreads, 2 * kStage, stream>>>(
      a.x, a.W, a.perm, a.topk_w, a.expert_off, a.tile_base, a.partial, a.d, a.N, a.E, a.k);
  return hipGetLastError();
}

}  // namespace mova
