// Grouped GEMM over the selected experts with a fused SiLU * weight epilogue.
//
// For every expert e, the pairs routed to it (rows perm[expert_off[e] ..
// expert_off[e+1])) form the A operand by gathering token rows of x; the
// expert's [N, d] weight (nn.Linear layout, k contiguous) is the B operand.
// z = x_t W_e^T is accumulated in fp32 on bf16 MFMA, then
// y = w[pair] * SiLU(z) is stored to the pair's own partial row
// (page "MoVA: routing the value vectors ...", section "Where the routing
// happens": SiLU on each expert's output, weighted by the routing weight).
// Each partial row is written by exactly one tile, so no atomics are needed;
// the k-way sum happens afterwards in a fixed slot order.
//
// Tiles: BM x BN = 128 x 128, k-steps of 64, 4 waves each owning 64 x 64.
// Both operand tiles are staged through LDS (double-buffered) with rows of
// 128 B whose 16-byte chunks are XOR-swizzled by (row & 7) so that the
// MFMA fragment reads hit distinct banks.
//
// Work order: tile id -> (expert, n-tile, m-tile), m fastest, so tiles that
// share an expert's weight slab are adjacent.  Workgroups are dealt round
// robin over the 8 XCDs; block b runs tile (b % 8) * per_xcd + b / 8, giving
// each XCD one contiguous run of tiles (and its L2 the weights they share).
#include "common.h"
#include "kernels.h"

namespace mova {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int kRowBytes = BK * 2;          // 128 B per staged row
constexpr int kTileBytes = BM * kRowBytes;  // 16 KB per operand tile
constexpr int kXcds = 8;

int gemm_block_m() { return BM; }

int gemm_max_mtiles(int T, int k, int E) { return (int)(((long long)T * k) / BM) + E; }

__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ (row & 7)) << 4); }

__global__ __launch_bounds__(256, 2) void grouped_gemm_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ W,
    const int32_t* __restrict__ perm, const float* __restrict__ topk_w,
    const int32_t* __restrict__ expert_off, const int32_t* __restrict__ tile_base,
    float* __restrict__ partial, int d, int N, int E, int k) {
  __shared__ __attribute__((aligned(16))) char smem[2][2][kTileBytes];

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
  const int wm = wave >> 1, wn = wave & 1;
  const int q = lane >> 4, r16 = lane & 15;

  // Global -> LDS copy assignment: 4 passes of 32 rows x 8 chunks of 16 B.
  const int cp_row = tid >> 3, cp_chunk = tid & 7;
  const bf16_t* a_src[4];
  const bf16_t* b_src[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = it * 32 + cp_row;
    const int pair = perm[row0 + min(r, rows - 1)];
    a_src[it] = x + (size_t)(pair / k) * d + cp_chunk * 8;
    const int n = min(n0 + r, N - 1);
    b_src[it] = W + ((size_t)e * N + n) * d + cp_chunk * 8;
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ra[4], rb[4];
  auto gload = [&](int k0) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      ra[it] = load16(a_src[it] + k0);
      rb[it] = load16(b_src[it] + k0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int r = it * 32 + cp_row;
      store16(&smem[buf][0][swz(r, cp_chunk)], ra[it]);
      store16(&smem[buf][1][swz(r, cp_chunk)], rb[it]);
    }
  };

  const int KT = d / BK;
  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int chunk = ks * 4 + q;
      Frag16 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra_row = wm * 64 + i * 16 + r16;
        fa[i].u = load16(&smem[buf][0][swz(ra_row, chunk)]);
        const int rb_row = wn * 64 + i * 16 + r16;
        fb[i].u = load16(&smem[buf][1][swz(rb_row, chunk)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(fa[i].h, fb[j].h, acc[i][j]);
    }
    if (kt + 1 < KT) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: y = w * SiLU(z) into the pair's partial row.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = wm * 64 + i * 16 + q * 4 + v;
      if (r < rows) {
        const int pair = perm[row0 + r];
        const float wt = topk_w[pair];
        float* dst = partial + (size_t)pair * N + n0 + wn * 64 + r16;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (n0 + wn * 64 + j * 16 + r16 < N) dst[j * 16] = wt * siluf(acc[i][j][v]);
        }
      }
    }
  }
}

hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t stream) {
  const long long ub = (long long)gemm_max_mtiles(a.T, a.k, a.E) * ceil_div(a.N, BN);
  const long long grid = ((ub + kXcds - 1) / kXcds) * kXcds;
  grouped_gemm_kernel<<<dim3((unsigned)grid), 256, 0, stream>>>(
      a.x, a.W, a.perm, a.topk_w, a.expert_off, a.tile_base, a.partial, a.d, a.N, a.E, a.k);
  return hipGetLastError();
}

}  // namespace mova
