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
// Block tile BM x BN (352 x 256, 256 x 256, 128 x 256 or 128 x 128), k steps
// of 64, 8 waves in a 2 x 4 grid (or 4 waves in 2 x 2 for 128 x 128), each
// wave owning a BM/2 x BN/4 (or BM/2 x BN/2) sub-tile of 16x16x32 MFMA tiles.  Operand
// tiles go global -> LDS with direct (global_load_lds) 16-byte loads into a
// ring of LDS stages: with 2 stages the loads of step k+1 are in flight while
// step k's MFMAs run, one barrier per step; with 3 or 4 stages (128 x 128
// only) the loads run 2 or 3 steps ahead, which pays when one workgroup per
// CU has to keep the CU's loads in flight by itself.  A staged row holds 64
// bf16 (128 B) whose 16-byte chunks sit at chunk ^ (row & 7), so the MFMA
// fragment reads hit distinct banks; since a direct load writes 64
// consecutive 16-byte slots, the swizzle is applied when choosing which
// global chunk each lane loads.
//
// Tile choice (measured): grouped mode takes 128 x 128 (2 stages, two
// workgroups per CU), 256 x 256 or 352 x 256 by the experts' average row count
// (gemm_tile_grouped); dense mode takes 256 x
// 256 once those tiles fill the 256 CUs, else 128 x 128 with 4 stages when
// the grid is a single round of workgroups and 2 stages otherwise.
//
// A tile whose valid rows end in the upper half keeps its lower waves in the
// k loop for the loads and barriers only (no MFMA work on empty rows); with 2
// stages, a wave whose valid rows fit in half of its row blocks computes only
// that half.
//
// Work order: tile id -> (expert, m-tile, n-tile) in routed modes and
// (m-tile, n-tile) in dense modes, n fastest, so the column tiles that share
// a row tile's token rows are adjacent and run at the same time on one XCD,
// which then fetches those rows once (measured: dense T = 8192 12 % faster
// than m fastest; skewed routed T = 32768 at the same speed with 1.65 instead
// of 2.80 GB leaving L2).  An expert's tiles stay contiguous, so the XCDs
// that share its weight slab are few.  Workgroups are dealt round robin over
// the 8 XCDs; block b runs tile (b % 8) * per_xcd + b / 8, giving each XCD
// one contiguous run of tiles.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace mova {

constexpr int BK = 64;
constexpr int kRowBytes = BK * 2;  // 128 B per staged row
constexpr int kXcds = 8;

// kBM x kBN block tile over a kWM x kWN grid of waves, kS LDS stages.
template <int kBM, int kBN, int kWM, int kWN, int kS>
struct Tile {
  static constexpr int kWaves = kWM * kWN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kTileA = kBM * kRowBytes;
  static constexpr int kTileB = kBN * kRowBytes;
  static constexpr int kStage = kTileA + kTileB;  // per buffer
  // A 1 KB direct load fills one 8-row block.  The A blocks are split over
  // the waves as evenly as whole blocks allow (352 rows: 44 blocks, six per
  // wave, the last wave taking the two left over).
  static constexpr int kBlocksA = kBM / 8;
  static constexpr int kLoadsA = (kBlocksA + kWaves - 1) / kWaves;  // per wave, at most
  static constexpr bool kEvenA = kBlocksA % kWaves == 0;
  static constexpr int kLoadsB = kBN * kRowBytes / 1024 / kWaves;
  static constexpr int kRowsW = kBM / kWM;  // rows per wave
  static constexpr int kColsW = kBN / kWN;  // columns per wave
  static constexpr int kMI = kRowsW / 16;   // MFMA row tiles per wave
  static constexpr int kNJ = kColsW / 16;   // MFMA column tiles per wave
};
#define MOVA_TILE_PARAMS int kBM, int kBN, int kWM, int kWN, int kS
#define MOVA_TILE_ARGS kBM, kBN, kWM, kWN, kS

// Tile shapes the kOvGemmTile override can force (tests, measurements), by
// its value 1 .. 7; 352 x 256 exists in the routed modes only (a dense call
// ignores it).
static bool forced_tile(GemmTile* t, bool routed) {
  static const GemmTile kTiles[] = {{256, 256, 8, 2}, {128, 256, 8, 2}, {128, 128, 8, 2},
                                    {128, 128, 8, 3}, {128, 128, 8, 4}, {128, 128, 4, 4},
                                    {352, 256, 8, 2}};
  const int v = override_value(kOvGemmTile);
  if (v < 1 || v > 7) return false;
  const GemmTile c = kTiles[v - 1];
  if (!routed && c.bm == 352) return false;
  *t = c;
  return true;
}

GemmTile gemm_tile_grouped(int T, int k, int E, int N) {
  GemmTile t;
  if (forced_tile(&t, true)) return t;
  // By the experts' average row count R = T k / E.  Which tile wins depends
  // on how the busiest expert's rows (about 1.2-1.3 R under near-uniform
  // routing) round up to whole M-tiles, and the tiles up to whole rounds of
  // workgroups (two 128 x 128, or one 256 x 256 or 352 x 256, per CU); a
  // tile tall enough to keep every expert within n M-tiles finishes in n
  // rounds when the experts' 256-column tiles fill the CUs.  Measured on the
  // value layer (d = 2560, N = 1024, E = 64, seeded uniform routing), call
  // times in us:
  //   R        48   96   128  192  208  224  256  272  288  320  384  448  512  576  640
  //   128x128  100  115  150  154  -    188  196  208  207  235  247  281  300  -    -
  //   256x256  114  119  124  137  202  201  197  -    209  212  218  285  289  299  350
  //   352x256  -    -    -    152  172  150  159  172  239  243  251  256  262  355  358
  // and for larger R (one session, uniform routing, then the Zipf-skewed
  // T = 32768 workload):
  //   R        768  1024  1536  2048  skewed
  //   256x256  375  455   642   848   831
  //   352x256  366  460   605   814   819
  // 352 x 256 for R in (200, 272], (408, 560] and above 704 when
  // E * N / 256 >= 256; otherwise 128 x 128 up to R = 112 and from 209 to
  // 304, 256 x 256 elsewhere.
  const long long R = ((long long)T * k + E / 2) / E;
  const bool fills = (long long)E * ceil_div(N, 256) >= 256;
  if (fills && ((R > 200 && R <= 272) || (R > 408 && R <= 560) || R > 704)) return {352, 256, 8, 2};
  if (R <= 112 || (R > 208 && R <= 304)) return {128, 128, 8, 2};
  return {256, 256, 8, 2};
}

GemmTile gemm_tile_grouped_ffn(int T, int k, int E) {
  GemmTile t;
  if (forced_tile(&t, true)) return t;
  // The FFN's experts (E = 100, k = 8, 1536 / 2560 columns), the same kind
  // of alternation as above; call times in us:
  //   R        20   82   123  164  246  328  492   655
  //   128x128  312  369  438  507  602  713  981   1225
  //   256x256  372  419  451  478  605  724  888   1130
  // and measured again beside the 352 x 256 tile:
  //   R        164  246  328  492
  //   128x128  521  624  744  1009
  //   256x256  495  620  740  920
  //   352x256  505  569  665  963
  // 128 x 128 up to R = 144, 352 x 256 from 209 to 352, 128 x 128 from 353
  // to 384, 256 x 256 elsewhere.
  const long long R = ((long long)T * k + E / 2) / E;
  if (R > 208 && R <= 352) return {352, 256, 8, 2};
  if (R <= 144 || (R > 352 && R <= 384)) return {128, 128, 8, 2};
  return {256, 256, 8, 2};
}

int gemm_max_mtiles(int T, int k, int E, int bm) { return (int)(((long long)T * k) / bm) + E; }

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ (row & 7)) << 4);
}

template <MOVA_TILE_PARAMS>
struct TileCtx {
  const char* a_src[Tile<MOVA_TILE_ARGS>::kLoadsA];  // per lane: (gathered) x row + its chunk
  const char* b_src[Tile<MOVA_TILE_ARGS>::kLoadsB];  // per lane: weight row + its chunk
};

// Direct loads of one k step: A block j (rows 8j .. 8j+7) for j = wave * kLoadsA + i,
// B block j for j = wave * kLoadsB + i; kAuxB is the B loads' cache policy.
template <MOVA_TILE_PARAMS, int kAuxB = 0>
__device__ __forceinline__ void issue_loads(const TileCtx<MOVA_TILE_ARGS>& c, char* stage, int wave,
                                            int k_byte) {
  using TL = Tile<MOVA_TILE_ARGS>;
#pragma unroll
  for (int i = 0; i < TL::kLoadsA; ++i)
    if (TL::kEvenA || wave * TL::kLoadsA + i < TL::kBlocksA)  // wave-uniform
      __builtin_amdgcn_global_load_lds((const void*)(c.a_src[i] + k_byte),
                                       (lds_void*)(stage + (wave * TL::kLoadsA + i) * 1024), 16, 0,
                                       0);
#pragma unroll
  for (int i = 0; i < TL::kLoadsB; ++i)
    __builtin_amdgcn_global_load_lds((const void*)(c.b_src[i] + k_byte),
                                     (lds_void*)(stage + TL::kTileA + (wave * TL::kLoadsB + i) * 1024),
                                     16, 0, kAuxB);
}

// One k step (two 32-wide MFMA steps) of the wave's sub-tile, for its first
// kUsed 16-row blocks (the rest hold no valid rows; their accumulators are
// never stored).
template <MOVA_TILE_PARAMS, int kUsed>
__device__ __forceinline__ void mma_step(f32x4 (&acc)[kBM / kWM / 16][kBN / kWN / 16],
                                         const char* stage, int wm, int wn, int q, int r16) {
  using TL = Tile<MOVA_TILE_ARGS>;
  constexpr int NJ = TL::kNJ;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int chunk = ks * 4 + q;
    Frag16 fa[kUsed], fb[NJ];
#pragma unroll
    for (int i = 0; i < kUsed; ++i) fa[i].u = load16(stage + swz(wm * TL::kRowsW + i * 16 + r16, chunk));
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      fb[j].u = load16(stage + TL::kTileA + swz(wn * TL::kColsW + j * 16 + r16, chunk));
#pragma unroll
    for (int i = 0; i < kUsed; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = mfma16x16x32(fa[i].h, fb[j].h, acc[i][j]);
  }
}

// The same k step with the next step's direct loads issued among the first
// sub-step's MFMAs, and the second sub-step's fragment reads among its last
// ones (tiles of up to 256 rows, equal loads per wave).  Issued together at
// the top of the step, the eight waves' loads reach the address unit as one
// burst, and the waves queued behind it issue no MFMAs meanwhile; spread out,
// they drain while the MFMAs run (measured: the dense T = 32768 GEMM 144-145
// -> 138-141 us).  The load pointers advance in place by k_inc (0 in the last
// step, which reloads its own k step into the unused stage and keeps the step
// free of branches), so no address temporaries are held across the MFMAs.
// The 352-row tile keeps mma_step: it has no registers to spare for this
// schedule (it spills), and without the schedule it measured mixed.
template <MOVA_TILE_PARAMS, int kUsed, int kAuxB = 0>
__device__ __forceinline__ void mma_step_spread(f32x4 (&acc)[kBM / kWM / 16][kBN / kWN / 16],
                                                const char* stage, int wm, int wn, int q, int r16,
                                                TileCtx<MOVA_TILE_ARGS>& c, char* next, int wave,
                                                int k_inc) {
  using TL = Tile<MOVA_TILE_ARGS>;
  static_assert(TL::kEvenA, "every wave issues the same loads");
  constexpr int NJ = TL::kNJ;
  constexpr int L = TL::kLoadsA + TL::kLoadsB;  // direct loads per wave and step
  constexpr int M0 = kUsed * NJ;                // MFMAs per sub-step
  constexpr int kPer = (M0 / 2) / L > 0 ? (M0 / 2) / L : 1;  // MFMAs before each load
  constexpr int kRest = M0 - kPer * L;
  constexpr int kR = kUsed + NJ;  // fragment reads per sub-step
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int chunk = ks * 4 + q;
    Frag16 fa[kUsed], fb[NJ];
#pragma unroll
    for (int i = 0; i < kUsed; ++i) fa[i].u = load16(stage + swz(wm * TL::kRowsW + i * 16 + r16, chunk));
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      fb[j].u = load16(stage + TL::kTileA + swz(wn * TL::kColsW + j * 16 + r16, chunk));
#pragma unroll
    for (int i = 0; i < kUsed; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = mfma16x16x32(fa[i].h, fb[j].h, acc[i][j]);
    if (ks == 0) {
#pragma unroll
      for (int i = 0; i < TL::kLoadsA; ++i) {
        c.a_src[i] += k_inc;
        __builtin_amdgcn_global_load_lds((const void*)c.a_src[i],
                                         (lds_void*)(next + (wave * TL::kLoadsA + i) * 1024), 16, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < TL::kLoadsB; ++i) {
        c.b_src[i] += k_inc;
        __builtin_amdgcn_global_load_lds((const void*)c.b_src[i],
                                         (lds_void*)(next + TL::kTileA + (wave * TL::kLoadsB + i) * 1024),
                                         16, 0, kAuxB);
      }
    }
  }
  // Order (sched_group_barrier masks: 0x100 LDS reads, 0x008 MFMA, 0x020
  // vector-memory reads): sub-step 0's reads; its first MFMAs with one load
  // after every kPer of them; its remaining MFMAs with sub-step 1's reads in
  // two halves among them; sub-step 1's MFMAs.  The closing sched_barrier
  // keeps the caller's wait and barrier after every MFMA of the step.
  __builtin_amdgcn_sched_group_barrier(0x100, kR, 0);
#pragma unroll
  for (int n = 0; n < L; ++n) {
    __builtin_amdgcn_sched_group_barrier(0x008, kPer, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, kRest / 2, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, kR / 2, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, kRest - kRest / 2, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, kR - kR / 2, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, M0, 0);
  __builtin_amdgcn_sched_barrier(0);
}

constexpr bool mode_routed(int m) {
  return m == kGemmRoutedSilu || m == kGemmRoutedSwiGLU || m == kGemmRoutedLinear;
}
constexpr bool mode_swiglu(int m) { return m == kGemmRoutedSwiGLU || m == kGemmDenseSwiGLU; }

// Routed modes: tiles over the experts' pair rows (perm, expert_off,
// tile_base), B = W[e].  Dense modes: tiles over T rows in order, B = W (one
// [N, d] weight).  A rows: token perm[r] / k of x (routed SiLU / SwiGLU),
// row perm[r] of x (routed linear: x holds one row per pair), or row r
// (dense).  Epilogues (kGemm* in kernels.h):
//   RoutedSilu    partial[pair, n] = fp16(w * SiLU(z))
//   Dense         out[r, n]        = bf16(z)
//   RoutedSwiGLU  out[pair, c]     = bf16(SiLU(z_gate) * z_up)
//   RoutedLinear  partial[pair, n] = fp16(w * z)
//   DenseSwiGLU   out[r, c]        = bf16(SiLU(z_gate) * z_up)
//   DenseF16      partial[r, n]    = fp16(z)
// SwiGLU weights interleave gate and up rows in blocks of 16: rows 32b .. 32b+15
// are gate rows 16b .. 16b+15 and rows 32b+16 .. 32b+31 the matching up rows,
// so the wave's column tiles 2j and 2j+1 hold the gate and up values of the
// same 16 outputs c = (column of tile 2j) / 2 .. + 15; out has N / 2 columns.
//
// kNtB: the weight (B) loads carry the non-temporal hint, for calls where
// each expert's weight tile is read by a single row tile (launch_routed_mode).
template <MOVA_TILE_PARAMS, int kMode, bool kNtB = false>
__global__ __launch_bounds__(64 * kWM * kWN) void gemm_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ W,
    const int32_t* __restrict__ perm, const float* __restrict__ topk_w,
    const int32_t* __restrict__ expert_off, const int32_t* __restrict__ tile_base,
    f16_t* __restrict__ partial, bf16_t* __restrict__ out, int T, int d, int N, int E, int k) {
  using TL = Tile<MOVA_TILE_ARGS>;
  constexpr bool kDense = !mode_routed(kMode);
  constexpr int WN = TL::kColsW;  // columns per wave
  static_assert(!mode_swiglu(kMode) || WN % 32 == 0, "SwiGLU pairs 16-column tiles");
  static_assert(TL::kEvenA || kS == 2, "the ring's wait counts assume equal loads per wave");
  static_assert(!kNtB || kS == 2, "the hint is wired into the 2-stage loops only");
  constexpr int kAuxB = kNtB ? kLdsLoadNonTemporal : 0;
  extern __shared__ __attribute__((aligned(1024))) char smem[];  // kS stages
  __shared__ int tile_pair[kDense ? 1 : kBM];
  __shared__ float tile_w[kDense ? 1 : kBM];

  const int NT = ceil_div(N, kBN);
  const int MTd = kDense ? ceil_div(T, kBM) : 0;
  const int total = kDense ? MTd * NT : tile_base[E] * NT;
  const int per_xcd = ceil_div(total, kXcds);
  const int local = blockIdx.x / kXcds;
  if (local >= per_xcd) return;
  const int wid = (blockIdx.x % kXcds) * per_xcd + local;
  if (wid >= total) return;

  int e = 0, nt, row0, rows;
  if constexpr (kDense) {
    // Column tiles fastest: an XCD's run of tiles covers a few row tiles
    // across all columns, so each token row is fetched into one XCD's L2
    // only; the weight, much smaller, is what the XCDs share.
    nt = wid % NT;
    row0 = (wid / NT) * kBM;
    rows = min(kBM, T - row0);
  } else {
    // Expert owning this tile: the last e with tile_base[e] * NT <= wid.
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tile_base[mid] * NT <= wid) lo = mid; else hi = mid;
    }
    e = lo;
    const int rel = wid - tile_base[e] * NT;
    nt = rel % NT;
    row0 = expert_off[e] + (rel / NT) * kBM;
    rows = min(kBM, expert_off[e + 1] - row0);
  }
  const int n0 = nt * kBN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWN, wn = wave % kWN;
  const int q = lane >> 4, r16 = lane & 15;

  if constexpr (!kDense) {
    for (int r = tid; r < kBM; r += TL::kThreads) {
      const int pair = perm[row0 + min(r, rows - 1)];
      tile_pair[r] = pair;
      tile_w[r] = kMode == kGemmRoutedSwiGLU ? 0.f : topk_w[pair];
    }
  }

  // Lane -> (row, chunk) of each direct load: LDS block j holds rows 8j .. 8j+7,
  // lane l lands in slot l, i.e. row 8j + l/8, physical chunk l%8, which holds
  // logical chunk (l%8) ^ (row & 7).  Rows past the tile's valid rows (or past
  // N) load a clamped row and are never stored.
  TileCtx<MOVA_TILE_ARGS> c;
#pragma unroll
  for (int i = 0; i < TL::kLoadsA; ++i) {
    const int row = (wave * TL::kLoadsA + i) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ (row & 7);
    const int rr = row0 + min(row, rows - 1);
    int arow = rr;
    if constexpr (kMode == kGemmRoutedLinear) arow = perm[rr];
    else if constexpr (!kDense) arow = perm[rr] / k;
    c.a_src[i] = reinterpret_cast<const char*>(x + (size_t)arow * d) + chunk * 16;
  }
#pragma unroll
  for (int i = 0; i < TL::kLoadsB; ++i) {
    const int row = (wave * TL::kLoadsB + i) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ (row & 7);
    const int n = min(n0 + row, N - 1);
    c.b_src[i] = reinterpret_cast<const char*>(W + ((size_t)e * N + n) * d) + chunk * 16;
  }

  f32x4 acc[TL::kMI][TL::kNJ];
#pragma unroll
  for (int i = 0; i < TL::kMI; ++i)
#pragma unroll
    for (int j = 0; j < TL::kNJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KT = d / BK;
  // Valid 16-row blocks of this wave's rows (wave-uniform).
  const int nv = min(TL::kMI, max(0, ceil_div(rows - wm * TL::kRowsW, 16)));
  const bool active = nv > 0;
  if constexpr (kS == 2) {
    issue_loads<MOVA_TILE_ARGS, kAuxB>(c, smem, wave, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // A wave whose valid rows fit in the first half of its row blocks runs
    // a copy of the loop that computes only those (a separate loop, not a
    // branch per block, keeps the register allocation of the full one).
    auto steps = [&](auto used) {
      for (int kt = 0; kt < KT; ++kt) {
        char* cur = smem + (kt & 1) * TL::kStage;
        char* nxt = smem + ((kt + 1) & 1) * TL::kStage;
        if constexpr (kBM <= 256) {
          mma_step_spread<MOVA_TILE_ARGS, decltype(used)::value, kAuxB>(acc, cur, wm, wn, q, r16, c, nxt, wave,
                                                                 kt + 1 < KT ? kRowBytes : 0);
        } else {
          if (kt + 1 < KT) issue_loads<MOVA_TILE_ARGS, kAuxB>(c, nxt, wave, (kt + 1) * kRowBytes);
          mma_step<MOVA_TILE_ARGS, decltype(used)::value>(acc, cur, wm, wn, q, r16);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
    };
    constexpr int kHalf = (TL::kMI + 1) / 2;
    if (nv > kHalf) {
      steps(std::integral_constant<int, TL::kMI>{});
    } else if (active) {
      steps(std::integral_constant<int, kHalf>{});
    } else {
      for (int kt = 0; kt < KT; ++kt) {
        if (kt + 1 < KT)
          issue_loads<MOVA_TILE_ARGS, kAuxB>(c, smem + ((kt + 1) & 1) * TL::kStage, wave,
                                      (kt + 1) * kRowBytes);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
      return;
    }
  } else {
    // Ring of kS stages, loads kS - 1 steps ahead.  Step kt: wait for this
    // wave's loads of step kt (the kS - 2 later steps may stay in flight) and
    // for its LDS reads, barrier (every wave's loads of step kt have landed,
    // and every wave is done reading step kt - 1's stage), run step kt's
    // MFMAs, then refill step kt - 1's stage with step kt + kS - 1.  (Issued
    // after the fragment reads, the refill keeps the compiler from waiting on
    // every outstanding direct load before those reads.)  Steps past KT load
    // step KT - 1 again (never read), so every step issues the same number of
    // loads and the wait count stays exact.  Waves without valid rows run the
    // same loop without the MFMAs.
    constexpr int L = TL::kLoadsA + TL::kLoadsB;
    __syncthreads();  // the tile's pair / weight table is written
#pragma unroll
    for (int st = 0; st < kS - 1; ++st)
      issue_loads<MOVA_TILE_ARGS>(c, smem + st * TL::kStage, wave, min(st, KT - 1) * kRowBytes);
    auto ring = [&](auto compute) {
      for (int kt = 0; kt < KT; ++kt) {
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm((kS - 2) * L));
        raw_barrier();
        const int nk = kt + kS - 1;
        if constexpr (decltype(compute)::value)
          mma_step<MOVA_TILE_ARGS, TL::kMI>(acc, smem + (kt % kS) * TL::kStage, wm, wn, q, r16);
        issue_loads<MOVA_TILE_ARGS>(c, smem + (nk % kS) * TL::kStage, wave,
                                    min(nk, KT - 1) * kRowBytes);
      }
      __builtin_amdgcn_s_waitcnt(0);
    };
    if (!active) {
      ring(std::false_type{});
      return;
    }
    ring(std::true_type{});
  }

  // Epilogue (see the mode table above).
  const int cb = n0 + wn * WN;  // first column of the wave's sub-tile
#pragma unroll
  for (int i = 0; i < TL::kMI; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = wm * TL::kRowsW + i * 16 + q * 4 + v;
      if (r < rows) {
        const size_t orow = kDense ? (size_t)(row0 + r) : (size_t)tile_pair[r];
        if constexpr (mode_swiglu(kMode)) {
          bf16_t* dst = out + orow * (N / 2) + cb / 2 + r16;
#pragma unroll
          for (int j = 0; j < TL::kNJ; j += 2)
            if (cb + j * 16 + r16 < N)
              dst[j * 8] = (bf16_t)(siluf(acc[i][j][v]) * acc[i][j + 1][v]);
        } else if constexpr (kMode == kGemmDense) {
          bf16_t* dst = out + orow * N + cb + r16;
#pragma unroll
          for (int j = 0; j < TL::kNJ; ++j)
            if (cb + j * 16 + r16 < N) dst[j * 16] = (bf16_t)acc[i][j][v];
        } else {
          f16_t* dst = partial + orow * N + cb + r16;
          const float wt = kDense ? 1.f : tile_w[r];
#pragma unroll
          for (int j = 0; j < TL::kNJ; ++j) {
            if (cb + j * 16 + r16 < N) {
              const float z = acc[i][j][v];
              if constexpr (kMode == kGemmRoutedSilu) dst[j * 16] = (f16_t)(wt * siluf(z));
              else if constexpr (kMode == kGemmRoutedLinear) dst[j * 16] = (f16_t)(wt * z);
              else dst[j * 16] = (f16_t)z;
            }
          }
        }
      }
    }
  }
}

template <MOVA_TILE_PARAMS, int kMode, bool kNtB = false>
hipError_t launch_tiles(const GemmArgs& a, long long tiles, hipStream_t stream) {
  auto kern = gemm_kernel<MOVA_TILE_ARGS, kMode, kNtB>;
  constexpr int smem = kS * Tile<MOVA_TILE_ARGS>::kStage;
  constexpr int threads = Tile<MOVA_TILE_ARGS>::kThreads;
  static std::atomic<unsigned long long> attr_done{0};
  hipError_t err = once_per_device(attr_done, [&]() {
    return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  });
  if (err != hipSuccess) return err;
  const long long grid = ((tiles + kXcds - 1) / kXcds) * kXcds;
  kern<<<dim3((unsigned)grid), threads, smem, stream>>>(a.x, a.W, a.perm, a.topk_w, a.expert_off,
                                                         a.tile_base, a.partial, a.out, a.T, a.d,
                                                         a.N, a.E, a.k);
  return hipGetLastError();
}

template <int kMode>
static hipError_t launch_routed_mode(const GemmArgs& a, long long ub, hipStream_t stream) {
  const GemmTile t = a.tile;
  if (t.bm == 352 && t.bn == 256) {
    // Value experts whose rows fit one 352-row tile (the busiest expert
    // holds about 1.3 R rows, R = T k / E) read each weight tile once:
    // the weight loads then take the non-temporal hint (measured below).
    if constexpr (kMode == kGemmRoutedSilu) {
      const long long R = ((long long)a.T * a.k + a.E / 2) / a.E;
      if (R * 13 <= 352 * 10) return launch_tiles<352, 256, 2, 4, 2, kMode, true>(a, ub, stream);
    }
    return launch_tiles<352, 256, 2, 4, 2, kMode>(a, ub, stream);
  }
  // The same for the 256- and 128-row tiles (2 stages).  Measured on the
  // value layer (d = 2560, N = 1024, E = 64, graph replay), call times in us
  // without / with the hint: T = 512 91 / 84, 1024 97 / 91, 1536 104 / 96,
  // 2048 118 / 110, 3072 129 / 122, and with the 352-row tile T = 4096
  // 146-147 / 141.  With several row tiles per expert (chunked R = 512,
  // skewed R = 2048) it was about 1 % slower, and on the dense T = 32768
  // GEMM, whose weight serves 128 row tiles, 14 % slower.
  if constexpr (kMode == kGemmRoutedSilu) {
    const long long R = ((long long)a.T * a.k + a.E / 2) / a.E;
    if (R * 13 <= (long long)t.bm * 10) {
      if (t.bm == 256 && t.bn == 256) return launch_tiles<256, 256, 2, 4, 2, kMode, true>(a, ub, stream);
      if (t.bm == 128 && t.bn == 128 && t.waves == 8 && t.stages == 2)
        return launch_tiles<128, 128, 2, 4, 2, kMode, true>(a, ub, stream);
    }
  }
  if (t.bm == 256 && t.bn == 256) return launch_tiles<256, 256, 2, 4, 2, kMode>(a, ub, stream);
  if (t.bm == 128 && t.bn == 256) return launch_tiles<128, 256, 2, 4, 2, kMode>(a, ub, stream);
  if (t.bm == 128 && t.bn == 128 && t.waves == 8) {
    if (t.stages == 3) return launch_tiles<128, 128, 2, 4, 3, kMode>(a, ub, stream);
    if (t.stages == 4) return launch_tiles<128, 128, 2, 4, 4, kMode>(a, ub, stream);
    return launch_tiles<128, 128, 2, 4, 2, kMode>(a, ub, stream);
  }
  if (t.bm == 128 && t.bn == 128) return launch_tiles<128, 128, 2, 2, 4, kMode>(a, ub, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t stream) {
  const GemmTile t = a.tile;
  const long long ub = (long long)gemm_max_mtiles(a.T, a.k, a.E, t.bm) * ceil_div(a.N, t.bn);
  switch (a.mode) {
    case kGemmRoutedSilu: return launch_routed_mode<kGemmRoutedSilu>(a, ub, stream);
    case kGemmRoutedSwiGLU: return launch_routed_mode<kGemmRoutedSwiGLU>(a, ub, stream);
    case kGemmRoutedLinear: return launch_routed_mode<kGemmRoutedLinear>(a, ub, stream);
    default: return hipErrorInvalidValue;
  }
}

GemmTile gemm_tile_dense(int T, int N) {
  GemmTile t;
  if (forced_tile(&t, false)) return t;
  // 256 x 256 once those tiles fill the 256 CUs; below that 128 x 128, with
  // a 4-stage ring when the grid is a single round of workgroups (one per
  // CU, so the ring is what keeps loads in flight), else 2 stages (two
  // workgroups per CU).
  if ((long long)ceil_div(T, 256) * ceil_div(N, 256) >= 256) return {256, 256, 8, 2};
  if ((long long)ceil_div(T, 128) * ceil_div(N, 128) <= 256) return {128, 128, 8, 4};
  return {128, 128, 8, 2};
}

template <int kMode>
static hipError_t launch_dense_mode(const GemmArgs& a, GemmTile t, long long tiles,
                                    hipStream_t stream) {
  if (t.bm == 256 && t.bn == 256) return launch_tiles<256, 256, 2, 4, 2, kMode>(a, tiles, stream);
  if (t.bm == 128 && t.bn == 256) return launch_tiles<128, 256, 2, 4, 2, kMode>(a, tiles, stream);
  if (t.waves == 8) {
    if (t.stages == 3) return launch_tiles<128, 128, 2, 4, 3, kMode>(a, tiles, stream);
    if (t.stages == 4) return launch_tiles<128, 128, 2, 4, 4, kMode>(a, tiles, stream);
    return launch_tiles<128, 128, 2, 4, 2, kMode>(a, tiles, stream);
  }
  return launch_tiles<128, 128, 2, 2, 4, kMode>(a, tiles, stream);
}

hipError_t launch_dense_gemm(const GemmArgs& a, hipStream_t stream) {
  const GemmTile t = gemm_tile_dense(a.T, a.N);
  const long long tiles = (long long)ceil_div(a.T, t.bm) * ceil_div(a.N, t.bn);
  switch (a.mode) {
    case kGemmDense: return launch_dense_mode<kGemmDense>(a, t, tiles, stream);
    case kGemmDenseSwiGLU: return launch_dense_mode<kGemmDenseSwiGLU>(a, t, tiles, stream);
    case kGemmDenseF16: return launch_dense_mode<kGemmDenseF16>(a, t, tiles, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mova
