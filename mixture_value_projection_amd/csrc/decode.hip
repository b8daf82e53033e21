// Decode path: a weight-streaming kernel for small token counts, for the
// value experts and, with other epilogues, the FFN experts' gate / up and down
// projections (same products, same order, same bits as the grouped GEMM).
//
// With few tokens per expert the layer is bound by reading the touched
// experts' weights (page "MoVA: routing the value vectors ...", section "So
// what does it cost?": decode is memory-bound and reads four experts per
// token).  Each workgroup owns one (expert, 128-column slice) and streams that
// slice's 128 x d weights exactly once from HBM; the tokens that chose the
// expert (at most a few dozen) ride along as the MFMA's other operand, read
// from cache.  No dispatch kernel is needed: the workgroup finds its tokens by
// scanning the [T, k] routing with wave ballots, which also keeps them in
// pair order.
//
// Each wave owns 32 of the slice's columns as two 16-column MFMA groups that
// share one token fragment; per 32-wide k step its 64 lanes read 2 x 16 rows x
// 64 B of weights and one 16-byte token fragment (token row = lane % 16, read
// straight from cache: the rows are a few hundred KB shared by the whole
// grid).  With 4-step batches and one row group, the weights are loaded as
// whole 256-byte row segments (16 lanes per row, which the vector cache
// serves with far fewer requests than 16 rows per 16 lanes) and turned into
// fragments through a small LDS scratch of the wave's own; these loads carry
// the non-temporal hint (the weights are read once per call; measured at
// T = 64: 60.4 -> 53.5 us, while on the fragment loads of the other layouts
// the hint was slower, T = 128 81 -> 92 us).  The k loop runs in batches of kUnroll steps over a ring of three
// register buffers, so three batches of loads are in flight while a batch's
// MFMAs run; the waves never wait for each other inside the loop.  The first
// two weight batches are issued before the routing scan, which they do not
// depend on; the scan reads every pair's expert id and weight in one round
// trip, and keeps the weights in LDS for the epilogue.  Tokens are handled 16
// at a time (one MFMA row group), or 32 at a time (two row groups) when the
// expert has more than 16; an expert with more than 32 tokens takes several
// passes over its weights.  For the value experts the epilogue writes
// w * SiLU(z) (fp16, rounded once) to the pair's partial row, like the grouped
// GEMM; the combine kernel then sums each token's k partials in slot order.
// The MFMA chain of every (token, column) runs over the k steps in order, as
// in the grouped GEMM, so both paths give identical bits.  (A fused
// last-arriver combine was measured and rejected: the agent-scope release
// each workgroup needs costs far more than the separate combine launch.)
//
// 64 experts x 1024 columns is 512 workgroups of 4 waves: at two workgroups
// per CU (up to 256 registers per lane) the whole grid is resident at once.
// The FFN's projections (100 experts, 1536 or 2560 columns) run in a few
// rounds of workgroups.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace mova {

// kGroups: 16-column MFMA groups per wave (2, or 1 for narrow outputs, see
// launch_decode_mode); a workgroup's 4 waves cover 64 * kGroups columns.

// kUnroll: k steps per batch; it divides the step count d / 32 (4 when it
// can, else 2, which always does since d % 64 == 0).  kPair32: experts with
// more than 16 pairs use 32-pair passes (worth it once the experts average
// more than 10 pairs; without it the kernel holds fewer registers and uses
// the row-segment loads, and such experts take 16-pair passes).
//
// kMode selects the epilogue, as in the grouped GEMM (GemmMode):
//   kGemmRoutedSilu    partial[pair, n] = fp16(w * SiLU(z))     (value experts)
//   kGemmRoutedSwiGLU  out_h[pair, c]   = bf16(SiLU(z_gate) * z_up)
//                      (FFN gate / up: rows interleaved in blocks of 16, so a
//                      wave's two column groups are one gate block and its
//                      up block, and c = its first column / 2 + lane % 16)
//   kGemmRoutedLinear  partial[pair, n] = fp16(w * z), A rows one per pair
//                      (FFN down, A = the pairs' h rows)
template <int kUnroll, bool kPair32, int kMode, int kGroups>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ W,
    const int32_t* __restrict__ idx, const float* __restrict__ topk_w,
    f16_t* __restrict__ partial, bf16_t* __restrict__ out_h, int T, int d, int N, int E, int k) {
  // An expert gets at most T * k pairs (k of them per token when a caller's
  // stored routing repeats an id; the router never does).
  __shared__ int plist[kDecodeMaxT * kMaxTopK];
  __shared__ float wlist[kDecodeMaxT * kMaxTopK];
  __shared__ int wave_hits[4];
  // Weight loads as whole row segments, turned into MFMA fragments through a
  // wave-private LDS scratch (4-step batches with one row group; measured:
  // 62.1 -> 60.4 us at T = 64, but 71 -> 75 us with the two-deep ring of
  // 32-pair passes, where the extra LDS round trip is not hidden).
  constexpr bool kRowLoads = kUnroll == 4 && !kPair32;
  __shared__ __attribute__((aligned(16))) char wscr[kRowLoads ? 4 : 1][kRowLoads ? kGroups * 16 * 256 : 16];

  static_assert(kGroups == 2 || (kGroups == 1 && kMode != kGemmRoutedSwiGLU),
                "SwiGLU pairs a gate group with its up group in one wave");
  constexpr int kSlice = 64 * kGroups;
  const int slices = ceil_div(N, kSlice);
  const int e = blockIdx.x / slices;
  const int n0 = (blockIdx.x % slices) * kSlice;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int npairs = T * k;

  // Column of each group; rows past N (N a multiple of 64 but not of 128)
  // load a clamped row and are never stored.
  int ncol[kGroups];
  const bf16_t* wrow[kGroups];
  const bf16_t* wseg[kGroups][4];
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    ncol[g] = n0 + wave * 16 * kGroups + g * 16 + r16;
    wrow[g] = W + ((size_t)e * N + min(ncol[g], N - 1)) * d + q * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wseg[g][i] = W +
                   ((size_t)e * N + min(n0 + wave * 16 * kGroups + g * 16 + 4 * i + (lane >> 4), N - 1)) * d +
                   (lane & 15) * 8;
  }
  const int nb = d / 32 / kUnroll;  // exact by the choice of kUnroll
  auto load_w = [&](Frag16 (&b)[kGroups][kUnroll], int bt) {
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      if constexpr (kRowLoads) {
#pragma unroll
        for (int i = 0; i < 4; ++i) b[g][i].u = load16_stream(wseg[g][i] + (size_t)bt * 128);
      } else {
        const bf16_t* p = wrow[g] + (size_t)bt * kUnroll * 32;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) b[g][u].u = load16(p + u * 32);
      }
    }
  };
  Frag16 b0[kGroups][kUnroll], b1[kGroups][kUnroll], b2[kGroups][kUnroll];
  load_w(b0, 0);
  if (nb > 1) load_w(b1, 1);

  // Pairs routed to this expert, in pair order, with their routing weights,
  // 256 pairs per round: each thread reads one
  // pair's expert id and weight, and the hits are ranked by wave ballots.
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int ce = 0;
  for (int base = 0; base < npairs; base += 256) {
    const int p = base + tid;
    const bool in = p < npairs;
    const int pe = in ? idx[p] : -1;
    const float pwv = in ? topk_w[p] : 0.f;
    const bool hit = pe == e;
    const uint64_t mm = __ballot(hit);
    if (lane == 0) wave_hits[wave] = __popcll(mm);
    __syncthreads();
    int before = ce;
    for (int w = 0; w < wave; ++w) before += wave_hits[w];
    if (hit) {
      const int slot = before + __popcll(mm & lt_mask);
      plist[slot] = p;
      wlist[slot] = pwv;
    }
    ce += (wave_hits[0] + wave_hits[1]) + (wave_hits[2] + wave_hits[3]);
    __syncthreads();
  }

  // One pass over the weights for RG row groups of 16 pairs (pairs p0 ..
  // p0 + 16 RG - 1); MFMA row r16 of group rg is pair p0 + 16 rg + r16, rows
  // past the expert's pairs repeat its last pair and are never stored.
  auto pass = [&](auto rg_tag, int p0) {
    constexpr int RG = decltype(rg_tag)::value;
    if (p0 > 0) {
      load_w(b0, 0);
      if (nb > 1) load_w(b1, 1);
    }
    const bf16_t* xr[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      const int pr = plist[min(p0 + rg * 16 + r16, ce - 1)];
      xr[rg] = x + (size_t)(kMode == kGemmRoutedLinear ? pr : pr / k) * d + q * 8;
    }
    auto load_x = [&](Frag16 (&f)[RG][kUnroll], int bt) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) f[rg][u].u = load16(xr[rg] + (bt * kUnroll + u) * 32);
    };
    // Ring of register batches: three deep for one row group, two for two
    // (which holds twice the token fragments per batch).
    constexpr int kRing = RG == 1 ? 3 : 2;
    Frag16 x0[RG][kUnroll], x1[RG][kUnroll], x2[RG][kUnroll];
    load_x(x0, 0);
    if (nb > 1) load_x(x1, 1);
    if (kRing == 3 && nb > 2) {
      load_w(b2, 2);
      load_x(x2, 2);
    }
    f32x4 acc[RG][kGroups];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int g = 0; g < kGroups; ++g) acc[rg][g] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Batch bt's MFMAs from (bc, xc), then refill them with batch bt + kRing.
    auto batch = [&](int bt, Frag16 (&bc)[kGroups][kUnroll], Frag16 (&xc)[RG][kUnroll]) {
      Frag16 bf[kGroups][kUnroll];
      if constexpr (kRowLoads) {
        char* scr = wscr[wave];
#pragma unroll
        for (int g = 0; g < kGroups; ++g)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = 16 * g + 4 * i + (lane >> 4);
            *reinterpret_cast<u32x4*>(scr + row * 256 + ((((lane & 15) ^ (row & 15))) << 4)) = bc[g][i].u;
          }
        __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(63));
#pragma unroll
        for (int g = 0; g < kGroups; ++g)
#pragma unroll
          for (int u = 0; u < kUnroll; ++u)
            bf[g][u].u = *reinterpret_cast<const u32x4*>(scr + (16 * g + r16) * 256 + ((((4 * u + q) ^ r16)) << 4));
      } else {
#pragma unroll
        for (int g = 0; g < kGroups; ++g)
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) bf[g][u] = bc[g][u];
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
          for (int g = 0; g < kGroups; ++g)
            acc[rg][g] = mfma16x16x32(xc[rg][u].h, bf[g][u].h, acc[rg][g]);
      if (bt + kRing < nb) {
        load_w(bc, bt + kRing);
        load_x(xc, bt + kRing);
      }
    };
    for (int bt = 0; bt < nb; bt += kRing) {
      batch(bt, b0, x0);
      if (bt + 1 < nb) batch(bt + 1, b1, x1);
      if (kRing == 3 && bt + 2 < nb) batch(bt + 2, b2, x2);
    }
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = p0 + rg * 16 + q * 4 + v;
        if (r < ce) {
          if constexpr (kMode == kGemmRoutedSwiGLU) {
            // Group 0 is the gate block, group 1 its up block (N % 32 == 0).
            bf16_t* dst = out_h + (size_t)plist[r] * (N / 2);
            if (ncol[0] < N)
              dst[(ncol[0] - r16) / 2 + r16] = (bf16_t)(siluf(acc[rg][0][v]) * acc[rg][1][v]);
          } else {
            const float wt = wlist[r];
            f16_t* dst = partial + (size_t)plist[r] * N;
#pragma unroll
            for (int g = 0; g < kGroups; ++g) {
              if (ncol[g] < N) {
                const float z = acc[rg][g][v];
                if constexpr (kMode == kGemmRoutedSilu) dst[ncol[g]] = (f16_t)(wt * siluf(z));
                else dst[ncol[g]] = (f16_t)(wt * z);
              }
            }
          }
        }
      }
    }
  };
  // Experts with more than 16 pairs take 32 per pass (two row groups), so up
  // to 32 pairs cost one pass over the weights.
  if (!kPair32 || ce <= 16) {
    for (int p0 = 0; p0 < ce; p0 += 16) pass(std::integral_constant<int, 1>{}, p0);
  } else {
    for (int p0 = 0; p0 < ce; p0 += 32) pass(std::integral_constant<int, 2>{}, p0);
  }
}

// ---- very small T: each chain's weights in registers, k split over waves ----
//
// With a handful of tokens only a few experts are touched, so the kernel
// above runs few workgroups, each walking its k loop in several rounds of
// loads.  Here a workgroup owns one (touched expert, column group): 16
// columns, or a 16-column gate block and its up block for the SwiGLU
// epilogue (80 or 160 KB of weights at d = 2560).  Its kWaves waves each load
// their share of the k steps (weight and token fragments) into registers at
// once, and the MFMA chain of every 16 x 16 output tile then runs through the
// shares in order, wave after wave, the fp32 accumulators handed on through
// LDS.  It is the same chain as in the other kernels (same operands, same
// order), so the bits are the same.  Workgroup i takes the (i / groups)-th
// touched expert in index order (the touched set is read from the routing);
// the weights stay in registers across passes of 16 pairs.  Epilogues as
// decode_kernel's kMode.
constexpr int kChainMaxPairs = 64;  // T * k this kernel accepts

template <int kQ, int kMode, int kWaves>  // kQ: k steps per wave (at most)
__global__ __launch_bounds__(64 * kWaves) void decode_chain_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ W,
    const int32_t* __restrict__ idx, const float* __restrict__ topk_w,
    f16_t* __restrict__ partial, bf16_t* __restrict__ out_h, int T, int d, int N, int E, int k) {
  constexpr int kG = kMode == kGemmRoutedSwiGLU ? 2 : 1;  // 16-column groups
  __shared__ int plist[kChainMaxPairs];
  __shared__ float wlist[kChainMaxPairs];
  __shared__ f32x4 handoff[kG][64];
  __shared__ unsigned long long touched[2];  // E <= 128
  __shared__ int wave_hits[kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r16 = lane & 15;
  const int npairs = T * k;  // <= kChainMaxPairs (launch condition)
  const int groups = N / (16 * kG);
  const int rank = blockIdx.x / groups;
  const int n0 = (blockIdx.x % groups) * 16 * kG;

  // The routing, read once: the touched experts, this workgroup's one, and
  // its pairs in pair order (one ballot round: npairs <= 64).
  const bool in = tid < npairs;
  const int pe = in ? idx[tid] : -1;
  const float pwv = in ? topk_w[tid] : 0.f;
  if (tid < 2) touched[tid] = 0ull;
  __syncthreads();
  if (pe >= 0 && pe < E) atomicOr(&touched[pe >> 6], 1ull << (pe & 63));
  __syncthreads();
  const uint64_t m0 = touched[0], m1 = touched[1];
  const int c0 = __popcll(m0);
  if (rank >= c0 + __popcll(m1)) return;  // uniform across the workgroup
  uint64_t m = rank < c0 ? m0 : m1;
  for (int i = rank < c0 ? rank : rank - c0; i > 0; --i) m &= m - 1;
  const int e = (rank < c0 ? 0 : 64) + __ffsll((unsigned long long)m) - 1;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const bool hit = pe == e;
  const uint64_t mm = __ballot(hit);
  if (lane == 0) wave_hits[wave] = __popcll(mm);
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wave_hits[w];
  int ce = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) ce += wave_hits[w];
  if (hit) {
    const int slot = before + __popcll(mm & lt_mask);
    plist[slot] = tid;
    wlist[slot] = pwv;
  }
  __syncthreads();

  // This wave's steps [s0, s0 + ns) of the chain.  Its weight fragments are
  // requested together with the first pass's token fragments (one round trip).
  const int steps = d / 32;
  const int per = ceil_div(steps, kWaves);  // <= kQ (launch condition)
  const int s0 = min(steps, wave * per);
  const int ns = min(steps, s0 + per) - s0;
  Frag16 wf[kG][kQ];
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    const bf16_t* wrow = W + ((size_t)e * N + n0 + g * 16 + r16) * d + q * 8;
#pragma unroll
    for (int i = 0; i < kQ; ++i)
      if (i < ns) wf[g][i].u = load16(wrow + (s0 + i) * 32);
  }

  for (int p0 = 0; p0 < ce; p0 += 16) {
    // Token fragments of this pass (MFMA row r16 = pair p0 + r16; rows past
    // the expert's pairs repeat its last pair and are never stored).
    const int pr = plist[min(p0 + r16, ce - 1)];
    const bf16_t* xr = x + (size_t)(kMode == kGemmRoutedLinear ? pr : pr / k) * d + q * 8;
    Frag16 xf[kQ];
#pragma unroll
    for (int i = 0; i < kQ; ++i)
      if (i < ns) xf[i].u = load16(xr + (s0 + i) * 32);
    f32x4 acc[kG];
#pragma unroll
    for (int g = 0; g < kG; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int w = 0; w < kWaves; ++w) {
      if (wave == w) {
#pragma unroll
        for (int g = 0; g < kG; ++g) {
          if (w > 0) acc[g] = handoff[g][lane];
#pragma unroll
          for (int i = 0; i < kQ; ++i)
            if (i < ns) acc[g] = mfma16x16x32(xf[i].h, wf[g][i].h, acc[g]);
          if (w < kWaves - 1) handoff[g][lane] = acc[g];
        }
      }
      __syncthreads();
    }
    if (wave == kWaves - 1) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = p0 + q * 4 + v;
        if (r < ce) {
          if constexpr (kMode == kGemmRoutedSwiGLU) {
            out_h[(size_t)plist[r] * (N / 2) + n0 / 2 + r16] =
                (bf16_t)(siluf(acc[0][v]) * acc[1][v]);
          } else {
            const float z = acc[0][v];
            f16_t* dst = partial + (size_t)plist[r] * N + n0 + r16;
            if constexpr (kMode == kGemmRoutedSilu) *dst = (f16_t)(wlist[r] * siluf(z));
            else *dst = (f16_t)(wlist[r] * z);
          }
        }
      }
    }
  }
}

// ---- few tokens, many experts each: token-major, the combine fused ---------
//
// With a handful of tokens the per-expert kernels above spread each token's k
// weight reads over k workgroups, and a separate combine then sums the k
// partial rows.  Here a workgroup owns one (token, 16-column group) and runs
// all of that token's k chains, one slot per wave (two for k > 4), so the
// k-way combine happens in the workgroup: fp16(w * SiLU(z)) of each slot,
// widened and summed in slot order, rounded once to bf16 -- the combine
// kernel's arithmetic.  Each chain is the one of the other kernels (token in
// the MFMA's rows, here all 16 rows, the same steps in the same order), so
// the bits are the same.
//
// A slot's 16 weight rows stream through a ring of kS LDS stages private to
// its wave: chunk j holds k steps 4j .. 4j + 3 (256 B of each row), copied
// by 1 KB direct loads of whole row segments (16 lanes per row), the piece p
// of row r at p ^ (r & 15) so that the 16 rows a fragment read touches fall
// in distinct bank groups.  Each wave also keeps its own copy of the token's
// row in LDS (the A fragment is one 64-byte piece read by all 16 rows).  No
// wave reads another's stages, so the loop has no barrier, only the wave's
// own counter waits.  Slots whose expert id is outside [0, E) (caller's
// routing) load expert 0's rows and add nothing.
constexpr int kTokSeg = 4 * 64;          // bytes of a row per chunk (4 k steps)
constexpr int kTokSlot = 16 * kTokSeg;   // one slot's 16 rows per chunk
constexpr int kTokHeader = 512;          // ids, weights, the slots' fp16 rows

__host__ __device__ inline int tok_x_bytes(int d) { return ceil_div(d * 2, 1024) * 1024; }
template <int kSW, int kS>
static int tok_smem(int d) { return kTokHeader + 4 * (tok_x_bytes(d) + kS * kSW * kTokSlot); }

// kRoute: the routing comes as the small-T router's class partials (plog, Tp
// rows per class plane); every wave adds them in class order and selects the
// token's top k with topk_tokens, the router's own selection (so each wave
// starts its weight loads without waiting for another), and wave 0 of the
// workgroups of column group 0 also writes the routing to idx / topk_w.
// kNt: the weight loads carry the non-temporal hint (chosen by T, see
// token_nontemporal).
template <int kSW, int kS, bool kRoute, bool kNt>  // kSW: slots per wave (k <= 4 * kSW); kS: ring stages
__global__ __launch_bounds__(256) void decode_token_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ W, int32_t* __restrict__ idx,
    float* __restrict__ topk_w, const float* __restrict__ plog, int Tp,
    const float* __restrict__ bias, float scale, bf16_t* __restrict__ out,
    const int64_t* __restrict__ slot, long long num_slots, bf16_t* __restrict__ cache, int T, int d,
    int N, int E, int k) {
  constexpr int kLoads = 4 * kSW;  // direct loads per wave per chunk
  static_assert((kS - 2) * kLoads < 64, "vmcnt range");
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  int* sh_e = reinterpret_cast<int*>(smem);                 // [8]
  float* sh_w = reinterpret_cast<float*>(smem + 32);        // [8]
  f16_t* sh_p = reinterpret_cast<f16_t*>(smem + 64);        // [8][16]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, r16 = lane & 15;
  const int groups = N / 16;
  const int t = blockIdx.x / groups;
  const int n0 = (blockIdx.x % groups) * 16;
  const int xb = tok_x_bytes(d);
  char* region = smem + kTokHeader + wave * (xb + kS * kSW * kTokSlot);
  char* ring = region + xb;
  const int steps = d / 32;
  const int nch = ceil_div(steps, 4);

  // The token's row into this wave's copy (element order kept; the last
  // load's lanes past d repeat the row's last piece, never read).  It does
  // not depend on the routing, so it is requested first.
  const bf16_t* xrow = x + (size_t)t * d;
  for (int i = 0; i < xb / 1024; ++i)
    __builtin_amdgcn_global_load_lds((const void*)(xrow + min(i * 512 + lane * 8, d - 8)),
                                     (lds_void*)(region + i * 1024), 16, 0, 0);

  // This wave's slots' expert ids and weights.
  int rs_e[kSW];
  float rs_w[kSW];
  if constexpr (kRoute) {
    const size_t cls = (size_t)Tp * kMaxExperts;
    const float* srcp = plog + (size_t)t * kMaxExperts + lane;
    const float lg[1] = {((srcp[0] + srcp[cls]) + srcp[2 * cls]) + srcp[3 * cls]};
    const float b_lane = (bias != nullptr && lane < E) ? bias[lane] : 0.f;
    int my_idx[1];
    float my_w[1];
    topk_tokens<1>(lg, b_lane, lane, E, k, scale, my_idx, my_w);
#pragma unroll
    for (int s2 = 0; s2 < kSW; ++s2) {
      const int j = wave + 4 * s2;
      rs_e[s2] = j < k ? __builtin_amdgcn_readlane(my_idx[0], j) : -1;
      rs_w[s2] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w[0]), j & 63));
    }
    if (wave == 0 && lane < k) {  // the ids for the combine below
      sh_e[lane] = my_idx[0];
      if (n0 == 0) {
        idx[(size_t)t * k + lane] = my_idx[0];
        topk_w[(size_t)t * k + lane] = my_w[0];
      }
    }
  } else {
    if (tid < k) {
      sh_e[tid] = idx[(size_t)t * k + tid];
      sh_w[tid] = topk_w[(size_t)t * k + tid];
    }
    __syncthreads();
#pragma unroll
    for (int s2 = 0; s2 < kSW; ++s2) {
      const int j = wave + 4 * s2;
      rs_e[s2] = j < k ? sh_e[j] : -1;
      rs_w[s2] = j < k ? sh_w[j] : 0.f;
    }
  }

  // This wave's slots and the source of its lane in each direct load: load
  // i of slot s covers rows 4i .. 4i + 3, the lane's row 4i + lane / 16 and
  // logical piece (lane % 16) ^ (row & 15).
  int sj[kSW];
  bool valid[kSW];
  const bf16_t* src[kSW][4];
  int off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * i + lane / 16;
    off[i] = ((lane % 16) ^ row) * 8;
  }
#pragma unroll
  for (int s = 0; s < kSW; ++s) {
    sj[s] = wave + 4 * s;
    const int e = rs_e[s];
    valid[s] = e >= 0 && e < E;
    const int ee = valid[s] ? e : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      src[s][i] = W + ((size_t)ee * N + n0 + 4 * i + lane / 16) * d;
  }
  auto issue = [&](int j) {
    char* stage = ring + (j % kS) * (kSW * kTokSlot);
#pragma unroll
    for (int s = 0; s < kSW; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(src[s][i] + min(j * 128 + off[i], d - 8)),
                                         (lds_void*)(stage + s * kTokSlot + i * 1024), 16, 0,
                                         kNt ? kLdsLoadNonTemporal : 0);
  };

  f32x4 acc[kSW];
#pragma unroll
  for (int s = 0; s < kSW; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < kS - 1 && j < nch; ++j) issue(j);
  for (int j = 0; j < nch; ++j) {
    if (j + kS - 2 < nch) __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm((kS - 2) * kLoads));
    else __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
    const char* stage = ring + (j % kS) * (kSW * kTokSlot);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int st = 4 * j + u;
      if (st < steps) {
        Frag16 a;
        a.u = *reinterpret_cast<const u32x4*>(region + (st * 32 + 8 * q) * 2);
#pragma unroll
        for (int s = 0; s < kSW; ++s) {
          if (valid[s]) {
            Frag16 b;
            b.u = *reinterpret_cast<const u32x4*>(stage + s * kTokSlot + r16 * kTokSeg +
                                                  (((u * 4 + q) ^ r16) << 4));
            acc[s] = mfma16x16x32(a.h, b.h, acc[s]);
          }
        }
      }
    }
    asm volatile("" ::: "memory");
    if (j + kS - 1 < nch) issue(j + kS - 1);
  }
  __builtin_amdgcn_s_waitcnt(0);
  // Row 0 of each chain (lanes 0 .. 15, element 0) is the token's z.
  if (lane < 16) {
#pragma unroll
    for (int s = 0; s < kSW; ++s)
      if (valid[s]) sh_p[sj[s] * 16 + lane] = (f16_t)(rs_w[s] * siluf(acc[s][0]));
  }
  __syncthreads();
  if (tid < 16) {
    float sum = 0.f;
    bool first = true;
    for (int j = 0; j < k; ++j) {
      const int e = sh_e[j];
      if (e < 0 || e >= E) continue;
      const float v = (float)sh_p[j * 16 + tid];
      sum = first ? v : sum + v;
      first = false;
    }
    const bf16_t r = (bf16_t)sum;
    if (out != nullptr) out[(size_t)t * N + n0 + tid] = r;
    if (cache != nullptr) {
      const long long sl = slot[t];
      if (sl >= 0 && sl < num_slots) cache[(size_t)sl * N + n0 + tid] = r;
    }
  }
}

// Whether the token-major kernel takes a call (value experts): 0 = no, else
// its ring stages.  Measured at d = 2560, N = 1024, k = 4 (graph replay, 4
// weight copies; per-expert kernels and the combine, the best of them, vs
// this kernel with 4 / 3 stages), call times in us:
//   T          1     2     4     6     8     12    16    24    32
//   others     16.5  20.3  29.6  37.2  43.7  58.9  62.1  64.6  66.0
//   4 stages   14.9  16.1  21.0  31.1  36.2  49.5  60.0  81.9  104.0
//   3 stages   16.2  -     21.5  -     34.3  49.0  54.7  -     -
// and, once the weight-streaming kernel's row loads took the non-temporal
// hint (one session, token-major vs streaming kernel):
//   T          6     8     10    12    14    16
//   token      26.2  30.0  42.5  46.2  50.0  52.7
//   streaming  34.1  38.0  43.9  49.6  49.6  50.8
// so it takes T * k <= 48, with 4 stages (84 KB of LDS, one workgroup per
// CU) while its workgroups fit in one per CU and 3 (68 KB, two per CU)
// beyond.  kOvDecodeChain = 3 forces it wherever it fits, 1 and 2 keep it
// off.
int decode_token_stages(int T, int d, int N, int E, int k) {
  (void)E;
  const int ov = override_value(kOvDecodeChain);
  if (ov == 1 || ov == 2) return 0;
  if (k > 8 || N % 16 != 0 || d % 64 != 0) return 0;
  if (ov != 3 && (long long)T * k > 48) return 0;
  if (k > 4) return tok_smem<2, 3>(d) <= 160 * 1024 ? 3 : 0;
  const int st = (long long)T * (N / 16) <= 256 ? 4 : 3;
  if (st == 4 && tok_smem<1, 4>(d) <= 160 * 1024) return 4;
  return tok_smem<1, 3>(d) <= 160 * 1024 ? 3 : 0;
}

// Whether the token kernel's weight loads take the non-temporal hint.
// Measured on the value experts (k = 4, graph replay, weights rotated over 4
// copies), call time in us without / with it:
//   T        1      2      4      6      8      12     16
//   plain    13.69  14.86  19.40  27.41  32.14  47.65  52.87
//   hint     13.95  15.30  18.96  26.39  30.12  46.70  54.25
// so it is taken for T = 3 .. 12 at k <= 4 (other k: not measured, plain).
static bool token_nontemporal(const DecodeTokenArgs& a) { return a.k <= 4 && a.T >= 3 && a.T <= 12; }

template <int kSW, int kS, bool kNt>
static hipError_t launch_token_nt(const DecodeTokenArgs& a, hipStream_t stream) {
  auto kern = a.plog != nullptr ? decode_token_kernel<kSW, kS, true, kNt>
                                : decode_token_kernel<kSW, kS, false, kNt>;
  const int smem = tok_smem<kSW, kS>(a.d);
  static std::atomic<unsigned long long> attr_done{0};
  hipError_t err = once_per_device(attr_done, [&]() {
    hipError_t e1 = hipFuncSetAttribute((const void*)decode_token_kernel<kSW, kS, true, kNt>,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    hipError_t e2 = hipFuncSetAttribute((const void*)decode_token_kernel<kSW, kS, false, kNt>,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    return e1 != hipSuccess ? e1 : e2;
  });
  if (err != hipSuccess) return err;
  kern<<<dim3((unsigned)(a.T * (a.N / 16))), 256, smem, stream>>>(
      a.x, a.W, a.idx, a.topk_w, a.plog, a.Tp, a.bias, a.scale, a.out, a.slot, a.num_slots,
      a.cache, a.T, a.d, a.N, a.E, a.k);
  return hipGetLastError();
}

template <int kSW, int kS>
static hipError_t launch_token_cfg(const DecodeTokenArgs& a, hipStream_t stream) {
  return token_nontemporal(a) ? launch_token_nt<kSW, kS, true>(a, stream)
                              : launch_token_nt<kSW, kS, false>(a, stream);
}

hipError_t launch_decode_token(const DecodeTokenArgs& a, int stages, hipStream_t stream) {
  if (a.k > 8 || a.N % 16 != 0 || a.d % 64 != 0 || a.T > kDecodeMaxT) return hipErrorInvalidValue;
  if (a.k > 4) {
    if (stages != 3 || tok_smem<2, 3>(a.d) > 160 * 1024) return hipErrorInvalidValue;
    return launch_token_cfg<2, 3>(a, stream);
  }
  if (stages == 4 && tok_smem<1, 4>(a.d) <= 160 * 1024) return launch_token_cfg<1, 4>(a, stream);
  if (stages == 3 && tok_smem<1, 3>(a.d) <= 160 * 1024) return launch_token_cfg<1, 3>(a, stream);
  return hipErrorInvalidValue;
}

// Whether the chain kernel takes a call: 0, or its k steps per wave.  The
// SwiGLU epilogue holds two groups of weights, so it splits k over 8 waves.
// T * k up to which it is the default, measured: the value experts (d =
// 2560, N = 1024) at T = 1, 2, 4, 8 took 16.1 / 20.1 / 30.5 / 50.4 us against
// 33.8 / 35.3 / 37.4 and 43.7 us for the streaming kernel with one column
// group per wave; the FFN (100 experts of width 768, top-8) at T = 1, 2, 3, 4
// 57 / 83 / 109 / 129 us against 94 / 103 / 114 / 121 us for the streaming
// kernels with their non-temporal row loads (before those loads, T = 4 took
// 150 us there, and the chain kernel was the default up to 32 pairs).
static int chain_auto_pairs(int mode) { return mode == kGemmRoutedSilu ? 16 : 24; }
static int chain_waves(int mode) { return mode == kGemmRoutedSwiGLU ? 8 : 4; }
static int chain_steps_per_wave(const DecodeArgs& a) {
  // 1 / 2 force it on / off (tests, measurement); 3 forces the token-major kernel.
  const int ov = override_value(kOvDecodeChain);
  const bool force_on = ov == 1, force_off = ov == 2 || ov == 3;
  const int per = ceil_div(a.d / 32, chain_waves(a.mode));
  const int max_per = a.mode == kGemmRoutedSwiGLU ? 16 : 24;  // registers (two groups)
  const bool fits = (long long)a.T * a.k <= kChainMaxPairs && a.E <= 128 &&
                    a.N % (a.mode == kGemmRoutedSwiGLU ? 32 : 16) == 0 && per <= max_per;
  if (!fits || force_off) return 0;
  if (!force_on && (long long)a.T * a.k > chain_auto_pairs(a.mode)) return 0;
  return per <= 8 ? 8 : per <= 16 ? 16 : 24;
}

template <int kMode, int kWaves>
static hipError_t launch_chain(const DecodeArgs& a, int q, hipStream_t stream) {
  constexpr int kG = kMode == kGemmRoutedSwiGLU ? 2 : 1;
  const dim3 grid((unsigned)(std::min(a.E, a.T * a.k) * (a.N / (16 * kG))));
  auto kern = q == 8 ? decode_chain_kernel<8, kMode, kWaves> : decode_chain_kernel<16, kMode, kWaves>;
  if constexpr (kMode != kGemmRoutedSwiGLU)  // at most 16 steps per wave for SwiGLU
    if (q == 24) kern = decode_chain_kernel<24, kMode, kWaves>;
  kern<<<grid, 64 * kWaves, 0, stream>>>(a.x, a.W, a.idx, a.topk_w, a.partial,
                                          (bf16_t*)a.out_h, a.T, a.d, a.N, a.E, a.k);
  return hipGetLastError();
}

template <int kMode, int kGroups>
static auto pick_decode_kernel(bool unroll4, bool pair32) {
  return unroll4 ? (pair32 ? decode_kernel<4, true, kMode, kGroups>
                           : decode_kernel<4, false, kMode, kGroups>)
                 : (pair32 ? decode_kernel<2, true, kMode, kGroups>
                           : decode_kernel<2, false, kMode, kGroups>);
}

// Narrow outputs (e.g. one GPU's share of the heads under tensor parallelism)
// give too few 128-column workgroups to fill the GPU's two per CU, and so do
// a few tokens, which touch few experts (at most T * k): one 16-column group
// per wave then doubles the workgroups (and the MFMA chains running at once).
// Each group's chain is the same either way, so are the bits.  The SwiGLU
// epilogue needs a gate and an up group in one wave.
template <int kMode>
static hipError_t launch_decode_mode(const DecodeArgs& a, hipStream_t stream) {
  constexpr int kRound = 512;  // two workgroups per CU
  const long long slices = ceil_div(a.N, 128);
  const long long busy = std::min<long long>(a.E, (long long)a.T * a.k) * slices;
  // busy: at most this many 128-column workgroups have pairs.  Measured at
  // d = 2560, N = 1024 (T = 8, 10, 12, 14: 43.7 vs 56.8, 52.1 vs 58.1, 58.6
  // vs 59.0, 62.3 vs 61.3 us, narrow vs not), narrow while busy <= 384.
  bool narrow = (long long)a.E * slices < kRound || busy <= 3 * kRound / 4;
  const int groups = override_value(kOvDecodeGroups);  // 1 or 2 (tests, measurement)
  if (groups == 1 || groups == 2) narrow = groups == 1;
  narrow = narrow && kMode != kGemmRoutedSwiGLU;
  const dim3 grid(a.E * ceil_div(a.N, narrow ? 64 : 128));
  const bool unroll4 = (a.d / 32) % 4 == 0;
  // 32-pair passes (fragment loads) once the experts average more than 10
  // pairs; below, 16-pair passes with the non-temporal row-segment loads win
  // even though an expert with more than 16 pairs reads its weights twice.
  // Measured on the value experts (k = 4, E = 64), call times in us, 16- vs
  // 32-pair passes: T = 96 64.3 vs 76.2, 128 79.4 vs 80.9, 160 81.5 vs 84.0,
  // 192 98.0 vs 89.0, 256 105 vs 94.
  const bool pair32 = (long long)a.T * a.k > 10LL * a.E;
  auto kern = narrow ? pick_decode_kernel<kMode, kMode == kGemmRoutedSwiGLU ? 2 : 1>(unroll4, pair32)
                     : pick_decode_kernel<kMode, 2>(unroll4, pair32);
  kern<<<grid, 256, 0, stream>>>(a.x, a.W, a.idx, a.topk_w, a.partial, (bf16_t*)a.out_h, a.T, a.d,
                                 a.N, a.E, a.k);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.T > kDecodeMaxT || a.k > kMaxTopK || a.d % 64 != 0 || a.N % 64 != 0)
    return hipErrorInvalidValue;
  if (const int q = chain_steps_per_wave(a)) {
    switch (a.mode) {
      case kGemmRoutedSilu: return launch_chain<kGemmRoutedSilu, 4>(a, q, stream);
      case kGemmRoutedSwiGLU:
        if (a.out_h == nullptr) return hipErrorInvalidValue;
        return launch_chain<kGemmRoutedSwiGLU, 8>(a, q, stream);
      case kGemmRoutedLinear: return launch_chain<kGemmRoutedLinear, 4>(a, q, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.mode) {
    case kGemmRoutedSilu: return launch_decode_mode<kGemmRoutedSilu>(a, stream);
    case kGemmRoutedSwiGLU:
      if (a.N % 32 != 0 || a.out_h == nullptr) return hipErrorInvalidValue;
      return launch_decode_mode<kGemmRoutedSwiGLU>(a, stream);
    case kGemmRoutedLinear: return launch_decode_mode<kGemmRoutedLinear>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mova
