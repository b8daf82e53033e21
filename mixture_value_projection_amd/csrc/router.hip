// Router: logits = x Wr^T (fp32 accumulation of bf16 products on MFMA),
// sigmoid scores, bias added for selection, wave-wide top-k with the lower
// expert index winning ties, renormalised weights times `scale`.
//
// Method: page "MoVA: routing the value vectors, and why the KV cache does not
// notice", section "Where the routing happens" (weight-only router linear map,
// sigmoid scoring, top-4, scaling factor 2.5).
//
// Summation order, shared by every router kernel so that a token's logits are
// the same bits whichever kernel, block shape or call processed it: the
// d-long dot product of a (token, expert) pair is split into four residue
// classes of 32-wide k steps (step mod 4); class rc is one MFMA chain over
// steps rc, rc + 4, rc + 8, ... in increasing order, with the token in MFMA
// row t % 16 and the expert in column e % 16; the four class partials are
// then added in class order, ((p0 + p1) + p2) + p3.  (A chain padded to a
// whole number of load batches multiplies a zeroed token operand, adding +0,
// which can only turn a -0 partial into +0.)
//
// Kernels:
//   router_lds_kernel      one workgroup per 16, 32 or 64 tokens, wave =
//                          class, operands staged through LDS by direct
//                          loads; selection and the per-chunk dispatch
//                          histogram in the same kernel (T above the decode
//                          range, and routing-only calls);
//   router_partial_kernel  + router_topk_kernel: the same chains spread over
//                          single-wave workgroups for small T.
#include <stdlib.h>
#include <string.h>

#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace mova {

// ---- LDS-staged router: one workgroup of 4 waves per TM = 16 * TG tokens ----
//
// A fragment load straight from memory (lane = row % 16, 16 B of k per lane)
// touches 16 rows per 16 lanes, and the per-request cost of the vector cache,
// not bandwidth, then sets the load rate (measured: the same bytes with 4
// lanes per row arrive three times sooner).  Here every load is a
// 1 KB direct global -> LDS copy of whole row segments: chunk j holds k steps
// kCS j .. kCS j + kCS - 1 of the router weight's 64 rows and of the tile's
// token rows (kCS * 64 B per row, one 16- or 32-lane group per row).  The
// chunks stream through a ring of kS LDS stages, kS - 1 chunks ahead, with
// one barrier per chunk.  Within a row segment the 16-byte piece p sits at
// p ^ (row & 15), so the 16 rows a fragment read touches fall in distinct
// bank groups.  Wave rc runs class rc's chains (its steps of each chunk, in
// increasing order) for the TG token groups against the four expert blocks:
// the chains of the small-T router, so the same bits.  Selection: lane =
// expert, TM / 4 tokens per wave (topk_tokens).  A workgroup's tokens form
// one dispatch chunk: with chunk_counts given, it receives the workgroup's
// per-expert pair counts.
template <int TG, int kCS, int kS, int kEB>
constexpr int router_lds_body() {
  constexpr int ring = kS * (16 * kEB + 16 * TG) * kCS * 64;
  constexpr int part = 4 * 16 * TG * (16 * kEB + 1) * 4;
  return ring > part ? ring : part;
}

template <int TG, int kCS, int kS, int kEB>
__global__ __launch_bounds__(256) void router_lds_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr, const float* __restrict__ bias,
    int T, int d, int E, int k, float scale,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out, int32_t* __restrict__ chunk_counts) {
  static_assert(kCS == 4 || kCS == 8, "row segments of 16 or 32 pieces");
  static_assert(kEB == 4 || kEB == 8, "64 or 128 expert rows");
  constexpr int TM = 16 * TG;
  constexpr int kER = 16 * kEB;                  // expert rows (one or two per lane)
  constexpr int kRows = kER + TM;                // the router weight's rows, then the tokens'
  constexpr int kSeg = kCS * 64;                 // bytes of a row per chunk
  constexpr int kLanesRow = kSeg / 16;           // lanes (16-byte pieces) per row segment
  constexpr int kRowsLoad = 64 / kLanesRow;      // row segments per 1 KB load
  constexpr int kStage = kRows * kSeg;
  constexpr int kLoads = kRows / kRowsLoad / 4;  // direct loads per wave per chunk
  static_assert(kRows % (4 * kRowsLoad) == 0, "loads split evenly over the waves");
  static_assert((kS - 2) * kLoads < 64, "vmcnt range");
  constexpr int kPad = kER + 1;
  // Dynamic LDS (router_lds_body bytes, then kER ints): the stages (later the
  // class partials), then the histogram.  (With a static array, the compiler
  // makes every fragment read wait for all of the ring's outstanding direct
  // loads.)
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  int* hist = reinterpret_cast<int*>(smem + router_lds_body<TG, kCS, kS, kEB>());

  const int lane = threadIdx.x & 63;
  const int rc = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4, r16 = lane & 15;
  const int t0 = blockIdx.x * TM;
  const int steps = d / 32;
  const int nch = ceil_div(steps, kCS);

  if (threadIdx.x < kER) hist[threadIdx.x] = 0;
  // The selection biases, requested now so that their latency hides behind
  // the loop.
  const float b_lane = (bias != nullptr && lane < E) ? bias[lane] : 0.f;
  const float b_lane1 = (kEB == 8 && bias != nullptr && lane + 64 < E) ? bias[lane + 64] : 0.f;

  // This lane's part of its direct loads: load i fills row segments
  // (rc * kLoads + i) * kRowsLoad ..; the lane's 16 B land at physical piece
  // lane % kLanesRow of row lane / kLanesRow, and hold the row's logical
  // piece (lane % kLanesRow) ^ (row & 15).  Expert rows past E and token
  // rows past T are clamped (computed, never used); pieces past d load the
  // row's last piece (never read).
  const bf16_t* src[kLoads];
  int off[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int row = (rc * kLoads + i) * kRowsLoad + lane / kLanesRow;
    src[i] = row < kER ? wr + (size_t)min(row, E - 1) * d
                       : x + (size_t)min(t0 + row - kER, T - 1) * d;
    off[i] = (((lane % kLanesRow) ^ (row & 15))) * 8;
  }
  auto issue = [&](int j) {
    char* stage = smem + (j % kS) * kStage;
    const int base = j * kCS * 32;
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(src[i] + min(base + off[i], d - 8)),
                                       (lds_void*)(stage + (rc * kLoads + i) * 1024), 16, 0, 0);
  };

  f32x4 acc[TG][kEB];
#pragma unroll
  for (int g = 0; g < TG; ++g)
#pragma unroll
    for (int eb = 0; eb < kEB; ++eb) acc[g][eb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Chunk j: wait for this wave's loads of it (those of the next kS - 2
  // chunks may stay in flight) and its LDS reads, barrier (every wave's loads
  // of chunk j have landed and every wave is done with chunk j - 1's stage),
  // run the wave's steps of chunk j, then refill chunk j - 1's stage with
  // chunk j + kS - 1 (issued after the fragment reads, so that the compiler
  // does not wait for the ring's loads before them).
  for (int j = 0; j < kS - 1 && j < nch; ++j) issue(j);
  for (int j = 0; j < nch; ++j) {
    if (j + kS - 2 < nch) __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm((kS - 2) * kLoads));
    else __builtin_amdgcn_s_waitcnt(0);
    raw_barrier();
    const char* stage = smem + (j % kS) * kStage;
#pragma unroll
    for (int u = 0; u < kCS / 4; ++u) {
      const int sl = 4 * u + rc;  // the wave's step within the chunk
      if (j * kCS + sl < steps) {
        const int pc = (((sl * 4 + q) ^ r16)) << 4;
        Frag16 b[kEB];
#pragma unroll
        for (int eb = 0; eb < kEB; ++eb)
          b[eb].u = *reinterpret_cast<const u32x4*>(stage + (eb * 16 + r16) * kSeg + pc);
#pragma unroll
        for (int g = 0; g < TG; ++g) {
          Frag16 a;
          a.u = *reinterpret_cast<const u32x4*>(stage + (kER + g * 16 + r16) * kSeg + pc);
#pragma unroll
          for (int eb = 0; eb < kEB; ++eb) acc[g][eb] = mfma16x16x32(a.h, b[eb].h, acc[g][eb]);
        }
      }
    }
    if (j + kS - 1 < nch) issue(j + kS - 1);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // every load has landed and every read is done: the stages hold the partials
  float(*part)[TM][kPad] = reinterpret_cast<float(*)[TM][kPad]>(smem);
#pragma unroll
  for (int g = 0; g < TG; ++g)
#pragma unroll
    for (int eb = 0; eb < kEB; ++eb)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[rc][g * 16 + q * 4 + i][eb * 16 + r16] = acc[g][eb][i];
  __syncthreads();

  // Wave rc selects for tokens rc, rc + 4, rc + 8, ... of the tile.
  constexpr int NT = TM / 4;
  int my_idx[NT];
  float my_w[NT];
  {
    float logit[NT], logit1[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int r = rc + 4 * i;
      logit[i] = ((part[0][r][lane] + part[1][r][lane]) + part[2][r][lane]) + part[3][r][lane];
      if constexpr (kEB == 8)
        logit1[i] = ((part[0][r][lane + 64] + part[1][r][lane + 64]) + part[2][r][lane + 64]) +
                    part[3][r][lane + 64];
    }
    if constexpr (kEB == 8)
      topk_tokens2<NT>(logit, logit1, b_lane, b_lane1, lane, E, k, scale, my_idx, my_w);
    else
      topk_tokens<NT>(logit, b_lane, lane, E, k, scale, my_idx, my_w);
  }
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int t = t0 + rc + 4 * i;
    if (t < T && lane < k) {
      idx_out[(size_t)t * k + lane] = my_idx[i];
      w_out[(size_t)t * k + lane] = my_w[i];
      if (chunk_counts != nullptr) atomicAdd(&hist[my_idx[i]], 1);
    }
  }
  if (chunk_counts != nullptr) {
    __syncthreads();
    if (threadIdx.x < E) chunk_counts[(size_t)blockIdx.x * E + threadIdx.x] = hist[threadIdx.x];
  }
}

// Router configuration for T: tokens per workgroup (the dispatch chunk) and
// LDS stages.  Measured with the value layer's shape (routing alone, graph
// replay, us):
//   T               64    4096  8192  16384  32768
//   16 tok, 3 st    10.2  10.9  16.6  29.0   53.0   (61 KB: two workgroups per CU)
//   16 tok, 6 st    10.3  11.7  21.3  38.9   73.9
//   32 tok, 4 st    13.1  13.9  15.2  27.6   51.5   (97 KB: one per CU)
//   32 tok, 3 st    13.1  13.9  16.0  22.5   40.1   (73 KB: two per CU)
//   64 tok, 4 st    20.1  21.4  22.3  24.8   45.8   (131 KB: one per CU)
//   64 tok, 2 st    21.4  27.8  29.5  31.4   39.4   (67 KB: two per CU)
// Deeper rings do not help: a CU's direct loads run at about 60 GB/s,
// whatever is in flight.  The kOvRouter override forces a configuration
// (1: 16 tokens, 2: 32 tokens with 4 stages, 3: 32 tokens with 3 stages, 4: 64
// tokens) for measurements and tests.
struct RouterChoice {
  int tokens;  // tokens per workgroup (the dispatch chunk)
  int stages;  // LDS stages of the ring
};

static RouterChoice router_choice(int T) {
  switch (override_value(kOvRouter)) {
    case 1: return {16, 3};
    case 2: return {32, 4};
    case 3: return {32, 3};
    case 4: return {64, 2};
    default: break;
  }
  if (T <= 6144) return {16, 3};
  if (T <= 12288) return {32, 4};
  if (T <= 24576) return {32, 3};
  return {64, 2};
}

int router_chunk_tokens(int T) { return router_choice(T).tokens; }  // >= 16 for every choice

template <int TG, int kS, int kEB = 4>
static hipError_t launch_lds_config(const RouterArgs& a, hipStream_t stream) {
  constexpr int kCS = 4;
  auto kern = router_lds_kernel<TG, kCS, kS, kEB>;
  constexpr int smem = router_lds_body<TG, kCS, kS, kEB>() + 16 * kEB * 4;
  static std::atomic<unsigned long long> attr_done{0};
  hipError_t err = once_per_device(attr_done, [&]() {
    return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  });
  if (err != hipSuccess) return err;
  kern<<<ceil_div(a.T, 16 * TG), 256, smem, stream>>>(a.x, a.wr, a.bias, a.T, a.d, a.E, a.k,
                                                      a.scale, a.idx, a.w, a.chunk_counts);
  return hipGetLastError();
}

hipError_t launch_router_lds(const RouterArgs& a, hipStream_t stream) {
  const RouterChoice rch = router_choice(a.T);
  if (rch.tokens == 16) return launch_lds_config<1, 3>(a, stream);
  if (rch.tokens == 32) {
    if (rch.stages == 4) return launch_lds_config<2, 4>(a, stream);
    return launch_lds_config<2, 3>(a, stream);
  }
  return launch_lds_config<4, 2>(a, stream);
}

// The FFN router's configuration (up to 128 experts, two per selecting lane):
// 16 tokens per workgroup, the FFN's dispatch chunk.
hipError_t launch_router_lds_wide(const RouterArgs& a, hipStream_t stream) {
  if (a.E > 128) return hipErrorInvalidValue;
  return launch_lds_config<1, 3, 8>(a, stream);
}

// ---- small T: the same chains spread over many single-wave workgroups ------
//
// Block (g, eb, rc) computes the class-rc partial logits of token group g (16
// tokens) against expert block eb (16 experts), all of its loads issued before
// its MFMAs.  The top-k kernel adds the four class partials in class order and
// selects with one wave per token.  plog rows are ld floats apart (64 for the
// value experts, 128 for the FFN's up to 128 experts).
template <int U>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 2))) void router_partial_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr, int T, int d, int E,
    float* __restrict__ plog /* [4][Tp][ld] */, int Tp, int ld) {
  const int g = blockIdx.x, eb = blockIdx.y, rc = blockIdx.z;
  const int lane = threadIdx.x, q = lane >> 4, r16 = lane & 15;
  const bf16_t* xrow = x + (size_t)min(g * 16 + r16, T - 1) * d + q * 8;
  const bf16_t* wrow = wr + (size_t)min(eb * 16 + r16, E - 1) * d + q * 8;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int steps = d / 32;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int s0 = rc; s0 < steps; s0 += 4 * U) {
    Frag16 a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sc = min(s0 + 4 * u, steps - 1);
      b[u].u = load16(wrow + sc * 32);
      a[u].u = load16(xrow + sc * 32);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      Frag16 av;
      av.u = (s0 + 4 * u < steps) ? a[u].u : zero;
      acc = mfma16x16x32(av.h, b[u].h, acc);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    plog[((size_t)rc * Tp + g * 16 + q * 4 + i) * ld + eb * 16 + r16] = acc[i];
}

__global__ __launch_bounds__(256) void router_topk_kernel(
    const float* __restrict__ plog, int Tp, const float* __restrict__ bias, int T, int E, int k,
    float scale, int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;  // one token per wave
  if (t >= T) return;
  const float b_lane = (bias != nullptr && lane < E) ? bias[lane] : 0.f;
  const size_t cls = (size_t)Tp * kMaxExperts;
  const float* src = plog + (size_t)t * kMaxExperts + lane;
  const float logit = ((src[0] + src[cls]) + src[2 * cls]) + src[3 * cls];
  const float lg[1] = {logit};
  int my_idx[1];
  float my_w[1];
  topk_tokens<1>(lg, b_lane, lane, E, k, scale, my_idx, my_w);
  if (lane < k) {
    idx_out[(size_t)t * k + lane] = my_idx[0];
    w_out[(size_t)t * k + lane] = my_w[0];
  }
}

int router_small_plog_floats(int T) { return 4 * ceil_div(T, 16) * 16 * kMaxExperts; }

hipError_t launch_router_partial(const RouterArgs& a, float* plog, hipStream_t stream) {
  const int G = ceil_div(a.T, 16);
  router_partial_kernel<20><<<dim3(G, 4, 4), 64, 0, stream>>>(a.x, a.wr, a.T, a.d, a.E, plog, G * 16,
                                                             kMaxExperts);
  return hipGetLastError();
}

hipError_t launch_router_partial_wide(const RouterArgs& a, float* plog, hipStream_t stream) {
  if (a.E > kMaxDispatchExperts) return hipErrorInvalidValue;
  const int G = ceil_div(a.T, 16);
  router_partial_kernel<20><<<dim3(G, ceil_div(a.E, 16), 4), 64, 0, stream>>>(
      a.x, a.wr, a.T, a.d, a.E, plog, G * 16, kMaxDispatchExperts);
  return hipGetLastError();
}

hipError_t launch_router_small(const RouterArgs& a, float* plog, hipStream_t stream) {
  const int Tp = ceil_div(a.T, 16) * 16;
  hipError_t err = launch_router_partial(a, plog, stream);
  if (err != hipSuccess) return err;
  router_topk_kernel<<<ceil_div(a.T, 4), 256, 0, stream>>>(plog, Tp, a.bias, a.T, a.E, a.k, a.scale,
                                                          a.idx, a.w);
  return hipGetLastError();
}

}  // namespace mova
