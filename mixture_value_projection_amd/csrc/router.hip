// Router: logits = x Wr^T (fp32 accumulation of bf16 products on MFMA),
// sigmoid scores, bias added for selection, wave-wide top-k with the lower
// expert index winning ties, renormalised weights times `scale`.
//
// Method: page "MoVA: routing the value vectors, and why the KV cache does not
// notice", section "Where the routing happens" (weight-only router linear map,
// sigmoid scoring, top-4, scaling factor 2.5).
//
// One workgroup = 16 waves handles TM = 16 * TG tokens.  The d-long dot
// products are split into four residue classes of 32-wide k steps
// (step mod 4); wave w owns expert block w % 4 (16 experts) and residue class
// w / 4 for all of the block's tokens (TG MFMA tiles accumulated in place).
// Each wave issues the loads of U k steps before their MFMAs, so a wave keeps
// U * (TG + 1) 1-KB loads in flight.  The four class partials meet in LDS and
// are added in class order, so a token's logits are the same bits whichever
// block shape (or call) processed it.  Top-k then runs with one lane per
// expert (E <= 64).  Optionally each workgroup writes how many of its
// (token, slot) pairs chose each expert -- the per-chunk histogram the
// dispatch step scans.
#include "common.h"
#include "kernels.h"

namespace mova {

constexpr int kRouterThreads = 1024;

// Sigmoid, bias-for-selection, top-k and renormalisation for one token, one
// lane per expert.  `logit` is lane e's logit; `scratch` is this wave's own 72
// floats of LDS.  Returns (in lanes j < k) the j-th selected expert and its
// weight.  Selection order: score desc, index asc.
//
// Lane e's rank is the number of experts that come before it in that order,
// counted over all 64 scores (broadcast LDS reads); ranks 0 .. k-1 are the
// selection, in order.  The k chosen sigmoid scores are summed in rank order.
__device__ __forceinline__ void topk_lane(float logit, float b_lane, int lane, int E, int k,
                                          float scale, float* scratch, int& my_idx,
                                          float& my_w) {
  const float sc = sigmoidf_fast(logit);
  const float sel = lane < E ? sc + b_lane : -__builtin_inff();
  scratch[lane] = sel;
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  int rank = 0;
#pragma unroll 16
  for (int j = 0; j < kMaxExperts; ++j) {
    const float v = scratch[j];
    rank += (v > sel || (v == sel && j < lane)) ? 1 : 0;
  }
  if (rank < k) {
    scratch[kMaxExperts + rank] = sc;
    reinterpret_cast<int*>(scratch)[kMaxExperts + kMaxTopK + rank] = lane;
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  float ssum = 0.f;
  for (int j = 0; j < k; ++j) ssum += scratch[kMaxExperts + j];
  const int slot = min(lane, k - 1);
  // Clamped so that even non-finite scores (undefined results) can never
  // produce an out-of-range expert index for the kernels that follow.
  my_idx = min(max(reinterpret_cast<const int*>(scratch)[kMaxExperts + kMaxTopK + slot], 0), E - 1);
  my_w = scale * scratch[kMaxExperts + slot] / ssum;
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

constexpr int kTopkScratch = kMaxExperts + 2 * kMaxTopK;  // floats per wave

template <int TG, int U>
__global__ __launch_bounds__(kRouterThreads) void router_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr, const float* __restrict__ bias,
    int T, int d, int E, int k, float scale,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out, int32_t* __restrict__ chunk_counts) {
  constexpr int TM = 16 * TG;
  constexpr int kWaves = kRouterThreads / 64;
  __shared__ float part[4][TM][kMaxExperts];
  __shared__ int hist[kMaxExperts];
  __shared__ float topk_scratch[kWaves][kTopkScratch];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int eb = wave & 3;   // expert block
  const int rc = wave >> 2;  // k-step residue class
  const int q = lane >> 4;
  const int r16 = lane & 15;
  const int tile_t0 = blockIdx.x * TM;

  if (threadIdx.x < kMaxExperts) hist[threadIdx.x] = 0;
  // A operand: token rows (clamped into range; rows past T are never written).
  const bf16_t* xrow[TG];
#pragma unroll
  for (int g = 0; g < TG; ++g)
    xrow[g] = x + (size_t)min(tile_t0 + g * 16 + r16, T - 1) * d + q * 8;
  // B operand: expert rows (clamped; lanes for experts >= E are masked in top-k).
  const bf16_t* wrow = wr + (size_t)min(eb * 16 + r16, E - 1) * d + q * 8;

  f32x4 acc[TG];
#pragma unroll
  for (int g = 0; g < TG; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Steps s = rc, rc + 4, rc + 8, ... in order; U of them per batch.  Steps
  // past the end read a clamped address and multiply a zeroed operand, so
  // every MFMA runs unconditionally.
  const int steps = d / 32;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int s0 = rc; s0 < steps; s0 += 4 * U) {
    Frag16 a[U][TG], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sc = min(s0 + 4 * u, steps - 1);
      b[u].u = load16(wrow + sc * 32);
#pragma unroll
      for (int g = 0; g < TG; ++g) a[u][g].u = load16(xrow[g] + sc * 32);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = s0 + 4 * u < steps;
#pragma unroll
      for (int g = 0; g < TG; ++g) {
        Frag16 av;
        av.u = live ? a[u][g].u : zero;
        acc[g] = mfma16x16x32(av.h, b[u].h, acc[g]);
      }
    }
  }

#pragma unroll
  for (int g = 0; g < TG; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[rc][g * 16 + q * 4 + i][eb * 16 + r16] = acc[g][i];
  __syncthreads();

  // Top-k: wave `wave` takes tile rows wave, wave + 16, ...; lane = expert.
  const float b_lane = (bias != nullptr && lane < E) ? bias[lane] : 0.f;
  for (int r = wave; r < TM; r += kWaves) {
    const int t = tile_t0 + r;
    if (t >= T) break;
    const float logit = ((part[0][r][lane] + part[1][r][lane]) + part[2][r][lane]) + part[3][r][lane];
    int my_idx;
    float my_w;
    topk_lane(logit, b_lane, lane, E, k, scale, topk_scratch[wave], my_idx, my_w);
    if (lane < k) {
      idx_out[(size_t)t * k + lane] = my_idx;
      w_out[(size_t)t * k + lane] = my_w;
      if (chunk_counts != nullptr) atomicAdd(&hist[my_idx], 1);
    }
  }
  if (chunk_counts != nullptr) {
    __syncthreads();
    if (threadIdx.x < E) chunk_counts[(size_t)blockIdx.x * E + threadIdx.x] = hist[threadIdx.x];
  }
}

int router_tokens_per_block(bool wide) { return wide ? 64 : 16; }

hipError_t launch_router(const RouterArgs& a, bool wide, hipStream_t stream) {
  const int TM = router_tokens_per_block(wide);
  const dim3 grid(ceil_div(a.T, TM));
  if (wide) {
    router_kernel<4, 4><<<grid, kRouterThreads, 0, stream>>>(
        a.x, a.wr, a.bias, a.T, a.d, a.E, a.k, a.scale, a.idx, a.w, a.chunk_counts);
  } else {
    router_kernel<1, 10><<<grid, kRouterThreads, 0, stream>>>(
        a.x, a.wr, a.bias, a.T, a.d, a.E, a.k, a.scale, a.idx, a.w, a.chunk_counts);
  }
  return hipGetLastError();
}


// ---- small T: the same sums spread over many single-wave workgroups --------
//
// Block (g, eb, rc) computes the residue-class-rc partial logits of token
// group g (16 tokens) against expert block eb (16 experts): the same MFMA
// chain, in the same step order, as wave (eb, rc) of router_kernel.  All of
// its loads are issued before its MFMAs.  The top-k kernel then adds the four
// class partials in class order, so the result has the same bits as
// router_kernel's.
template <int U>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 2))) void router_partial_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr, int T, int d, int E,
    float* __restrict__ plog /* [4][Tp][64] */, int Tp) {
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
    plog[((size_t)rc * Tp + g * 16 + q * 4 + i) * kMaxExperts + eb * 16 + r16] = acc[i];
}

__global__ __launch_bounds__(256) void router_topk_kernel(
    const float* __restrict__ plog, int Tp, const float* __restrict__ bias, int T, int E, int k,
    float scale, int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  __shared__ float topk_scratch[4][kTopkScratch];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float b_lane = (bias != nullptr && lane < E) ? bias[lane] : 0.f;
  const size_t cls = (size_t)Tp * kMaxExperts;
  // Wave w handles tokens t0 + w + 4 i (i < 4); every load is issued first.
  const int t0 = blockIdx.x * 16 + wave;
  float p[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float* src = plog + (size_t)min(t0 + 4 * i, Tp - 1) * kMaxExperts + lane;
#pragma unroll
    for (int c = 0; c < 4; ++c) p[i][c] = src[c * cls];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * i;
    if (t >= T) break;
    const float logit = ((p[i][0] + p[i][1]) + p[i][2]) + p[i][3];
    int my_idx;
    float my_w;
    topk_lane(logit, b_lane, lane, E, k, scale, topk_scratch[wave], my_idx, my_w);
    if (lane < k) {
      idx_out[(size_t)t * k + lane] = my_idx;
      w_out[(size_t)t * k + lane] = my_w;
    }
  }
}

int router_small_plog_floats(int T) { return 4 * ceil_div(T, 16) * 16 * kMaxExperts; }

hipError_t launch_router_small(const RouterArgs& a, float* plog, hipStream_t stream) {
  const int G = ceil_div(a.T, 16);
  const int Tp = G * 16;
  router_partial_kernel<20><<<dim3(G, 4, 4), 64, 0, stream>>>(a.x, a.wr, a.T, a.d, a.E, plog, Tp);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  router_topk_kernel<<<G, 256, 0, stream>>>(plog, Tp, a.bias, a.T, a.E, a.k, a.scale, a.idx, a.w);
  return hipGetLastError();
}

}  // namespace mova
