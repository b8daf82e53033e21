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
  const int t = blockIdx.x * 4 + wave;  // one token per wave
  if (t >= T) return;
  const float b_lane = (bias != nullptr && lane < E) ? bias[lane] : 0.f;
  const size_t cls = (size_t)Tp * kMaxExperts;
  const float* src = plog + (size_t)t * kMaxExperts + lane;
  const float logit = ((src[0] + src[cls]) + src[2 * cls]) + src[3 * cls];
  int my_idx;
  float my_w;
  topk_lane(logit, b_lane, lane, E, k, scale, topk_scratch[wave], my_idx, my_w);
  if (lane < k) {
    idx_out[(size_t)t * k + lane] = my_idx;
    w_out[(size_t)t * k + lane] = my_w;
  }
}

int router_small_plog_floats(int T) { return 4 * ceil_div(T, 16) * 16 * kMaxExperts; }

hipError_t launch_router_small(const RouterArgs& a, float* plog, hipStream_t stream) {
  const int G = ceil_div(a.T, 16);
  const int Tp = G * 16;
  router_partial_kernel<20><<<dim3(G, 4, 4), 64, 0, stream>>>(a.x, a.wr, a.T, a.d, a.E, plog, Tp);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  router_topk_kernel<<<ceil_div(a.T, 4), 256, 0, stream>>>(plog, Tp, a.bias, a.T, a.E, a.k, a.scale,
                                                          a.idx, a.w);
  return hipGetLastError();
}

// ---- large T: residue-class slices of the router weight kept in LDS --------
//
// Block (r, c) handles k-step residue class r (steps s = r, r + 4, ...) for a
// contiguous range of 64-token rounds.  It first copies that class's slice of
// the router weight (all E <= 64 experts, 64 bytes per step per expert) into
// LDS with direct loads, then each wave streams 16 tokens' x per round: one
// 16-byte x load per step, the four expert-block operands from LDS.  Every x
// element is read once; the router weight once per block.  The MFMA chain of
// each (token, expert) runs over the class's steps in increasing order -- the
// same chain as the other router kernels -- and is stored as a class partial;
// router_select_kernel adds the four partials in class order.
constexpr int kBigRouterMaxClassSteps = 32;  // d <= 4096

constexpr int kClassThreads = 1024;  // 16 waves, 16 tokens each: 256-token rounds

__global__ __launch_bounds__(kClassThreads) void router_class_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr, int T, int d, int E,
    float* __restrict__ plog /* [4][Tp][64] */, int Tp, int rounds_per_block) {
  extern __shared__ __attribute__((aligned(1024))) char wslice[];  // [class steps][64][64 B]
  constexpr int kWaves = kClassThreads / 64;
  const int rc = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int steps = d / 32;
  const int csteps = (steps - rc + 3) / 4;  // steps of this class

  // Stage: LDS block (step i, expert block eb) = experts eb*16 .. +15, 64 B each;
  // lane l writes slot l: expert eb*16 + l/4, 16-byte piece l%4.
  for (int blk = wave; blk < csteps * 4; blk += kWaves) {
    const int i = blk >> 2, eb = blk & 3;
    const int e = min(eb * 16 + (lane >> 2), E - 1);
    const int s = rc + 4 * i;
    const char* src = reinterpret_cast<const char*>(wr + (size_t)e * d + s * 32) + (lane & 3) * 16;
    __builtin_amdgcn_global_load_lds((const void*)src,
                                     (__attribute__((address_space(3))) void*)(wslice + blk * 1024), 16, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int round0 = blockIdx.x * rounds_per_block;
  for (int rd = round0; rd < round0 + rounds_per_block; ++rd) {
    if (rd * 256 >= T) break;
    const int t0 = rd * 256 + wave * 16;
    const bf16_t* xrow = x + (size_t)min(t0 + r16, T - 1) * d + rc * 32 + q * 8;
    f32x4 acc[4];
#pragma unroll
    for (int eb = 0; eb < 4; ++eb) acc[eb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // x loads in batches of 16 steps, each batch issued before its MFMAs.
    for (int u0 = 0; u0 < csteps; u0 += 16) {
      Frag16 a[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) a[u].u = load16(xrow + (size_t)min(u0 + u, csteps - 1) * 128);
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const bool live = u0 + u < csteps;
        const int i = min(u0 + u, csteps - 1);
        Frag16 av;
        av.u = live ? a[u].u : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int eb = 0; eb < 4; ++eb) {
          Frag16 b;
          b.u = load16(wslice + i * 4096 + (eb * 16 + r16) * 64 + q * 16);
          acc[eb] = mfma16x16x32(av.h, b.h, acc[eb]);
        }
      }
    }
#pragma unroll
    for (int eb = 0; eb < 4; ++eb)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        plog[((size_t)rc * Tp + t0 + q * 4 + v) * kMaxExperts + eb * 16 + r16] = acc[eb][v];
  }
}

// One lane per token: adds the four class partials in class order, sigmoid,
// bias for selection, and keeps the k best by insertion over experts 0..E-1
// (a later expert displaces an entry only with a strictly larger score, so
// ties keep the lower index first).  Same selection, order and weight bits as
// topk_lane.  Also writes each block's per-expert pair count (the dispatch
// histogram; a block covers 256 tokens).
__global__ __launch_bounds__(256) void router_select_kernel(
    const float* __restrict__ plog, int Tp, const float* __restrict__ bias, int T, int E, int k,
    float scale, int32_t* __restrict__ idx_out, float* __restrict__ w_out,
    int32_t* __restrict__ chunk_counts) {
  __shared__ int hist[kMaxExperts];
  if (threadIdx.x < kMaxExperts) hist[threadIdx.x] = 0;
  __syncthreads();
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int tc = min(t, T - 1);
  const size_t cls = (size_t)Tp * kMaxExperts;
  float bv[kMaxTopK], bs[kMaxTopK];
  int bi[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    bv[j] = -__builtin_inff();
    bs[j] = 0.f;
    bi[j] = 0;
  }
  const float* row = plog + (size_t)tc * kMaxExperts;
  // Experts in groups of 16 (four 16-byte loads per class); the next group's
  // loads are in flight while the current group is inserted.
  f32x4 buf[2][4][4];
  auto load_group = [&](f32x4 (&g)[4][4], int e0) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        g[c][m] = *reinterpret_cast<const f32x4*>(row + c * cls + min(e0 + 4 * m, kMaxExperts - 4));
  };
  auto insert_group = [&](const f32x4 (&g)[4][4], int e0) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int e = e0 + m;
      if (e >= E) break;
      const float logit = ((g[0][m >> 2][m & 3] + g[1][m >> 2][m & 3]) + g[2][m >> 2][m & 3]) +
                          g[3][m >> 2][m & 3];
      const float sc = sigmoidf_fast(logit);
      float cv = sc + (bias != nullptr ? bias[e] : 0.f);
      float cs = sc;
      int ci = e;
      // Insert at the first slot the candidate beats; everything from there
      // on shifts down one slot (the carried entry always ranks ahead of the
      // ones after it, so once moving it takes every later slot).
      bool moving = false;
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        if (j < k && (moving || cv > bv[j])) {
          const float tv = bv[j], ts = bs[j];
          const int ti = bi[j];
          bv[j] = cv; bs[j] = cs; bi[j] = ci;
          cv = tv; cs = ts; ci = ti;
          moving = true;
        }
      }
    }
  };
  load_group(buf[0], 0);
  for (int e0 = 0; e0 < E; e0 += 32) {
    load_group(buf[1], e0 + 16);
    insert_group(buf[0], e0);
    if (e0 + 32 < E) load_group(buf[0], e0 + 32);
    if (e0 + 16 < E) insert_group(buf[1], e0 + 16);
  }
  float ssum = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (j < k) ssum += bs[j];
  if (t < T) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        const int e = min(max(bi[j], 0), E - 1);
        idx_out[(size_t)t * k + j] = e;
        w_out[(size_t)t * k + j] = scale * bs[j] / ssum;
        if (chunk_counts != nullptr) atomicAdd(&hist[e], 1);
      }
    }
  }
  if (chunk_counts != nullptr) {
    __syncthreads();
    if (threadIdx.x < E) chunk_counts[(size_t)blockIdx.x * E + threadIdx.x] = hist[threadIdx.x];
  }
}

int router_big_supported(int d) { return (d / 32 + 3) / 4 <= kBigRouterMaxClassSteps; }
int router_big_plog_floats(int T) { return 4 * ceil_div(T, 256) * 256 * kMaxExperts; }

hipError_t launch_router_big(const RouterArgs& a, float* plog, hipStream_t stream) {
  const int Tp = ceil_div(a.T, 256) * 256;
  const int rounds = ceil_div(a.T, 256);
  const int rounds_per_block = ceil_div(rounds, 64);
  const int blocks = ceil_div(rounds, rounds_per_block);
  const int csteps = (a.d / 32 + 3) / 4;
  const size_t lds = (size_t)csteps * 4 * 1024;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute((const void*)router_class_kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         kBigRouterMaxClassSteps * 4 * 1024);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  router_class_kernel<<<dim3(blocks, 4), kClassThreads, lds, stream>>>(a.x, a.wr, a.T, a.d, a.E,
                                                                       plog, Tp, rounds_per_block);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  router_select_kernel<<<ceil_div(a.T, 256), 256, 0, stream>>>(plog, Tp, a.bias, a.T, a.E, a.k,
                                                              a.scale, a.idx, a.w, a.chunk_counts);
  return hipGetLastError();
}

}  // namespace mova
