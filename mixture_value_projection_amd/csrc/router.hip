// Router: logits = x Wr^T (fp32 accumulation of bf16 products on MFMA),
// sigmoid scores, bias added for selection, wave-wide top-k with the lower
// expert index winning ties, renormalised weights times `scale`.
//
// Method: page "MoVA: routing the value vectors, and why the KV cache does not
// notice", section "Where the routing happens" (weight-only router linear map,
// sigmoid scoring, top-4, scaling factor 2.5).
//
// One workgroup = 4 waves handles TM = 16 * TG tokens.  The d-long dot
// products are split into four residue classes of 32-wide k steps
// (step mod 4); wave w owns class w for all of the block's tokens and all 64
// expert columns (TG x 4 MFMA tiles, accumulated in place).  The four partial
// logits meet in LDS and are added in class order, so a token's logits are
// the same bits whichever block shape (or call) processed it.  Top-k then
// runs with one lane per expert (E <= 64).  Optionally each workgroup writes
// how many of its (token, slot) pairs chose each expert -- the per-chunk
// histogram the dispatch step scans.
#include "common.h"
#include "kernels.h"

namespace mova {

template <int TG>
__global__ __launch_bounds__(256) void router_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr, const float* __restrict__ bias,
    int T, int d, int E, int k, float scale,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out, int32_t* __restrict__ chunk_counts) {
  constexpr int TM = 16 * TG;
  __shared__ float part[4][TM][kMaxExperts];
  __shared__ int hist[kMaxExperts];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;  // k-step residue class
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
  const bf16_t* wrow[4];
#pragma unroll
  for (int eb = 0; eb < 4; ++eb) wrow[eb] = wr + (size_t)min(eb * 16 + r16, E - 1) * d + q * 8;

  f32x4 acc[TG][4];
#pragma unroll
  for (int g = 0; g < TG; ++g)
#pragma unroll
    for (int eb = 0; eb < 4; ++eb) acc[g][eb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int steps = d / 32;
  for (int s = wave; s < steps; s += 4) {
    Frag16 a[TG], b[4];
#pragma unroll
    for (int g = 0; g < TG; ++g) a[g].u = load16(xrow[g] + s * 32);
#pragma unroll
    for (int eb = 0; eb < 4; ++eb) b[eb].u = load16(wrow[eb] + s * 32);
#pragma unroll
    for (int g = 0; g < TG; ++g)
#pragma unroll
      for (int eb = 0; eb < 4; ++eb) acc[g][eb] = mfma16x16x32(a[g].h, b[eb].h, acc[g][eb]);
  }

#pragma unroll
  for (int g = 0; g < TG; ++g)
#pragma unroll
    for (int eb = 0; eb < 4; ++eb)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[wave][g * 16 + q * 4 + i][eb * 16 + r16] = acc[g][eb][i];
  __syncthreads();

  // Top-k: wave `wave` takes tile rows wave, wave + 4, ...; lane = expert.
  const float b_lane = (bias != nullptr && lane < E) ? bias[lane] : 0.f;
  for (int r = wave; r < TM; r += 4) {
    const int t = tile_t0 + r;
    if (t >= T) break;
    const float logit = ((part[0][r][lane] + part[1][r][lane]) + part[2][r][lane]) + part[3][r][lane];
    const float sc = sigmoidf_fast(logit);
    float sel = lane < E ? sc + b_lane : -__builtin_inff();
    int my_idx = 0;
    float my_s = 0.f, ssum = 0.f;
    for (int j = 0; j < k; ++j) {
      float bv = sel;
      int bi = lane;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      const float sb = __shfl(sc, bi);
      ssum += sb;
      if (lane == j) {
        my_idx = bi;
        my_s = sb;
      }
      if (lane == bi) sel = -__builtin_inff();
    }
    if (lane < k) {
      idx_out[(size_t)t * k + lane] = my_idx;
      w_out[(size_t)t * k + lane] = scale * my_s / ssum;
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
    router_kernel<4><<<grid, 256, 0, stream>>>(a.x, a.wr, a.bias, a.T, a.d, a.E, a.k, a.scale,
                                                a.idx, a.w, a.chunk_counts);
  } else {
    router_kernel<1><<<grid, 256, 0, stream>>>(a.x, a.wr, a.bias, a.T, a.d, a.E, a.k, a.scale,
                                                a.idx, a.w, a.chunk_counts);
  }
  return hipGetLastError();
}

}  // namespace mova
