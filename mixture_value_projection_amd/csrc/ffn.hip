// FFN mixture of experts on the same dispatch and tiled-GEMM machinery as
// the value experts: the sparse FFN that the model runs beside its routed
// value projection, 100 experts with top-8 routing plus one shared expert
// (the thevalue.engineering page on the MoVA architecture, section "Dual
// sparsity": 100 FFN experts top-8+1 next to 64 value experts top-4).  The
// pages give no FFN expert shape or routing function; the library takes
// SwiGLU experts of any intermediate width (the caller's argument) and routes
// them with the value router's function (sigmoid scores, bias for
// selection, top-k renormalised and scaled by the caller's scale).
//
// This file holds the FFN router (E up to 128, one lane per two experts) and
// the gate/up weight interleaving; the experts run as tiled-GEMM modes
// (kGemmRoutedSwiGLU, kGemmRoutedLinear, kGemmDenseSwiGLU, kGemmDenseF16).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace mova {

constexpr int kFfnTokens = 16;  // tokens per router workgroup (= dispatch chunk)

int ffn_router_chunk_tokens() { return kFfnTokens; }

// 64-bit wave maximum by butterfly shuffles (every lane ends with the max).
__device__ __forceinline__ void key_max_wave(uint32_t& h, uint32_t& l) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const uint32_t ph = (uint32_t)__shfl_xor((int)h, m);
    const uint32_t pl = (uint32_t)__shfl_xor((int)l, m);
    const bool gt = ph > h || (ph == h && pl > l);
    h = gt ? ph : h;
    l = gt ? pl : l;
  }
}

__device__ __forceinline__ uint32_t order_key(float sel) {
  sel = (sel == 0.f) ? 0.f : sel;  // -0 and +0 rank as equal, as in a float compare
  const uint32_t u = __float_as_uint(sel);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One workgroup of 4 waves per 16 tokens.  Logits: wave w computes expert
// column tiles 2w and 2w + 1 (16 experts each) for the 16 tokens as one MFMA
// chain over the 32-wide k steps in order (token fragments and router rows
// read straight from cache).  Selection: wave w takes tokens 4w .. 4w + 3;
// lane l holds experts l and l + 64; each of the k rounds takes the wave-wide
// maximum of a 64-bit key (selection score's bits mapped to an order-keeping
// unsigned integer, then 127 - expert, so equal scores rank the lower expert
// first) and drops the winner.  Weights: scale * s_j / (sum of the k chosen
// sigmoid scores, added in rank order).  The workgroup's per-expert pair
// counts go to counts[blockIdx.x, :] for the dispatch.
__global__ __launch_bounds__(256) void ffn_router_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr, const float* __restrict__ bias,
    int T, int d, int E, int k, float scale, int32_t* __restrict__ idx_out,
    float* __restrict__ w_out, int32_t* __restrict__ counts) {
  __shared__ float lg[kFfnTokens][kMaxDispatchExperts + 1];
  __shared__ int hist[kMaxDispatchExperts];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int t0 = blockIdx.x * kFfnTokens;
  if (tid < kMaxDispatchExperts) hist[tid] = 0;

  const bf16_t* xr = x + (size_t)min(t0 + r16, T - 1) * d + q * 8;
  const bf16_t* br[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) br[c] = wr + (size_t)min((2 * wave + c) * 16 + r16, E - 1) * d + q * 8;
  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  const bool live = 2 * wave * 16 < E;  // wave-uniform: some expert in its tiles
  if (live) {
    const int nsteps = d / 32;
    int s = 0;
    for (; s + 4 <= nsteps; s += 4) {
      Frag16 a[4], b0[4], b1[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u].u = load16(xr + (s + u) * 32);
        b0[u].u = load16(br[0] + (s + u) * 32);
        b1[u].u = load16(br[1] + (s + u) * 32);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc[0] = mfma16x16x32(a[u].h, b0[u].h, acc[0]);
        acc[1] = mfma16x16x32(a[u].h, b1[u].h, acc[1]);
      }
    }
    for (; s < nsteps; ++s) {
      Frag16 a, b0, b1;
      a.u = load16(xr + s * 32);
      b0.u = load16(br[0] + s * 32);
      b1.u = load16(br[1] + s * 32);
      acc[0] = mfma16x16x32(a.h, b0.h, acc[0]);
      acc[1] = mfma16x16x32(a.h, b1.h, acc[1]);
    }
  }
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int v = 0; v < 4; ++v) lg[q * 4 + v][(2 * wave + c) * 16 + r16] = acc[c][v];
  __syncthreads();

  const float b0 = (bias != nullptr && lane < E) ? bias[lane] : 0.f;
  const float b1 = (bias != nullptr && lane + 64 < E) ? bias[lane + 64] : 0.f;
  for (int i = 0; i < 4; ++i) {
    const int tl = wave * 4 + i;
    const int t = t0 + tl;
    if (t >= T) break;  // wave-uniform
    const float s0 = sigmoidf_fast(lg[tl][lane]);
    const float s1 = sigmoidf_fast(lg[tl][lane + 64]);
    uint32_t h0 = 0u, l0 = 0u, h1 = 0u, l1 = 0u;
    if (lane < E) {
      h0 = order_key(s0 + b0);
      l0 = 127u - (uint32_t)lane;
    }
    if (lane + 64 < E) {
      h1 = order_key(s1 + b1);
      l1 = 63u - (uint32_t)lane;
    }
    float ssum = 0.f, my_s = 0.f;
    int my_e = 0;
    for (int r = 0; r < k; ++r) {
      const bool first = h0 > h1 || (h0 == h1 && l0 > l1);
      uint32_t mh = first ? h0 : h1, ml = first ? l0 : l1;
      key_max_wave(mh, ml);
      const int e = 127 - (int)ml;
      // The owner drops the winner; every lane learns its score.
      if (e == lane) { h0 = 0u; l0 = 0u; }
      if (e == lane + 64) { h1 = 0u; l1 = 0u; }
      const float se = __shfl(e < 64 ? s0 : s1, e & 63);
      ssum += se;
      if (lane == r) {
        my_e = e;
        my_s = se;
      }
    }
    if (lane < k) {
      idx_out[(size_t)t * k + lane] = my_e;
      w_out[(size_t)t * k + lane] = scale * my_s / ssum;
      atomicAdd(&hist[my_e], 1);
    }
  }
  __syncthreads();
  if (counts != nullptr && tid < E) counts[(size_t)blockIdx.x * E + tid] = hist[tid];
}

hipError_t launch_ffn_router(const RouterArgs& a, hipStream_t stream) {
  const int blocks = ceil_div(a.T, kFfnTokens);
  ffn_router_kernel<<<blocks, 256, 0, stream>>>(a.x, a.wr, a.bias, a.T, a.d, a.E, a.k, a.scale,
                                                a.idx, a.w, a.chunk_counts);
  return hipGetLastError();
}

// gate_up[e, 32 b + j] = gate[e, 16 b + j] and gate_up[e, 32 b + 16 + j] =
// up[e, 16 b + j] (j < 16): the row order the SwiGLU GEMM modes read.  One
// thread per 16-byte chunk of a destination row.
__global__ __launch_bounds__(256) void ffn_pack_gate_up_kernel(const bf16_t* __restrict__ gate,
                                                               const bf16_t* __restrict__ up,
                                                               bf16_t* __restrict__ dst, int E,
                                                               int inter, int d) {
  const int cpr = d / 8;  // 16-byte chunks per row
  const long long total = (long long)E * 2 * inter * cpr;
  for (long long v = blockIdx.x * 256ll + threadIdx.x; v < total; v += (long long)gridDim.x * 256) {
    const long long row = v / cpr;
    const int c = (int)(v % cpr);
    const int e = (int)(row / (2 * inter));
    const int rr = (int)(row % (2 * inter));
    const int blk = rr / 32, j = rr % 32;
    const bf16_t* src = (j < 16 ? gate : up) + ((size_t)e * inter + blk * 16 + (j & 15)) * d;
    store16(dst + (size_t)row * d + c * 8, load16(src + c * 8));
  }
}

hipError_t launch_ffn_pack_gate_up(const __bf16* gate, const __bf16* up, __bf16* dst, int E,
                                   int inter, int d, hipStream_t stream) {
  const long long total = (long long)E * 2 * inter * (d / 8);
  const long long blocks = std::min<long long>((total + 255) / 256, 256ll * 16);
  ffn_pack_gate_up_kernel<<<dim3((unsigned)blocks), 256, 0, stream>>>(gate, up, dst, E, inter, d);
  return hipGetLastError();
}

}  // namespace mova
