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
#include "topk.h"

namespace mova {

constexpr int kFfnTokens = 16;  // tokens per router workgroup (= dispatch chunk)

int ffn_router_chunk_tokens() { return kFfnTokens; }

// Router in two kernels below kFfnLdsMinT tokens, so that even a few tokens
// spread the router weight over many CUs: the value router's partial-logit
// kernel (launch_router_partial_wide: one wave per 16 tokens, 16 experts and
// residue class, all loads in flight), then ffn_topk_kernel.
//
// ffn_topk_kernel: one workgroup per 16 tokens (the dispatch chunk), one
// wave per token.  Logits are the four class sums added in class order,
// ((c0 + c1) + c2) + c3; lane l holds experts l and l + 64, and
// topk_tokens2 selects (the LDS-staged router's own selection, so the two
// give the same bits).  The workgroup's per-expert pair counts go to
// counts[blockIdx.x, :] for the dispatch.

size_t ffn_router_plog_floats(int T) {
  return (size_t)4 * ceil_div(T, kFfnTokens) * kFfnTokens * kMaxDispatchExperts;
}

constexpr int kTopkThreads = 64 * kFfnTokens;  // one token per wave

__global__ __launch_bounds__(kTopkThreads) void ffn_topk_kernel(const float* __restrict__ plog,
                                                       const float* __restrict__ bias, int T, int E,
                                                       int k, float scale,
                                                       int32_t* __restrict__ idx_out,
                                                       float* __restrict__ w_out,
                                                       int32_t* __restrict__ counts) {
  __shared__ int hist[kMaxDispatchExperts];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x * kFfnTokens + wave;
  const size_t cs = (size_t)gridDim.x * kFfnTokens * kMaxDispatchExperts;  // one class plane
  if (tid < kMaxDispatchExperts) hist[tid] = 0;
  __syncthreads();
  const float b0 = (bias != nullptr && lane < E) ? bias[lane] : 0.f;
  const float b1 = (bias != nullptr && lane + 64 < E) ? bias[lane + 64] : 0.f;
  const float* p = plog + (size_t)min(t, T - 1) * kMaxDispatchExperts + lane;
  const float lg0[1] = {((p[0] + p[cs]) + p[2 * cs]) + p[3 * cs]};
  const float lg1[1] = {((p[64] + p[cs + 64]) + p[2 * cs + 64]) + p[3 * cs + 64]};
  int my_idx[1];
  float my_w[1];
  topk_tokens2<1>(lg0, lg1, b0, b1, lane, E, k, scale, my_idx, my_w);
  if (t < T && lane < k) {
    idx_out[(size_t)t * k + lane] = my_idx[0];
    w_out[(size_t)t * k + lane] = my_w[0];
    atomicAdd(&hist[my_idx[0]], 1);
  }
  __syncthreads();
  if (counts != nullptr && tid < E) counts[(size_t)blockIdx.x * E + tid] = hist[tid];
}

// Above kFfnLdsMinT tokens the LDS-staged router (router.hip) takes the call:
// the same chains, selection order and weights, hence the same bits, with its
// operands loaded as whole row segments instead of MFMA fragments.
constexpr int kFfnLdsMinT = 1024;

hipError_t launch_ffn_router(const RouterArgs& a, float* plog, hipStream_t stream) {
  if (a.T >= kFfnLdsMinT) return launch_router_lds_wide(a, stream);
  const int tb = ceil_div(a.T, kFfnTokens);
  hipError_t err = launch_router_partial_wide(a, plog, stream);
  if (err != hipSuccess) return err;
  ffn_topk_kernel<<<tb, kTopkThreads, 0, stream>>>(plog, a.bias, a.T, a.E, a.k, a.scale, a.idx, a.w,
                                          a.chunk_counts);
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
