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

__device__ __forceinline__ uint32_t order_key(float sel) {
  sel = (sel == 0.f) ? 0.f : sel;  // -0 and +0 rank as equal, as in a float compare
  const uint32_t u = __float_as_uint(sel);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Router in two kernels, so that even a few tokens spread the router weight
// over many CUs.
//
// ffn_logits_kernel: one wave per (16 tokens, 16 or 64 experts, residue
// class c of the 32-wide k steps mod 4); class c runs steps c, c + 4, c + 8, ... as one
// MFMA chain in increasing order (token fragments and router rows read
// straight from cache) and writes plog[c][t][e].
//
// ffn_topk_kernel: one workgroup per 16 tokens (the dispatch chunk), one
// wave per token.  Logits are the four class sums added in class order,
// ((c0 + c1) + c2) + c3.  Lane l holds experts l and l + 64; each of the k rounds takes the
// wave-wide maximum of a 64-bit key (selection score's bits mapped to an
// order-keeping unsigned integer, then 127 - expert, so equal scores rank
// the lower expert first) and drops the winner.
// Weights: scale * s_j / (sum of the k chosen sigmoid scores, added in rank
// order).  The workgroup's per-expert pair counts go to counts[blockIdx.x, :]
// for the dispatch.

size_t ffn_router_plog_floats(int T) {
  return (size_t)4 * ceil_div(T, kFfnTokens) * kFfnTokens * kMaxDispatchExperts;
}

// TPW: expert tiles per wave (sharing the token fragments); 1 for few
// tokens, where the number of waves matters more than the loads they share.
template <int TPW>
__global__ __launch_bounds__(64) void ffn_logits_kernel(const bf16_t* __restrict__ x,
                                                        const bf16_t* __restrict__ wr, int T, int d,
                                                        int E, float* __restrict__ plog) {
  const int lane = threadIdx.x;
  const int q = lane >> 4, r16 = lane & 15;
  const int tb = blockIdx.x, c0 = blockIdx.y * TPW, cls = blockIdx.z;
  const int Tp = gridDim.x * kFfnTokens;
  const bf16_t* xr = x + (size_t)min(tb * kFfnTokens + r16, T - 1) * d + q * 8;
  const bf16_t* br[TPW];
#pragma unroll
  for (int c = 0; c < TPW; ++c) br[c] = wr + (size_t)min((c0 + c) * 16 + r16, E - 1) * d + q * 8;
  const int nsteps = d / 32;
  f32x4 acc[TPW];
#pragma unroll
  for (int c = 0; c < TPW; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  int s = cls;
  for (; s + 12 < nsteps; s += 16) {
    Frag16 a[4], b[4][TPW];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u].u = load16(xr + (s + 4 * u) * 32);
#pragma unroll
      for (int c = 0; c < TPW; ++c) b[u][c].u = load16(br[c] + (s + 4 * u) * 32);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < TPW; ++c) acc[c] = mfma16x16x32(a[u].h, b[u][c].h, acc[c]);
  }
  for (; s < nsteps; s += 4) {
    Frag16 a, b[TPW];
    a.u = load16(xr + s * 32);
#pragma unroll
    for (int c = 0; c < TPW; ++c) b[c].u = load16(br[c] + s * 32);
#pragma unroll
    for (int c = 0; c < TPW; ++c) acc[c] = mfma16x16x32(a.h, b[c].h, acc[c]);
  }
#pragma unroll
  for (int c = 0; c < TPW; ++c)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      plog[((size_t)cls * Tp + tb * kFfnTokens + q * 4 + v) * kMaxDispatchExperts + (c0 + c) * 16 + r16] =
          acc[c][v];
}

// Wave-wide maximum of a 64-bit key (h, l), returned in every lane: row
// rotations by 1, 2, 4 and 8 lanes leave each row of 16 lanes with its row's
// maximum, two row broadcasts carry the maximum into lane 63, which is then
// read by all lanes.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ void dpp_key_max(uint32_t& h, uint32_t& l) {
  const uint32_t ph = (uint32_t)__builtin_amdgcn_update_dpp((int)h, (int)h, kCtrl, kRowMask, 0xF, false);
  const uint32_t pl = (uint32_t)__builtin_amdgcn_update_dpp((int)l, (int)l, kCtrl, kRowMask, 0xF, false);
  const bool gt = ph > h || (ph == h && pl > l);
  h = gt ? ph : h;
  l = gt ? pl : l;
}

__device__ __forceinline__ void wave_key_max(uint32_t& h, uint32_t& l) {
  dpp_key_max<0x121, 0xF>(h, l);  // row_ror:1
  dpp_key_max<0x122, 0xF>(h, l);  // row_ror:2
  dpp_key_max<0x124, 0xF>(h, l);  // row_ror:4
  dpp_key_max<0x128, 0xF>(h, l);  // row_ror:8
  dpp_key_max<0x142, 0xA>(h, l);  // row_bcast:15 into rows 1 and 3
  dpp_key_max<0x143, 0xC>(h, l);  // row_bcast:31 into rows 2 and 3
  h = (uint32_t)__builtin_amdgcn_readlane((int)h, 63);
  l = (uint32_t)__builtin_amdgcn_readlane((int)l, 63);
}

constexpr int kTopkNT = 1;                                  // tokens per wave
constexpr int kTopkThreads = 64 * kFfnTokens / kTopkNT;     // one chunk per workgroup

__global__ __launch_bounds__(kTopkThreads) void ffn_topk_kernel(const float* __restrict__ plog,
                                                       const float* __restrict__ bias, int T, int E,
                                                       int k, float scale,
                                                       int32_t* __restrict__ idx_out,
                                                       float* __restrict__ w_out,
                                                       int32_t* __restrict__ counts) {
  constexpr int NT = kTopkNT;
  __shared__ int hist[kMaxDispatchExperts];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int tw = blockIdx.x * kFfnTokens + wave * NT;  // the wave's first token
  const size_t cs = (size_t)gridDim.x * kFfnTokens * kMaxDispatchExperts;  // one class plane
  if (tid < kMaxDispatchExperts) hist[tid] = 0;
  __syncthreads();
  const float b0 = (bias != nullptr && lane < E) ? bias[lane] : 0.f;
  const float b1 = (bias != nullptr && lane + 64 < E) ? bias[lane + 64] : 0.f;
  float s0[NT], s1[NT], ssum[NT], my_s[NT];
  uint32_t h0[NT], l0[NT], h1[NT], l1[NT];
  int my_e[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const float* p = plog + (size_t)min(tw + i, T - 1) * kMaxDispatchExperts + lane;
    s0[i] = sigmoidf_fast(((p[0] + p[cs]) + p[2 * cs]) + p[3 * cs]);
    s1[i] = sigmoidf_fast(((p[64] + p[cs + 64]) + p[2 * cs + 64]) + p[3 * cs + 64]);
    h0[i] = l0[i] = h1[i] = l1[i] = 0u;
    if (lane < E) {
      h0[i] = order_key(s0[i] + b0);
      l0[i] = 127u - (uint32_t)lane;
    }
    if (lane + 64 < E) {
      h1[i] = order_key(s1[i] + b1);
      l1[i] = 63u - (uint32_t)lane;
    }
    ssum[i] = 0.f;
    my_s[i] = 0.f;
    my_e[i] = 0;
  }
  for (int r = 0; r < k; ++r) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const bool first = h0[i] > h1[i] || (h0[i] == h1[i] && l0[i] > l1[i]);
      uint32_t mh = first ? h0[i] : h1[i], ml = first ? l0[i] : l1[i];
      wave_key_max(mh, ml);
      const int e = 127 - (int)(ml & 127u);
      // The owner drops the winner; every lane reads its score.
      if (e == lane) h0[i] = l0[i] = 0u;
      if (e == lane + 64) h1[i] = l1[i] = 0u;
      const float sv = e < 64 ? s0[i] : s1[i];  // e is wave-uniform
      const float se = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv), e & 63));
      ssum[i] += se;
      if (lane == r) {
        my_e[i] = e;
        my_s[i] = se;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int t = tw + i;
    if (t < T && lane < k) {
      // Clamped so that even non-finite scores (undefined selection) cannot
      // hand an out-of-range expert to the kernels that follow.
      const int e = min(max(my_e[i], 0), E - 1);
      idx_out[(size_t)t * k + lane] = e;
      w_out[(size_t)t * k + lane] = scale * my_s[i] / ssum[i];
      atomicAdd(&hist[e], 1);
    }
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
  const int tiles = ceil_div(a.E, 16);
  if (a.T >= 1024)
    ffn_logits_kernel<4><<<dim3(tb, ceil_div(tiles, 4), 4), 64, 0, stream>>>(a.x, a.wr, a.T, a.d,
                                                                           a.E, plog);
  else
    ffn_logits_kernel<1><<<dim3(tb, tiles, 4), 64, 0, stream>>>(a.x, a.wr, a.T, a.d, a.E, plog);
  hipError_t err = hipGetLastError();
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
