// Decode path: a weight-streaming kernel for small token counts.
//
// With few tokens per expert the layer is bound by reading the touched
// experts' weights (page "MoVA: routing the value vectors ...", section "So
// what does it cost?": decode is memory-bound and reads four experts per
// token).  Each workgroup owns one (expert, 64-column slice) and streams that
// slice's 64 x d weights exactly once from HBM; the tokens that chose the
// expert (at most a few dozen) ride along as the MFMA's other operand, read
// from cache.  No dispatch kernel is needed: the workgroup finds its tokens by
// scanning the [T, k] routing with wave ballots, which also keeps them in
// pair order.
//
// Each wave owns 16 of the slice's columns; its 64 lanes read 16 rows x 64 B
// per 32-wide k step (whole 128 B lines over two steps).  The fused epilogue
// writes w * SiLU(z) to the pair's partial row, like the grouped GEMM.
#include "common.h"
#include "kernels.h"

namespace mova {

constexpr int kSlice = 64;   // columns per workgroup
constexpr int kGroups = 4;   // 16-token MFMA groups per pass (64 tokens)
constexpr int kUnroll = 8;   // k steps whose weight loads are in flight together

// One pass over the slice's weights for NG groups of 16 tokens starting at
// plist[p0].  NG is a template argument so that every MFMA in the k loop runs
// unconditionally: accumulators updated under data-dependent branches were
// compiled into AGPR<->VGPR copies at the loop head that read MFMA results too
// early.
template <int NG>
__device__ __forceinline__ void decode_pass(const bf16_t* __restrict__ x, const bf16_t* wrow,
                                            const int* plist, int p0, int ce,
                                            const float* __restrict__ topk_w,
                                            float* __restrict__ partial, int d, int N, int k,
                                            int n, int q, int r16) {
  const bf16_t* xrow[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int r = min(p0 + g * 16 + r16, ce - 1);
    xrow[g] = x + (size_t)(plist[r] / k) * d + q * 8;
  }
  f32x4 acc[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int steps = d / 32;  // even, since d % 64 == 0
  int s = 0;
  for (; s + kUnroll <= steps; s += kUnroll) {
    Frag16 b[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) b[u].u = load16(wrow + (s + u) * 32);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        Frag16 a;
        a.u = load16(xrow[g] + (s + u) * 32);
        acc[g] = mfma16x16x32(a.h, b[u].h, acc[g]);
      }
    }
  }
  for (; s < steps; s += 2) {
    Frag16 b0, b1;
    b0.u = load16(wrow + s * 32);
    b1.u = load16(wrow + (s + 1) * 32);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      Frag16 a0, a1;
      a0.u = load16(xrow[g] + s * 32);
      a1.u = load16(xrow[g] + (s + 1) * 32);
      acc[g] = mfma16x16x32(a0.h, b0.h, acc[g]);
      acc[g] = mfma16x16x32(a1.h, b1.h, acc[g]);
    }
  }

#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = p0 + g * 16 + q * 4 + v;
      if (r < ce) {
        const int pair = plist[r];
        partial[(size_t)pair * N + n] = topk_w[pair] * siluf(acc[g][v]);
      }
    }
  }
}

__global__ __launch_bounds__(256) void decode_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ W,
    const int32_t* __restrict__ idx, const float* __restrict__ topk_w,
    float* __restrict__ partial, int T, int d, int N, int E, int k) {
  __shared__ int plist[kDecodeMaxPairs];
  __shared__ int count;

  const int slices = N / kSlice;
  const int e = blockIdx.x / slices;
  const int n0 = (blockIdx.x % slices) * kSlice;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int npairs = T * k;

  if (wave == 0) {
    int c = 0;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = 0; base < npairs; base += 64) {
      const int p = base + lane;
      const bool hit = p < npairs && idx[p] == e;
      const uint64_t m = __ballot(hit);
      if (hit) plist[c + __popcll(m & lt_mask)] = p;
      c += __popcll(m);
    }
    if (lane == 0) count = c;
  }
  __syncthreads();
  const int ce = count;
  if (ce == 0) return;

  const int n = n0 + wave * 16 + r16;
  const bf16_t* wrow = W + ((size_t)e * N + n) * d + q * 8;
  for (int p0 = 0; p0 < ce; p0 += kGroups * 16) {
    const int ng = min(kGroups, ceil_div(ce - p0, 16));
    if (ng == 1)
      decode_pass<1>(x, wrow, plist, p0, ce, topk_w, partial, d, N, k, n, q, r16);
    else if (ng == 2)
      decode_pass<2>(x, wrow, plist, p0, ce, topk_w, partial, d, N, k, n, q, r16);
    else if (ng == 3)
      decode_pass<3>(x, wrow, plist, p0, ce, topk_w, partial, d, N, k, n, q, r16);
    else
      decode_pass<4>(x, wrow, plist, p0, ce, topk_w, partial, d, N, k, n, q, r16);
  }
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.E * (a.N / kSlice));
  decode_kernel<<<grid, 256, 0, stream>>>(a.x, a.W, a.idx, a.topk_w, a.partial, a.T, a.d, a.N,
                                          a.E, a.k);
  return hipGetLastError();
}

}  // namespace mova
