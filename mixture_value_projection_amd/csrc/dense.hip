// Dense value projection for few tokens: out = x W_v^T (bf16 in, fp32
// accumulation, bf16 out).
//
// This is the plain GQA value projection of the model's dense layers (page
// "MoVA: routing the value vectors ...", section "So what does it cost?":
// one contiguous [N, d] weight read per layer instead of k scattered expert
// reads).  With up to a few hundred tokens the product is bound by reading
// that weight once, so the kernel spreads the weight over many workgroups by
// splitting k:
//
// * a wave owns 16 columns and one k piece of 4 MFMA steps (128 of d): it
//   loads its 16 x 128 weight block once (four 16-byte loads per lane) and
//   runs every token through it, 16 tokens per MFMA row group, reading the
//   token fragments straight from cache (x is a few hundred KB shared by the
//   whole grid);
// * a workgroup's 4 waves take 4 consecutive k pieces of the same 16 columns
//   and add their results in LDS in wave order;
// * S = ceil(pieces / 4) workgroups cover d; each writes an fp32 partial
//   [S, T, N], and a second kernel adds the S partials in split order and
//   rounds once to bf16.
//
// Every output is a fixed-order sum (MFMA chain inside a piece, then waves,
// then splits), so results are bitwise reproducible and do not depend on T.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace mova {

constexpr int kPieceSteps = 4;  // 32-wide k steps per wave piece
constexpr int kSkinnyWaves = 4;

int dense_skinny_splits(int d) {
  const int pieces = ceil_div(d / 32, kPieceSteps);
  return ceil_div(pieces, kSkinnyWaves);
}

size_t dense_skinny_partial_floats(int T, int d, int N) {
  return (size_t)dense_skinny_splits(d) * T * N;
}

// RGP: MFMA row groups (16 tokens each) per pass; a pass's token fragments
// for the wave's 4 steps are loaded while the previous pass computes.
template <int RGP>
__global__ __launch_bounds__(256) void dense_skinny_kernel(const bf16_t* __restrict__ x,
                                                           const bf16_t* __restrict__ W,
                                                           float* __restrict__ part, int T, int d,
                                                           int N) {
  extern __shared__ float red[];  // [4 waves][rows][16 columns], rows = 16 * row groups
  const int cgroups = N / 16;
  const int cg = blockIdx.x % cgroups;
  const int s = blockIdx.x / cgroups;
  const int n0 = cg * 16;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int nsteps = d / 32;
  const int k0 = (s * kSkinnyWaves + wave) * kPieceSteps;
  const int np = min(max(nsteps - k0, 0), kPieceSteps);  // 0, 2 or 4 (nsteps is even)
  const int rgt = ceil_div(T, 16);
  const int rows = rgt * 16;
  const int passes = ceil_div(rgt, RGP);

  // The wave's weight block: column n0 + r16, k = 32 (k0 + u) + 8 q .. + 7.
  Frag16 b[kPieceSteps];
  const bf16_t* wp = W + (size_t)(n0 + r16) * d + q * 8;
#pragma unroll
  for (int u = 0; u < kPieceSteps; ++u) b[u].u = load16(wp + min(k0 + u, nsteps - 1) * 32);

  auto load_a = [&](Frag16 (&a)[RGP][kPieceSteps], int g) {
#pragma unroll
    for (int rg = 0; rg < RGP; ++rg) {
      const int t = min((g * RGP + rg) * 16 + r16, T - 1);
      const bf16_t* xp = x + (size_t)t * d + q * 8;
#pragma unroll
      for (int u = 0; u < kPieceSteps; ++u) a[rg][u].u = load16(xp + min(k0 + u, nsteps - 1) * 32);
    }
  };
  // MFMA row r16 of row group rg is token (g RGP + rg) 16 + r16; the result
  // lane holds tokens ... + 4 q + v of column n0 + r16.
  auto compute = [&](Frag16 (&a)[RGP][kPieceSteps], int g) {
    f32x4 acc[RGP];
#pragma unroll
    for (int rg = 0; rg < RGP; ++rg) acc[rg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kPieceSteps; ++u)
      if (u < np)
#pragma unroll
        for (int rg = 0; rg < RGP; ++rg) acc[rg] = mfma16x16x32(a[rg][u].h, b[u].h, acc[rg]);
#pragma unroll
    for (int rg = 0; rg < RGP; ++rg) {
      const int gr = g * RGP + rg;
      if (gr < rgt) {
#pragma unroll
        for (int v = 0; v < 4; ++v) red[((size_t)wave * rows + gr * 16 + q * 4 + v) * 16 + r16] = acc[rg][v];
      }
    }
  };
  Frag16 a0[RGP][kPieceSteps], a1[RGP][kPieceSteps];
  load_a(a0, 0);
  for (int g = 0; g < passes; g += 2) {
    if (g + 1 < passes) load_a(a1, g + 1);
    compute(a0, g);
    if (g + 1 < passes) {
      if (g + 2 < passes) load_a(a0, g + 2);
      compute(a1, g + 1);
    }
  }
  __syncthreads();

  // Sum the 4 waves in order and write this split's partial rows (4 columns
  // per thread).
  float* dst = part + (size_t)s * T * N;
  for (int i = tid; i < T * 4; i += 256) {
    const int t = i >> 2, c4 = (i & 3) * 4;
    f32x4 sum;
#pragma unroll
    for (int j = 0; j < 4; ++j) sum[j] = red[((size_t)0 * rows + t) * 16 + c4 + j];
#pragma unroll
    for (int w = 1; w < kSkinnyWaves; ++w)
#pragma unroll
      for (int j = 0; j < 4; ++j) sum[j] += red[((size_t)w * rows + t) * 16 + c4 + j];
    *reinterpret_cast<f32x4*>(dst + (size_t)t * N + n0 + c4) = sum;
  }
}

// out[t, n] = bf16( sum_{s < S} part[s, t, n] ), s in order; 8 columns per
// thread.  kOut selects the output: kDenseOutBf16 as above; kDenseOutF16 the
// same sum rounded to fp16; kDenseOutSwiGLU the SwiGLU of gate / up columns
// interleaved in blocks of 16 (column 32b + j is gate 16b + j, column
// 32b + 16 + j the matching up), out[t, c] = bf16(SiLU(gate_c) * up_c) with
// N / 2 columns.
__device__ __forceinline__ void split_sum8(const float* __restrict__ part, size_t plane, int S,
                                           size_t o, float (&v)[8]) {
  f32x4 lo = *reinterpret_cast<const f32x4*>(part + o);
  f32x4 hi = *reinterpret_cast<const f32x4*>(part + o + 4);
  for (int s = 1; s < S; ++s) {
    const f32x4 l2 = *reinterpret_cast<const f32x4*>(part + s * plane + o);
    const f32x4 h2 = *reinterpret_cast<const f32x4*>(part + s * plane + o + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo[j] += l2[j];
      hi[j] += h2[j];
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] = lo[j];
    v[j + 4] = hi[j];
  }
}

template <int kOut>
__global__ __launch_bounds__(256) void dense_split_reduce_kernel(const float* __restrict__ part,
                                                                 void* __restrict__ out, int T,
                                                                 int N, int S) {
  const int NO = kOut == kDenseOutSwiGLU ? N / 2 : N;  // output columns
  const long long total = (long long)T * NO / 8;
  const size_t plane = (size_t)T * N;
  for (long long v = blockIdx.x * 256ll + threadIdx.x; v < total; v += (long long)gridDim.x * 256) {
    const size_t oo = (size_t)v * 8;  // first output element
    float r[8];
    if constexpr (kOut == kDenseOutSwiGLU) {
      const size_t t = oo / NO;
      const int c = (int)(oo % NO);
      const size_t gcol = (size_t)(c / 16) * 32 + (c % 16);
      float g[8], u[8];
      split_sum8(part, plane, S, t * N + gcol, g);
      split_sum8(part, plane, S, t * N + gcol + 16, u);
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = siluf(g[j]) * u[j];
    } else {
      split_sum8(part, plane, S, oo, r);
    }
    u32x4 packed;
    if constexpr (kOut == kDenseOutF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        packed[i] = (uint32_t)__builtin_bit_cast(uint16_t, (f16_t)r[2 * i]) |
                    ((uint32_t)__builtin_bit_cast(uint16_t, (f16_t)r[2 * i + 1]) << 16);
      store16((f16_t*)out + oo, packed);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        packed[i] = (uint32_t)f32_to_bf16_bits(r[2 * i]) | ((uint32_t)f32_to_bf16_bits(r[2 * i + 1]) << 16);
      store16((bf16_t*)out + oo, packed);
    }
  }
}

hipError_t launch_dense_skinny(const DenseArgs& a, hipStream_t stream) {
  const int S = dense_skinny_splits(a.d);
  const int rgt = ceil_div(a.T, 16);
  const size_t lds = (size_t)kSkinnyWaves * rgt * 16 * 16 * sizeof(float);
  const dim3 grid((unsigned)(S * (a.N / 16)));
  auto kern = rgt >= 3 ? dense_skinny_kernel<4>
                       : (rgt == 2 ? dense_skinny_kernel<2> : dense_skinny_kernel<1>);
  static std::atomic<unsigned long long> attr_done{0};
  hipError_t aerr = once_per_device(attr_done, []() {
    const int max_lds = kSkinnyWaves * kDenseSkinnyMaxT * 16 * (int)sizeof(float);
    for (auto k : {dense_skinny_kernel<1>, dense_skinny_kernel<2>, dense_skinny_kernel<4>}) {
      hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         max_lds);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  });
  if (aerr != hipSuccess) return aerr;
  kern<<<grid, 256, lds, stream>>>(a.x, a.W, a.part, a.T, a.d, a.N);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int NO = a.out_mode == kDenseOutSwiGLU ? a.N / 2 : a.N;
  const long long total = (long long)a.T * NO / 8;
  const long long blocks = std::min<long long>((total + 255) / 256, 256ll * 16);
  const dim3 g((unsigned)blocks);
  if (a.out_mode == kDenseOutSwiGLU)
    dense_split_reduce_kernel<kDenseOutSwiGLU><<<g, 256, 0, stream>>>(a.part, a.out_any, a.T, a.N, S);
  else if (a.out_mode == kDenseOutF16)
    dense_split_reduce_kernel<kDenseOutF16><<<g, 256, 0, stream>>>(a.part, a.out_any, a.T, a.N, S);
  else
    dense_split_reduce_kernel<kDenseOutBf16><<<g, 256, 0, stream>>>(a.part, a.out, a.T, a.N, S);
  return hipGetLastError();
}

}  // namespace mova
