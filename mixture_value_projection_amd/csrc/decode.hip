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
// per 32-wide k step.  The k loop runs in batches of kUnroll steps: a batch's
// weight loads are issued first, then the token rows of the next batch are
// copied into LDS (double-buffered, 16-byte chunks XOR-swizzled by row), then
// the batch's MFMAs read their token operand from LDS.  Tokens are handled 16
// at a time (one MFMA row group); an expert with more than 16 tokens takes
// several passes over its weights.  The epilogue writes w * SiLU(z) to the
// pair's partial row, like the grouped GEMM; the combine kernel then sums each
// token's k partials in slot order, so both paths give identical bits.  (A
// fused last-arriver combine was measured and rejected: the agent-scope release
// each workgroup needs costs far more than the separate combine launch.)
#include "common.h"
#include "kernels.h"

namespace mova {

constexpr int kSlice = 64;    // columns per workgroup
constexpr int kUnroll = 8;    // k steps per batch
constexpr int kRowBytes = kUnroll * 64;       // one token's k range per batch
constexpr int kChunks = kRowBytes / 16;       // 16-byte chunks per staged row


__device__ __forceinline__ int xs_off(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ (row & 7)) << 4);
}

__global__ __launch_bounds__(256) void decode_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ W,
    const int32_t* __restrict__ idx, const float* __restrict__ topk_w,
    float* __restrict__ partial, int T, int d, int N, int E, int k) {
  __shared__ int plist[kDecodeMaxT];
  __shared__ __attribute__((aligned(16))) char xs[2][16 * kRowBytes];
  __shared__ int count;

  const int slices = N / kSlice;
  const int e = blockIdx.x / slices;
  const int n0 = (blockIdx.x % slices) * kSlice;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int npairs = T * k;

  // Pairs routed to this expert, in pair order (a token picks e at most once).
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

  const int n = n0 + wave * 16 + r16;
  const bf16_t* wrow = W + ((size_t)e * N + n) * d + q * 8;
  const int steps = d / 32;            // even, since d % 64 == 0
  const int nb = ceil_div(steps, kUnroll);
  static_assert(16 * kChunks == 2 * 256, "two 16-byte chunks per thread per batch");

  for (int p0 = 0; p0 < ce; p0 += 16) {
    const bf16_t* src[2];
    int cp_row[2], cp_ch[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * 256;
      cp_row[i] = c / kChunks;
      cp_ch[i] = c % kChunks;
      const int pair = plist[min(p0 + cp_row[i], ce - 1)];
      src[i] = x + (size_t)(pair / k) * d;
    }
    // Copy batch bt of the 16 token rows into xs[buf].  k offsets past the end
    // of the row (d not a multiple of the batch) read a clamped address and
    // store zeros, so those steps contribute nothing.
    auto stage = [&](int bt, int buf) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int kk = bt * kUnroll * 32 + cp_ch[i] * 8;
        u32x4 v = load16(src[i] + min(kk, d - 8));
        if (kk >= d) v = u32x4{0u, 0u, 0u, 0u};
        store16(&xs[buf][xs_off(cp_row[i], cp_ch[i])], v);
      }
    };
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    stage(0, 0);
    __syncthreads();
    for (int bt = 0; bt < nb; ++bt) {
      const int buf = bt & 1;
      Frag16 b[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) b[u].u = load16(wrow + min(bt * kUnroll + u, steps - 1) * 32);
      if (bt + 1 < nb) stage(bt + 1, buf ^ 1);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        Frag16 a;
        a.u = load16(&xs[buf][xs_off(r16, u * 4 + q)]);
        acc = mfma16x16x32(a.h, b[u].h, acc);
      }
      __syncthreads();
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = p0 + q * 4 + v;
      if (r < ce) {
        const int pair = plist[r];
        partial[(size_t)pair * N + n] = topk_w[pair] * siluf(acc[v]);
      }
    }
  }

}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.E * (a.N / kSlice));
  decode_kernel<<<grid, 256, 0, stream>>>(a.x, a.W, a.idx, a.topk_w, a.partial, a.T, a.d, a.N,
                                          a.E, a.k);
  return hipGetLastError();
}

}  // namespace mova
