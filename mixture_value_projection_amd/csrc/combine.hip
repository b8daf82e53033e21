// k-way combine: out[t, n] = sum_{i<k} partial[t * k + i, n], the fp16 slot
// partials widened to fp32, summed in slot order i = 0 .. k-1 and rounded once
// to bf16 (nearest even).  The [T, N] result is the [T, n_kv_heads, head_dim]
// value tensor with column n = h * head_dim + j (page "MoVA: routing the
// value vectors ...", section "Where the routing happens": the mixture is
// summed per token and viewed as heads of 128).
//
// Paged variant: the same row is also (or only) stored at row slot[t] of a
// paged value pool [num_blocks, block_size, n_kv_heads, head_dim], whose rows
// are contiguous N-element vectors, so slot s is simply row s (page "IFM K2
// Horizon Deep Dive ...", section "The Two Architectural Caching Strategies
// for MoVA", Option A: the routed vector is kept in the ordinary paged
// pools).  Slots outside [0, num_slots) store nothing.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace mova {

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;

// kMasked: the routing came from the caller, and a slot whose expert id is
// outside [0, E) has no partial row; it is skipped (adds nothing).
// extra (unmasked form only; may be null): a [T, N] fp16 term added after the
// k slots -- the FFN's shared expert.
// kBatch: every slot's piece is requested before the first is added (one
// memory round trip instead of k), then the pieces are summed in slot order;
// the same bits.  Taken when the grid is at most one round of workgroups
// (launch_combine), where the kernel waits on latency: measured, the decode
// step at T = 64 62.9 -> 61.8 us and the FFN at T = 64 222.9-225.5 ->
// 221.9-222.0 us; with thousands of workgroups (prefill T = 4096) it was
// slower, 142.3 -> 146.7-149.2 us.
template <bool kPaged, bool kMasked, bool kBatch>
__global__ __launch_bounds__(256) void combine_kernel(const f16_t* __restrict__ partial,
                                                      bf16_t* __restrict__ out, int T, int N, int k,
                                                      const int64_t* __restrict__ slot,
                                                      long long num_slots,
                                                      bf16_t* __restrict__ cache,
                                                      const int32_t* __restrict__ idx, int E,
                                                      const f16_t* __restrict__ extra) {
  const int vec_per_row = N / 8;
  const long long total = (long long)T * vec_per_row;
  for (long long v = blockIdx.x * 256ll + threadIdx.x; v < total; v += (long long)gridDim.x * 256) {
    const long long t = v / vec_per_row;
    const int c = (int)(v % vec_per_row) * 8;
    const f16_t* src = partial + (size_t)t * k * N + c;
    float s[8];
    if constexpr (kBatch && !kMasked) {
      u32x4 h[kMaxTopK];
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j)
        if (j < k) h[j] = load16(src + (size_t)j * N);
      u32x4 hx = {0u, 0u, 0u, 0u};
      if (extra != nullptr) hx = load16(extra + (size_t)t * N + c);
      const f16x8 h0 = __builtin_bit_cast(f16x8, h[0]);
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] = (float)h0[i];
#pragma unroll
      for (int j = 1; j < kMaxTopK; ++j) {
        if (j < k) {
          const f16x8 h2 = __builtin_bit_cast(f16x8, h[j]);
#pragma unroll
          for (int i = 0; i < 8; ++i) s[i] += (float)h2[i];
        }
      }
      if (extra != nullptr) {
        const f16x8 h2 = __builtin_bit_cast(f16x8, hx);
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] += (float)h2[i];
      }
    } else if constexpr (kBatch) {
      // Masked, batched: the valid slots' pieces first, then the sum below's
      // order (first valid slot assigned).
      bool valid[kMaxTopK];
      u32x4 h[kMaxTopK];
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        const int e = j < k ? idx[(size_t)t * k + j] : -1;
        valid[j] = e >= 0 && e < E;
      }
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j)
        if (valid[j]) h[j] = load16(src + (size_t)j * N);
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] = 0.f;
      bool first = true;
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        if (!valid[j]) continue;
        const f16x8 h2 = __builtin_bit_cast(f16x8, h[j]);
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] = first ? (float)h2[i] : s[i] + (float)h2[i];
        first = false;
      }
    } else if (!kMasked) {
      const f16x8 h = __builtin_bit_cast(f16x8, load16(src));
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] = (float)h[i];
      for (int j = 1; j < k; ++j) {
        const f16x8 h2 = __builtin_bit_cast(f16x8, load16(src + (size_t)j * N));
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] += (float)h2[i];
      }
      if (extra != nullptr) {
        const f16x8 h2 = __builtin_bit_cast(f16x8, load16(extra + (size_t)t * N + c));
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] += (float)h2[i];
      }
    } else {
      // Same sum over the valid slots, in slot order; the first valid slot is
      // assigned rather than added to 0, so with every id valid the bits
      // equal the unmasked sum (a -0 partial stays -0).
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] = 0.f;
      bool first = true;
      for (int j = 0; j < k; ++j) {
        const int e = idx[(size_t)t * k + j];
        if (e < 0 || e >= E) continue;
        const f16x8 h2 = __builtin_bit_cast(f16x8, load16(src + (size_t)j * N));
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] = first ? (float)h2[i] : s[i] + (float)h2[i];
        first = false;
      }
    }
    u32x4 packed;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      packed[i] = (uint32_t)f32_to_bf16_bits(s[2 * i]) | ((uint32_t)f32_to_bf16_bits(s[2 * i + 1]) << 16);
    if (!kPaged) {
      store16(out + (size_t)t * N + c, packed);
    } else {
      if (out != nullptr) store16(out + (size_t)t * N + c, packed);
      const long long sl = slot[t];
      if (sl >= 0 && sl < num_slots) store16(cache + (size_t)sl * N + c, packed);
    }
  }
}

template <bool kBatch>
static void launch_combine_cfg(const CombineArgs& a, dim3 grid, hipStream_t stream) {
  if (a.idx != nullptr)
    combine_kernel<false, true, kBatch><<<grid, 256, 0, stream>>>(
        a.partial, a.out, a.T, a.N, a.k, nullptr, 0, nullptr, a.idx, a.E, nullptr);
  else if (a.cache == nullptr)
    combine_kernel<false, false, kBatch><<<grid, 256, 0, stream>>>(
        a.partial, a.out, a.T, a.N, a.k, nullptr, 0, nullptr, nullptr, 0, a.extra);
  else
    combine_kernel<true, false, kBatch><<<grid, 256, 0, stream>>>(
        a.partial, a.out, a.T, a.N, a.k, a.slot, a.num_slots, a.cache, nullptr, 0, a.extra);
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.k > kMaxTopK) return hipErrorInvalidValue;
  const long long total = (long long)a.T * (a.N / 8);
  const long long blocks = std::min<long long>((total + 255) / 256, 256ll * 16);
  const dim3 grid((unsigned)blocks);
  if (blocks <= 256) launch_combine_cfg<true>(a, grid, stream);
  else launch_combine_cfg<false>(a, grid, stream);
  return hipGetLastError();
}

}  // namespace mova
