// Dispatch: group the (token, slot) pairs by expert for the grouped GEMM.
//
// The reference implementation walks the touched experts one by one in a
// Python loop (page "MoVA: routing the value vectors ...", section "So what
// does it cost?").  Here the router already left a per-chunk, per-expert
// count (chunk = one router workgroup's tokens).  Two kernels finish the job
// without atomics on global memory:
//
//   count:   (only when the routing comes from the caller instead of the
//            router) the per-chunk, per-expert counts;
//   scan:    per expert, exclusive prefix of the counts over chunks (in
//            place), expert offsets, and the first M-tile of each expert;
//   scatter: each chunk re-reads its routing and writes every pair id
//            (t * k + slot) at expert_off[e] + chunk_off[c][e] + rank, where
//            rank counts earlier pairs of the same expert in the chunk.
//
// The result is stable: within an expert, pairs appear in increasing pair id,
// so the GEMM's row order -- and hence every output bit -- is independent of
// scheduling.  A pair whose expert id lies outside [0, E) is not counted and
// not placed (caller-supplied routing); the router never produces one.
#include "common.h"
#include "kernels.h"

namespace mova {

constexpr int kScanThreads = 1024;
constexpr int kScanMaxGroups = kScanThreads / 64;  // chunk ranges at E <= 64
constexpr int kScanRegs = 32;  // counts a thread keeps in registers between passes

// One workgroup.  Thread column = expert (64 columns when E <= 64, else 128),
// so every count load is a contiguous row of the [C, E] table; the
// 1024 / columns groups split the chunks, group w owning chunks
// [w * per, (w + 1) * per).  Pass 1 sums each thread's counts, the groups'
// sums give each range its starting offset, pass 2 rewrites the counts as
// offsets.  With at most kScanRegs chunks per thread (C <= 512 at E <= 64)
// the counts stay in registers between the passes, so the table is read
// once.
__global__ __launch_bounds__(kScanThreads) void dispatch_scan_kernel(
    int32_t* __restrict__ counts, int C, int E, int block_m,
    int32_t* __restrict__ expert_off, int32_t* __restrict__ tile_base) {
  __shared__ int wave_sum[kScanMaxGroups][kMaxDispatchExperts];
  __shared__ int total[kMaxDispatchExperts];
  __shared__ int mtiles[kMaxDispatchExperts];
  const int cols = E <= 64 ? 64 : kMaxDispatchExperts;
  const int groups = kScanThreads / cols;
  const int e = threadIdx.x % cols;
  const int w = threadIdx.x / cols;
  const int per = ceil_div(C, groups);
  const int c0 = min(C, w * per), c1 = min(C, c0 + per);
  const bool live = e < E;
  const bool cached = per <= kScanRegs;  // uniform

  int s = 0;
  int v[kScanRegs];
  if (cached) {
#pragma unroll
    for (int i = 0; i < kScanRegs; ++i) v[i] = (live && c0 + i < c1) ? counts[(size_t)(c0 + i) * E + e] : 0;
#pragma unroll
    for (int i = 0; i < kScanRegs; ++i) s += v[i];
  } else if (live) {
    for (int cb = c0; cb < c1; cb += 16) {
      int u[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) u[i] = (cb + i < c1) ? counts[(size_t)(cb + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) s += u[i];
    }
  }
  wave_sum[w][e] = s;
  __syncthreads();
  int run = 0;
  for (int i = 0; i < w; ++i) run += wave_sum[i][e];
  if (w == groups - 1) {
    total[e] = live ? run + s : 0;
    mtiles[e] = live ? ceil_div(run + s, block_m) : 0;
  }
  // Rewrite counts as offsets (reloading, block by block, when they were not
  // kept: each block of 16 is loaded before any of its stores).
  if (cached) {
    if (live) {
#pragma unroll
      for (int i = 0; i < kScanRegs; ++i) {
        if (c0 + i < c1) counts[(size_t)(c0 + i) * E + e] = run;
        run += v[i];
      }
    }
  } else if (live) {
    for (int cb = c0; cb < c1; cb += 16) {
      int u[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) u[i] = (cb + i < c1) ? counts[(size_t)(cb + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (cb + i < c1) counts[(size_t)(cb + i) * E + e] = run;
        run += u[i];
      }
    }
  }
  // The totals are in LDS; the offset stores above may still be in flight
  // (nothing below reads them), so the barrier waits for LDS work only.
  __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(63));
  raw_barrier();
  if (w == 0) {
    // Expert offsets and first M-tiles: exclusive prefix sums over the
    // experts (entries past E are zero), by an inclusive scan across each
    // wave's lanes; with 128 columns the second wave adds the first wave's
    // sum, which it reduces itself from the same table.
    const int lane = threadIdx.x & 63;
    int it = total[e], imt = mtiles[e];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int a = __shfl_up(it, o, 64), b = __shfl_up(imt, o, 64);
      if (lane >= o) {
        it += a;
        imt += b;
      }
    }
    if (e >= 64) {
      int st = total[lane], smt = mtiles[lane];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        st += __shfl_xor(st, o, 64);
        smt += __shfl_xor(smt, o, 64);
      }
      it += st;
      imt += smt;
    }
    if (e < E) {
      expert_off[e] = it - total[e];
      tile_base[e] = imt - mtiles[e];
    }
    if (e == cols - 1) {
      expert_off[E] = it;
      tile_base[E] = imt;
    }
  }
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ chunk_off,
    const int32_t* __restrict__ expert_off, int32_t* __restrict__ perm,
    int T, int E, int k, int chunk_tokens) {
  __shared__ int running[kMaxDispatchExperts];
  __shared__ int wave_cnt[4][kMaxDispatchExperts];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = blockIdx.x;
  const int p0 = c * chunk_tokens * k;
  const int npairs = min(T * k, p0 + chunk_tokens * k) - p0;

  if (threadIdx.x < kMaxDispatchExperts) running[threadIdx.x] = 0;
  for (int i = threadIdx.x; i < 4 * kMaxDispatchExperts; i += 256) (&wave_cnt[0][0])[i] = 0;
  __syncthreads();

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < npairs; base += 256) {
    const int p = base + threadIdx.x;
    const int e_raw = p < npairs ? idx[p0 + p] : 0;
    const bool valid = p < npairs && e_raw >= 0 && e_raw < E;
    const int e = valid ? e_raw : 0;
    // Lanes of this wave holding the same expert (7 ballots over the id bits).
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 7; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t on = __ballot(bit);
      peers &= bit ? on : ~on;
    }
    const int rank_in_wave = __popcll(peers & lt_mask);
    if (valid && rank_in_wave == 0) wave_cnt[wave][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int rank = running[e] + rank_in_wave;
      for (int w = 0; w < wave; ++w) rank += wave_cnt[w][e];
      perm[expert_off[e] + chunk_off[(size_t)c * E + e] + rank] = p0 + p;
    }
    __syncthreads();
    if (threadIdx.x < kMaxDispatchExperts) {
      const int x = threadIdx.x;
      running[x] += wave_cnt[0][x] + wave_cnt[1][x] + wave_cnt[2][x] + wave_cnt[3][x];
      wave_cnt[0][x] = wave_cnt[1][x] = wave_cnt[2][x] = wave_cnt[3][x] = 0;
    }
    __syncthreads();
  }
}

// Per-chunk expert counts of caller-supplied routing: one workgroup per chunk,
// LDS histogram (integer counts, so the order of the atomics does not matter).
__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ idx,
                                                             int32_t* __restrict__ counts, int T,
                                                             int E, int k, int chunk_tokens) {
  __shared__ int hist[kMaxDispatchExperts];
  const int c = blockIdx.x;
  const int p0 = c * chunk_tokens * k;
  const int npairs = min(T * k, p0 + chunk_tokens * k) - p0;
  if (threadIdx.x < kMaxDispatchExperts) hist[threadIdx.x] = 0;
  __syncthreads();
  for (int p = threadIdx.x; p < npairs; p += 256) {
    const int e = idx[p0 + p];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  if (threadIdx.x < E) counts[(size_t)c * E + threadIdx.x] = hist[threadIdx.x];
}

hipError_t launch_dispatch_count(const DispatchArgs& a, hipStream_t stream) {
  const int C = ceil_div(a.T, a.chunk_tokens);
  dispatch_count_kernel<<<C, 256, 0, stream>>>(a.idx, a.chunk_counts, a.T, a.E, a.k,
                                               a.chunk_tokens);
  return hipGetLastError();
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t stream) {
  const int C = ceil_div(a.T, a.chunk_tokens);
  dispatch_scan_kernel<<<1, kScanThreads, 0, stream>>>(a.chunk_counts, C, a.E, a.block_m,
                                                       a.expert_off, a.tile_base);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  dispatch_scatter_kernel<<<C, 256, 0, stream>>>(a.idx, a.chunk_counts, a.expert_off, a.perm,
                                                 a.T, a.E, a.k, a.chunk_tokens);
  return hipGetLastError();
}

}  // namespace mova
