// Compact routing record of the compact value cache: per token, the k
// selected expert ids packed at 6 bits each into one 32-bit word (slot j in
// bits 6j .. 6j + 5, so k <= 5) and the k routing weights as fp16 (nearest
// even).  Page "IFM K2 Horizon Deep Dive: Inside Mixture-of-Value Attention
// (MoVA) ...", section "The Two Architectural Caching Strategies for MoVA",
// Option B, keeps x_t with its top-4 expert ids and four fp16 weights and
// rebuilds v_t from them; at k = 4 the record is 12 bytes per token.
#include "common.h"
#include "kernels.h"

namespace mova {

__global__ __launch_bounds__(256) void record_pack_kernel(const int32_t* __restrict__ idx,
                                                          const float* __restrict__ w, int T, int k,
                                                          uint32_t* __restrict__ ids,
                                                          f16_t* __restrict__ w16) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  uint32_t packed = 0;
  for (int j = 0; j < k; ++j) {
    packed |= (uint32_t)(idx[(size_t)t * k + j] & ((1 << kRecordIdBits) - 1)) << (kRecordIdBits * j);
    w16[(size_t)t * k + j] = (f16_t)w[(size_t)t * k + j];
  }
  ids[t] = packed;
}

__global__ __launch_bounds__(256) void record_unpack_kernel(const uint32_t* __restrict__ ids,
                                                            const f16_t* __restrict__ w16, int T, int k,
                                                            int32_t* __restrict__ idx,
                                                            float* __restrict__ w) {
  const long long i = blockIdx.x * 256ll + threadIdx.x;
  if (i >= (long long)T * k) return;
  const int t = (int)(i / k), j = (int)(i % k);
  idx[i] = (int32_t)((ids[t] >> (kRecordIdBits * j)) & ((1u << kRecordIdBits) - 1));
  w[i] = (float)w16[i];
}

hipError_t launch_record_pack(const int32_t* idx, const float* w, int T, int k, uint32_t* ids,
                              f16_t* w16, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  record_pack_kernel<<<ceil_div(T, 256), 256, 0, stream>>>(idx, w, T, k, ids, w16);
  return hipGetLastError();
}

hipError_t launch_record_unpack(const uint32_t* ids, const f16_t* w16, int T, int k, int32_t* idx,
                                float* w, hipStream_t stream) {
  const long long n = (long long)T * k;
  if (n <= 0) return hipSuccess;
  record_unpack_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(ids, w16, T, k, idx, w);
  return hipGetLastError();
}

}  // namespace mova
