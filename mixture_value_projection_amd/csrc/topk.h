// Wave-wide top-k selection shared by the router kernels and the small-T
// expert kernel that selects for its own token.
#pragma once

#include "common.h"

namespace mova {

// Sigmoid, bias-for-selection, top-k and renormalisation for NT tokens at
// once, one lane per expert.  logit[i] is lane e's logit for token i.  Returns
// (in lanes j < k) the j-th selected expert of each token and its weight.
// Selection order: score desc, index asc.
//
// Each lane's selection score is mapped to an unsigned 32-bit key of the
// same order (-0 and +0 alike).  Each of the k rounds takes, per token, the
// wave-wide maximum key: rows of 16 lanes reduce with four DPP rotations,
// then two row broadcasts carry the maximum into lane 63.  The lanes holding
// that key are found with one ballot, and the lowest of them (the lowest
// expert index among equal scores) wins and drops out of later rounds.  The
// k chosen sigmoid scores are summed in rank order.  The NT tokens' chains
// are independent, which lets their latencies overlap.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t max_dpp(uint32_t v) {
  // Rows outside kRowMask read 0, the identity of an unsigned max (this lets
  // the compiler fold the move into the max as one DPP instruction).
  const uint32_t p = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, kRowMask, 0xF, false);
  return p > v ? p : v;
}

template <int NT>
__device__ __forceinline__ void topk_tokens(const float (&logit)[NT], float b_lane, int lane, int E,
                                            int k, float scale, int (&my_idx)[NT],
                                            float (&my_w)[NT]) {
  float sc[NT], ssum[NT], mine[NT];
  uint32_t key[NT];
  int pick[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    sc[i] = sigmoidf_fast(logit[i]);
    float sel = sc[i] + b_lane;
    sel = (sel == 0.f) ? 0.f : sel;  // -0 and +0 rank as equal, as in a float compare
    const uint32_t u = __float_as_uint(sel);
    key[i] = lane < E ? ((u & 0x80000000u) ? ~u : (u | 0x80000000u)) : 0u;  // no expert: minimum
    ssum[i] = 0.f;
    mine[i] = 0.f;
    pick[i] = 0;
  }
  for (int r = 0; r < k; ++r) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      uint32_t m = key[i];
      m = max_dpp<0x121, 0xF>(m);  // row_ror:1
      m = max_dpp<0x122, 0xF>(m);  // row_ror:2
      m = max_dpp<0x124, 0xF>(m);  // row_ror:4
      m = max_dpp<0x128, 0xF>(m);  // row_ror:8
      m = max_dpp<0x142, 0xA>(m);  // row_bcast:15 into rows 1 and 3
      m = max_dpp<0x143, 0xC>(m);  // row_bcast:31 into rows 2 and 3
      const uint32_t top = (uint32_t)__builtin_amdgcn_readlane((int)m, 63);
      const uint64_t hits = __ballot(key[i] == top);
      const int win = __builtin_amdgcn_readfirstlane(__ffsll((unsigned long long)hits) - 1);
      const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc[i]), win));
      ssum[i] += ws;
      if (lane == r) {
        pick[i] = win;
        mine[i] = ws;
      }
      if (lane == win) key[i] = 0u;
    }
  }
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    // Clamped so that even non-finite scores (undefined results) can never
    // produce an out-of-range expert index for the kernels that follow.
    my_idx[i] = min(max(pick[i], 0), E - 1);
    my_w[i] = scale * mine[i] / ssum[i];
  }
}

// topk_tokens for up to 128 experts, two per lane: lane l holds experts l
// (logit0) and l + 64 (logit1).  Each round takes the wave-wide maximum of
// the lanes' larger key; the winner is the lowest expert index among the
// keys equal to it (experts 0 .. 63 first, then 64 .. 127).  Same selection
// order, weight sum and weights as topk_tokens.
template <int NT>
__device__ __forceinline__ void topk_tokens2(const float (&logit0)[NT], const float (&logit1)[NT],
                                             float b0, float b1, int lane, int E, int k,
                                             float scale, int (&my_idx)[NT], float (&my_w)[NT]) {
  float sc0[NT], sc1[NT], ssum[NT], mine[NT];
  uint32_t key0[NT], key1[NT];
  int pick[NT];
  auto order = [](float sel) {
    sel = (sel == 0.f) ? 0.f : sel;  // -0 and +0 rank as equal, as in a float compare
    const uint32_t u = __float_as_uint(sel);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  };
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    sc0[i] = sigmoidf_fast(logit0[i]);
    sc1[i] = sigmoidf_fast(logit1[i]);
    key0[i] = lane < E ? order(sc0[i] + b0) : 0u;
    key1[i] = lane + 64 < E ? order(sc1[i] + b1) : 0u;
    ssum[i] = 0.f;
    mine[i] = 0.f;
    pick[i] = 0;
  }
  for (int r = 0; r < k; ++r) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      uint32_t m = key0[i] > key1[i] ? key0[i] : key1[i];
      m = max_dpp<0x121, 0xF>(m);
      m = max_dpp<0x122, 0xF>(m);
      m = max_dpp<0x124, 0xF>(m);
      m = max_dpp<0x128, 0xF>(m);
      m = max_dpp<0x142, 0xA>(m);
      m = max_dpp<0x143, 0xC>(m);
      const uint32_t top = (uint32_t)__builtin_amdgcn_readlane((int)m, 63);
      const uint64_t hits0 = __ballot(key0[i] == top);
      const uint64_t hits1 = __ballot(key1[i] == top);
      const int win = __builtin_amdgcn_readfirstlane(
          hits0 != 0ull ? __ffsll((unsigned long long)hits0) - 1
                        : 64 + __ffsll((unsigned long long)hits1) - 1);
      const float sv = win < 64 ? sc0[i] : sc1[i];  // win is wave-uniform
      const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv), win & 63));
      ssum[i] += ws;
      if (lane == r) {
        pick[i] = win;
        mine[i] = ws;
      }
      if (lane == win) key0[i] = 0u;
      if (lane + 64 == win) key1[i] = 0u;
    }
  }
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    my_idx[i] = min(max(pick[i], 0), E - 1);
    my_w[i] = scale * mine[i] / ssum[i];
  }
}

}  // namespace mova
