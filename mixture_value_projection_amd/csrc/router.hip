// Router: logits = x Wr^T (fp32 accumulation of bf16 products on MFMA),
// sigmoid scores, bias added for selection, wave-wide top-k with the lower
// expert index winning ties, renormalised weights times `scale`.
//
// Method: page "MoVA: routing the value vectors, and why the KV cache does not
// notice", section "Where the routing happens" (weight-only router linear map,
// sigmoid scoring, top-4, scaling factor 2.5).
//
// Summation order, shared by every router kernel so that a token's logits are
// the same bits whichever kernel, block shape or call processed it: the
// d-long dot product of a (token, expert) pair is split into four residue
// classes of 32-wide k steps (step mod 4); class rc is one MFMA chain over
// steps rc, rc + 4, rc + 8, ... in increasing order, with the token in MFMA
// row t % 16 and the expert in column e % 16; the four class partials are
// then added in class order, ((p0 + p1) + p2) + p3.  Chains padded to a whole
// number of load batches multiply a zeroed token operand, which adds +0.
//
// Kernels:
//   router_tile_kernel     one workgroup per 16 * TG tokens, wave = class;
//                          selection (lane = token) and the per-chunk
//                          dispatch histogram in the same kernel (large T,
//                          and routing-only calls);
//   router_staged_kernel   one workgroup per 32 or 64 tokens, the router
//                          weight staged through LDS once per workgroup and
//                          shared by its 8 or 16 waves (mid-size T);
//   router_partial_kernel  + router_topk_kernel: the same chains spread over
//                          single-wave workgroups for small T.
#include <stdlib.h>
#include <string.h>

#include "common.h"
#include "kernels.h"

namespace mova {

// Sigmoid, bias-for-selection, top-k and renormalisation for NT tokens at
// once, one lane per expert.  logit[i] is lane e's logit for token i.  Returns
// (in lanes j < k) the j-th selected expert of each token and its weight.
// Selection order: score desc, index asc.
//
// Each of the k rounds takes, per token, the wave-wide maximum of a 64-bit
// key: the selection score's bits mapped to an unsigned integer of the same
// order, then 63 - lane, so that equal scores rank the lower expert first.
// Rows of 16 lanes reduce with four DPP rotations, then two row broadcasts
// carry the maximum into lane 63.  The winner drops out of later rounds.  The
// k chosen sigmoid scores are summed in rank order.  The NT tokens' chains are
// independent, which lets their latencies overlap.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ void key_max_dpp(uint32_t& h, uint32_t& l) {
  const uint32_t ph = (uint32_t)__builtin_amdgcn_update_dpp((int)h, (int)h, kCtrl, kRowMask, 0xF, false);
  const uint32_t pl = (uint32_t)__builtin_amdgcn_update_dpp((int)l, (int)l, kCtrl, kRowMask, 0xF, false);
  const bool gt = ph > h || (ph == h && pl > l);
  h = gt ? ph : h;
  l = gt ? pl : l;
}

template <int NT>
__device__ __forceinline__ void topk_tokens(const float (&logit)[NT], float b_lane, int lane, int E,
                                            int k, float scale, int (&my_idx)[NT],
                                            float (&my_w)[NT]) {
  float sc[NT], ssum[NT], mine[NT];
  uint32_t kh[NT], kl[NT];
  int pick[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    sc[i] = sigmoidf_fast(logit[i]);
    float sel = sc[i] + b_lane;
    sel = (sel == 0.f) ? 0.f : sel;  // -0 and +0 rank as equal, as in a float compare
    const uint32_t u = __float_as_uint(sel);
    kh[i] = 0u;                      // lanes without an expert keep the minimum key
    kl[i] = 0u;
    if (lane < E) {
      kh[i] = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
      kl[i] = 63u - (uint32_t)lane;
    }
    ssum[i] = 0.f;
    mine[i] = 0.f;
    pick[i] = 0;
  }
  for (int r = 0; r < k; ++r) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      uint32_t mh = kh[i], ml = kl[i];
      key_max_dpp<0x121, 0xF>(mh, ml);  // row_ror:1
      key_max_dpp<0x122, 0xF>(mh, ml);  // row_ror:2
      key_max_dpp<0x124, 0xF>(mh, ml);  // row_ror:4
      key_max_dpp<0x128, 0xF>(mh, ml);  // row_ror:8
      key_max_dpp<0x142, 0xA>(mh, ml);  // row_bcast:15 into rows 1 and 3
      key_max_dpp<0x143, 0xC>(mh, ml);  // row_bcast:31 into rows 2 and 3
      const uint32_t bl = (uint32_t)__builtin_amdgcn_readlane((int)ml, 63);
      const int win = 63 - (int)(bl & 63u);
      const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc[i]), win));
      ssum[i] += ws;
      if (lane == r) {
        pick[i] = win;
        mine[i] = ws;
      }
      if (lane == win) {
        kh[i] = 0u;
        kl[i] = 0u;
      }
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

// One lane's running top-k list (slots 0 .. k-1 of KK >= k), ordered by
// (selection score desc, expert index asc).  A candidate enters at the first
// slot whose score it strictly exceeds, and everything from there shifts down
// one slot (the carried entry ranks ahead of all later ones).  Candidates
// offered in increasing expert index therefore keep the lower index first
// among equal scores: the same order as topk_tokens.
template <int KK>
__device__ __forceinline__ void insert_ranked(float (&bv)[KK], float (&bs)[KK], int (&bi)[KK],
                                              int k, float cv, float cs, int ci) {
  bool moving = false;
#pragma unroll
  for (int j = 0; j < KK; ++j) {
    if (j < k && (moving || cv > bv[j])) {
      const float tv = bv[j], ts = bs[j];
      const int ti = bi[j];
      bv[j] = cv;
      bs[j] = cs;
      bi[j] = ci;
      cv = tv;
      cs = ts;
      ci = ti;
      moving = true;
    }
  }
}

// Selection with lane = token for a tile of TM <= 64 tokens whose class
// partials sit in part[4][TM][kMaxExperts + 1]: wave w < 4 keeps each token's
// top-k over experts 16w .. 16w + 15 (offered in index order), and wave 0
// merges the other three waves' lists in wave order -- the same selection,
// order and weight sum as topk_tokens.  Every thread of the workgroup calls
// it (it holds a barrier); waves past 3 only take part in the barrier.  bq:
// the biases of the wave's 16 experts (load_selection_bias).  Writes rows
// t0 .. t0 + TM - 1 (those below T) of idx / w, and counts the selected
// experts into hist when it is not null.
constexpr int kSelQ = kMaxExperts / 4;  // experts per selecting wave

__device__ __forceinline__ void load_selection_bias(const float* __restrict__ bias, int wave, int E,
                                                    float (&bq)[kSelQ]) {
  const int wq = __builtin_amdgcn_readfirstlane(wave & 3);  // wave-uniform: scalar loads
#pragma unroll
  for (int j = 0; j < kSelQ; ++j) bq[j] = (bias != nullptr && wq * kSelQ + j < E) ? bias[wq * kSelQ + j] : 0.f;
}

template <int TM, int KK>
__device__ __forceinline__ void select_lane_token(
    const float (*part)[TM][kMaxExperts + 1], float (*cand_v)[KK][TM], float (*cand_s)[KK][TM],
    int (*cand_i)[KK][TM], int wave, int lane, const float (&bq)[kSelQ], int E, int k,
    float scale, int t0, int T, int32_t* __restrict__ idx_out, float* __restrict__ w_out,
    int* hist) {
  constexpr int kQ = kSelQ;
  float bv[KK], bs[KK];
  int bi[KK];
#pragma unroll
  for (int j = 0; j < KK; ++j) {
    bv[j] = -__builtin_inff();
    bs[j] = 0.f;
    bi[j] = 0;
  }
  if (wave < 4 && lane < TM) {
#pragma unroll
    for (int j = 0; j < kQ; ++j) {
      const int e = wave * kQ + j;
      if (e < E) {
        const float logit =
            ((part[0][lane][e] + part[1][lane][e]) + part[2][lane][e]) + part[3][lane][e];
        const float sc = sigmoidf_fast(logit);
        insert_ranked<KK>(bv, bs, bi, k, sc + bq[j], sc, e);
      }
    }
    if (wave > 0) {
#pragma unroll
      for (int j = 0; j < KK; ++j) {
        cand_v[wave - 1][j][lane] = bv[j];
        cand_s[wave - 1][j][lane] = bs[j];
        cand_i[wave - 1][j][lane] = bi[j];
      }
    }
  }
  __syncthreads();
  if (wave == 0 && lane < TM) {
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
      for (int j = 0; j < KK; ++j)
        if (j < k)
          insert_ranked<KK>(bv, bs, bi, k, cand_v[w][j][lane], cand_s[w][j][lane], cand_i[w][j][lane]);
    float ssum = 0.f;
#pragma unroll
    for (int j = 0; j < KK; ++j)
      if (j < k) ssum += bs[j];
    const int t = t0 + lane;
    if (t < T) {
#pragma unroll
      for (int j = 0; j < KK; ++j) {
        if (j < k) {
          // Clamped so that even non-finite scores (undefined results) can
          // never produce an out-of-range expert index.
          const int e = min(max(bi[j], 0), E - 1);
          idx_out[(size_t)t * k + j] = e;
          w_out[(size_t)t * k + j] = scale * bs[j] / ssum;
          if (hist != nullptr) atomicAdd(&hist[e], 1);
        }
      }
    }
  }
}

// ---- tile router: one workgroup per 16 * TG tokens ------------------------
//
// Wave rc (of 4) runs class rc's chains for all TG token groups against all
// four expert blocks: per k step it loads one 16-byte token fragment per token
// group and one router-weight fragment per expert block, U steps per batch,
// all loads of a batch before its MFMAs.  Class partials meet in LDS (rows
// padded by one word so that a column read by 64 lanes hits 64 banks).
// Selection: 16-token tiles use topk_tokens (lane = expert, four tokens per
// wave); larger tiles run with lane = token: wave w keeps each token's top-k
// over experts 16w .. 16w + 15 (offered in index order), and wave 0 merges
// the other three waves' lists in wave order -- the same selection, order and
// weight sum as topk_tokens, at a fraction of the cost per token.  A
// workgroup's tokens form one dispatch chunk: when chunk_counts is given, it
// receives the workgroup's per-expert pair counts.  KK: list length (k <= KK).
template <int TG, int U, int KK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void router_tile_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr, const float* __restrict__ bias,
    int T, int d, int E, int k, float scale,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out, int32_t* __restrict__ chunk_counts) {
  constexpr int TM = 16 * TG;
  constexpr int kPad = kMaxExperts + 1;
  __shared__ float part[4][TM][kPad];
  constexpr bool kLaneToken = TG > 1;        // selection with lane = token
  constexpr int TC = kLaneToken ? TM : 1;
  __shared__ float cand_v[3][KK][TC];       // selection lists of waves 1..3
  __shared__ float cand_s[3][KK][TC];
  __shared__ int cand_i[3][KK][TC];
  __shared__ int hist[kMaxExperts];

  const int lane = threadIdx.x & 63;
  const int rc = threadIdx.x >> 6;
  const int q = lane >> 4;
  const int r16 = lane & 15;
  const int t0 = blockIdx.x * TM;

  if (threadIdx.x < kMaxExperts) hist[threadIdx.x] = 0;
  // Biases of this wave's selection experts.
  float bq[kSelQ];
  load_selection_bias(bias, rc, E, bq);
  // Token rows clamped into range (rows past T are never written); expert rows
  // clamped (experts >= E are never offered to the selection).
  const bf16_t* xrow[TG];
#pragma unroll
  for (int g = 0; g < TG; ++g) xrow[g] = x + (size_t)min(t0 + g * 16 + r16, T - 1) * d + q * 8;
  const bf16_t* wrow[4];
#pragma unroll
  for (int eb = 0; eb < 4; ++eb) wrow[eb] = wr + (size_t)min(eb * 16 + r16, E - 1) * d + q * 8;

  f32x4 acc[TG][4];
#pragma unroll
  for (int g = 0; g < TG; ++g)
#pragma unroll
    for (int eb = 0; eb < 4; ++eb) acc[g][eb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int steps = d / 32;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int s0 = rc; s0 < steps; s0 += 4 * U) {
    Frag16 a[U][TG], b[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sc = min(s0 + 4 * u, steps - 1);
#pragma unroll
      for (int g = 0; g < TG; ++g) a[u][g].u = load16(xrow[g] + sc * 32);
#pragma unroll
      for (int eb = 0; eb < 4; ++eb) b[u][eb].u = load16(wrow[eb] + sc * 32);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool live = s0 + 4 * u < steps;
#pragma unroll
      for (int g = 0; g < TG; ++g) {
        Frag16 av;
        av.u = live ? a[u][g].u : zero;
#pragma unroll
        for (int eb = 0; eb < 4; ++eb) acc[g][eb] = mfma16x16x32(av.h, b[u][eb].h, acc[g][eb]);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < TG; ++g)
#pragma unroll
    for (int eb = 0; eb < 4; ++eb)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[rc][g * 16 + q * 4 + i][eb * 16 + r16] = acc[g][eb][i];
  __syncthreads();

  if constexpr (!kLaneToken) {
    // 16-token tiles: lane = expert, wave rc selects for tokens rc, rc + 4,
    // rc + 8, rc + 12 together (topk_tokens).
    const float b_lane = (bias != nullptr && lane < E) ? bias[lane] : 0.f;
    float logit[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rc + 4 * i;
      logit[i] = ((part[0][r][lane] + part[1][r][lane]) + part[2][r][lane]) + part[3][r][lane];
    }
    int my_idx[4];
    float my_w[4];
    topk_tokens<4>(logit, b_lane, lane, E, k, scale, my_idx, my_w);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + rc + 4 * i;
      if (t < T && lane < k) {
        idx_out[(size_t)t * k + lane] = my_idx[i];
        w_out[(size_t)t * k + lane] = my_w[i];
        if (chunk_counts != nullptr) atomicAdd(&hist[my_idx[i]], 1);
      }
    }
  } else {
    // Larger tiles: lane = token (row `lane` of the tile).
    select_lane_token<TM, KK>(part, cand_v, cand_s, cand_i, rc, lane, bq, E, k, scale, t0, T,
                              idx_out, w_out, chunk_counts != nullptr ? hist : nullptr);
  }
  if (chunk_counts != nullptr) {
    __syncthreads();
    if (threadIdx.x < E) chunk_counts[(size_t)blockIdx.x * E + threadIdx.x] = hist[threadIdx.x];
  }
}

// ---- staged-weight router: one workgroup per TM = 32 or 64 tokens --------
//
// The tile router's workgroups each read the whole router weight (d * E * 2
// bytes) from L2 for their 16 .. 64 tokens, and that read, not the tokens,
// sets its time at large T.  Here the weight goes through LDS once per
// workgroup and is shared by 4 * TM / 16 waves: wave w runs class rc = w % 4's
// chains for token group g = w / 4 against all four expert blocks.  The
// weight arrives in chunks of 8 k steps (all 64 expert rows, 32 KB): thread
// slots copy 16-byte pieces global -> registers -> LDS, kChunksAhead chunks
// ahead in registers, into two LDS buffers with one barrier per chunk; the
// token fragments (two per chunk per wave: steps 8j + rc and 8j + 4 + rc) are
// read straight from global memory the same number of chunks ahead.  Every
// chain adds the same products in the same order as the tile router's, so
// the logits, and everything after them, have the same bits.  Staged rows are
// 512 B; the 16-byte piece c of row r sits at c ^ (r & 7), so the 16 rows a
// fragment read touches fall in distinct bank groups.
constexpr int kStageSteps = 8;                                // k steps per staged chunk
constexpr int kStageRowBytes = kStageSteps * 32 * 2;          // 512 B per expert row
constexpr int kStageBytes = kMaxExperts * kStageRowBytes;     // 32 KB per chunk
constexpr int kChunksAhead = 3;

template <int TM, int KK>
__global__ __launch_bounds__(4 * TM * 4) void router_staged_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr, const float* __restrict__ bias,
    int T, int d, int E, int k, float scale,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out, int32_t* __restrict__ chunk_counts) {
  constexpr int kGroupsT = TM / 16;
  constexpr int kThreads = 64 * 4 * kGroupsT;
  constexpr int kPieces = kStageBytes / 16 / kThreads;  // 16-byte pieces per thread per chunk
  constexpr int kPad = kMaxExperts + 1;
  // The class partials are written only after the k loop, into the memory
  // of the weight buffers (32-token tiles then fit two workgroups per CU).
  constexpr int kPartBytes = 4 * TM * kPad * 4;
  constexpr int kUnion = kPartBytes > 2 * kStageBytes ? kPartBytes : 2 * kStageBytes;
  __shared__ __attribute__((aligned(16))) char smem[kUnion];
  char(*stage)[kStageBytes] = reinterpret_cast<char(*)[kStageBytes]>(smem);
  float(*part)[TM][kPad] = reinterpret_cast<float(*)[TM][kPad]>(smem);
  __shared__ float cand_v[3][KK][TM];
  __shared__ float cand_s[3][KK][TM];
  __shared__ int cand_i[3][KK][TM];
  __shared__ int hist[kMaxExperts];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rc = wave & 3;
  const int g = wave >> 2;
  const int q = lane >> 4;
  const int r16 = lane & 15;
  const int t0 = blockIdx.x * TM;
  const int steps = d / 32;
  const int nch = ceil_div(steps, kStageSteps);

  if (tid < kMaxExperts) hist[tid] = 0;
  float bq[kSelQ];
  load_selection_bias(bias, wave, E, bq);

  // This thread's pieces of a chunk: row er (expert, clamped below E), piece
  // c (16 B) of the row's 512 B; the last chunk's pieces past d are clamped
  // to d's last piece (loaded, never used: their steps are skipped).
  const bf16_t* wrow[kPieces];
  int wcol[kPieces];  // the piece's first element within the chunk's 256
  int wdst[kPieces];
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    const int slot = tid + i * kThreads;
    const int er = slot / (kStageRowBytes / 16);
    const int c = slot % (kStageRowBytes / 16);
    wrow[i] = wr + (size_t)min(er, E - 1) * d;
    wcol[i] = c * 8;
    wdst[i] = er * kStageRowBytes + ((c ^ (er & 7)) << 4);
  }
  const bf16_t* xrow = x + (size_t)min(t0 + g * 16 + r16, T - 1) * d + q * 8;

  u32x4 wq[kChunksAhead][kPieces];
  u32x4 xq[kChunksAhead][2];
  auto load_chunk = [&](int j, u32x4 (&w)[kPieces], u32x4 (&xf)[2]) {
    const int jj = min(j, nch - 1);  // past the end: reload the last chunk (never used)
#pragma unroll
    for (int i = 0; i < kPieces; ++i)
      w[i] = load16(wrow[i] + min(jj * kStageSteps * 32 + wcol[i], d - 8));
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int st = min(jj * kStageSteps + 4 * u + rc, steps - 1);
      xf[u] = load16(xrow + st * 32);
    }
  };
#pragma unroll
  for (int a = 0; a < kChunksAhead; ++a) load_chunk(a, wq[a], xq[a]);

  f32x4 acc[4];
#pragma unroll
  for (int eb = 0; eb < 4; ++eb) acc[eb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int j0 = 0; j0 < nch; j0 += kChunksAhead) {
#pragma unroll
    for (int a = 0; a < kChunksAhead; ++a) {
      const int j = j0 + a;
      if (j < nch) {  // uniform
        char* buf = stage[j & 1];
#pragma unroll
        for (int i = 0; i < kPieces; ++i) *reinterpret_cast<u32x4*>(buf + wdst[i]) = wq[a][i];
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int st = j * kStageSteps + 4 * u + rc;
          if (st < steps) {  // uniform per wave
            Frag16 av;
            av.u = xq[a][u];
#pragma unroll
            for (int eb = 0; eb < 4; ++eb) {
              const int row = eb * 16 + r16;
              const int c = (4 * u + rc) * 4 + q;
              Frag16 bw;
              bw.u = *reinterpret_cast<const u32x4*>(buf + row * kStageRowBytes + ((c ^ (row & 7)) << 4));
              acc[eb] = mfma16x16x32(av.h, bw.h, acc[eb]);
            }
          }
        }
        load_chunk(j + kChunksAhead, wq[a], xq[a]);
      }
    }
  }
  __syncthreads();  // every wave is done reading the weight buffers
#pragma unroll
  for (int eb = 0; eb < 4; ++eb)
#pragma unroll
    for (int i = 0; i < 4; ++i) part[rc][g * 16 + q * 4 + i][eb * 16 + r16] = acc[eb][i];
  __syncthreads();
  select_lane_token<TM, KK>(part, cand_v, cand_s, cand_i, wave, lane, bq, E, k, scale, t0, T,
                            idx_out, w_out, chunk_counts != nullptr ? hist : nullptr);
  if (chunk_counts != nullptr) {
    __syncthreads();
    if (tid < E) chunk_counts[(size_t)blockIdx.x * E + tid] = hist[tid];
  }
}

// Router kernel and tokens per workgroup for T.  The tile router's sizes were
// measured on the value layer's shape with the benchmark's inputs (the token
// rows are not cache-resident: a 32-token tile router is faster at T = 8192
// only when they are).
struct RouterChoice {
  bool staged;  // router_staged_kernel, else router_tile_kernel
  int tokens;   // tokens per workgroup (the dispatch chunk)
};

// Tile-router workgroup size by T (tokens re-read the weight from L2 per
// workgroup: larger tiles once there are enough workgroups).
static int tile_router_tokens(int T) { return T <= 8192 ? 16 : T <= 16384 ? 32 : 64; }

// Measured with the value layer's shape (routing alone, graph replay):
//   T       4096  4608  6144  8192  16384  20480  28672  32768
//   tile    17.2  28.4  28.9  28.8  38.4   47.9   48.8   48.6 us
//   staged  21.8  22.6  24.3  24.8  33.1   49.4   58.2   59.6   (32 tokens)
// so the staged router takes 4096 < T <= 18432.  The kOvRouter override
// forces the tile router (1) or the staged router with 32 (2) or 64 (3)
// tokens per workgroup (measurement, tests).
static RouterChoice router_choice(int T) {
  switch (override_value(kOvRouter)) {
    case 1: return {false, tile_router_tokens(T)};
    case 2: return {true, 32};
    case 3: return {true, 64};
    default: break;
  }
  if (T > 4096 && T <= 18432) return {true, 32};
  return {false, tile_router_tokens(T)};
}

int router_tile_tokens(int T) { return router_choice(T).tokens; }  // >= 16 for every choice

hipError_t launch_router_tile(const RouterArgs& a, hipStream_t stream) {
  const RouterChoice rch = router_choice(a.T);
  const int TM = rch.tokens;
  const dim3 grid(ceil_div(a.T, TM));
  if (rch.staged) {
    const bool small_k = a.k <= 4;
#define MOVA_ROUTER_STAGED(TMV, KK)                                                      \
  router_staged_kernel<TMV, KK><<<grid, 16 * TMV, 0, stream>>>(                          \
      a.x, a.wr, a.bias, a.T, a.d, a.E, a.k, a.scale, a.idx, a.w, a.chunk_counts)
    if (TM == 32) {
      if (small_k) MOVA_ROUTER_STAGED(32, 4); else MOVA_ROUTER_STAGED(32, 8);
    } else {
      if (small_k) MOVA_ROUTER_STAGED(64, 4); else MOVA_ROUTER_STAGED(64, 8);
    }
#undef MOVA_ROUTER_STAGED
    return hipGetLastError();
  }
#define MOVA_ROUTER_TILE(TG, U, KK)                                                            \
  router_tile_kernel<TG, U, KK><<<grid, 256, 0, stream>>>(a.x, a.wr, a.bias, a.T, a.d, a.E, a.k, \
                                                          a.scale, a.idx, a.w, a.chunk_counts)
  // U: k steps per load batch (TG + 4 fragments of 4 registers each per step).
  const bool small_k = a.k <= 4;
  if (TM == 16) {
    if (small_k) MOVA_ROUTER_TILE(1, 10, 4); else MOVA_ROUTER_TILE(1, 10, 8);
  } else if (TM == 32) {
    if (small_k) MOVA_ROUTER_TILE(2, 5, 4); else MOVA_ROUTER_TILE(2, 5, 8);
  } else {
    if (small_k) MOVA_ROUTER_TILE(4, 2, 4); else MOVA_ROUTER_TILE(4, 2, 8);
  }
#undef MOVA_ROUTER_TILE
  return hipGetLastError();
}

// ---- small T: the same chains spread over many single-wave workgroups ------
//
// Block (g, eb, rc) computes the class-rc partial logits of token group g (16
// tokens) against expert block eb (16 experts), all of its loads issued before
// its MFMAs.  The top-k kernel adds the four class partials in class order and
// selects with one wave per token.
template <int U>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 2))) void router_partial_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr, int T, int d, int E,
    float* __restrict__ plog /* [4][Tp][64] */, int Tp) {
  const int g = blockIdx.x, eb = blockIdx.y, rc = blockIdx.z;
  const int lane = threadIdx.x, q = lane >> 4, r16 = lane & 15;
  const bf16_t* xrow = x + (size_t)min(g * 16 + r16, T - 1) * d + q * 8;
  const bf16_t* wrow = wr + (size_t)min(eb * 16 + r16, E - 1) * d + q * 8;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int steps = d / 32;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int s0 = rc; s0 < steps; s0 += 4 * U) {
    Frag16 a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sc = min(s0 + 4 * u, steps - 1);
      b[u].u = load16(wrow + sc * 32);
      a[u].u = load16(xrow + sc * 32);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      Frag16 av;
      av.u = (s0 + 4 * u < steps) ? a[u].u : zero;
      acc = mfma16x16x32(av.h, b[u].h, acc);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    plog[((size_t)rc * Tp + g * 16 + q * 4 + i) * kMaxExperts + eb * 16 + r16] = acc[i];
}

__global__ __launch_bounds__(256) void router_topk_kernel(
    const float* __restrict__ plog, int Tp, const float* __restrict__ bias, int T, int E, int k,
    float scale, int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;  // one token per wave
  if (t >= T) return;
  const float b_lane = (bias != nullptr && lane < E) ? bias[lane] : 0.f;
  const size_t cls = (size_t)Tp * kMaxExperts;
  const float* src = plog + (size_t)t * kMaxExperts + lane;
  const float logit = ((src[0] + src[cls]) + src[2 * cls]) + src[3 * cls];
  const float lg[1] = {logit};
  int my_idx[1];
  float my_w[1];
  topk_tokens<1>(lg, b_lane, lane, E, k, scale, my_idx, my_w);
  if (lane < k) {
    idx_out[(size_t)t * k + lane] = my_idx[0];
    w_out[(size_t)t * k + lane] = my_w[0];
  }
}

int router_small_plog_floats(int T) { return 4 * ceil_div(T, 16) * 16 * kMaxExperts; }

hipError_t launch_router_small(const RouterArgs& a, float* plog, hipStream_t stream) {
  const int G = ceil_div(a.T, 16);
  const int Tp = G * 16;
  router_partial_kernel<20><<<dim3(G, 4, 4), 64, 0, stream>>>(a.x, a.wr, a.T, a.d, a.E, plog, Tp);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  router_topk_kernel<<<ceil_div(a.T, 4), 256, 0, stream>>>(plog, Tp, a.bias, a.T, a.E, a.k, a.scale,
                                                          a.idx, a.w);
  return hipGetLastError();
}

}  // namespace mova
