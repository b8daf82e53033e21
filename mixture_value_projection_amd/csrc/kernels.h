// Internal launch interface between the C ABI (mova_api.hip) and the kernels.
#pragma once

#include <atomic>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace mova {

// Runs set() once per device, for per-device function attributes (device
// ordinals from 64 on: every call).  Thread-safe: concurrent first calls may
// both run set(), which must be idempotent.
template <class F>
inline hipError_t once_per_device(std::atomic<unsigned long long>& done, F set) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = (dev >= 0 && dev < 64) ? 1ull << dev : 0ull;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  e = set();
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Kernel-choice overrides (tests and measurements), set only through
// mova_debug_override; 0 is the automatic choice.  Keys and values as the
// mova_override enum of include/mova.h.  A relaxed atomic load: no call reads
// the environment.
enum OverrideKey {
  kOvPath = 0,
  kOvRouter = 1,
  kOvGemmTile = 2,
  kOvDensePath = 3,
  kOvDecodeChain = 4,
  kOvDecodeGroups = 5,
  kOvSerial = 6,
  kOvCount = 7
};
int override_value(int key);

struct RouterArgs {
  const __bf16* x;
  const __bf16* wr;
  const float* bias;  // may be null
  int T, d, E, k;
  float scale;
  int32_t* idx;           // [T, k]
  float* w;               // [T, k]
  int32_t* chunk_counts;  // [blocks, E] or null
};

// LDS-staged router: one workgroup per router_chunk_tokens(T) tokens, top-k
// fused; with chunk_counts set, each workgroup writes its per-expert pair
// counts ([blocks, E]), so the dispatch chunk is router_chunk_tokens(T) tokens.
int router_chunk_tokens(int T);
hipError_t launch_router_lds(const RouterArgs& a, hipStream_t stream);
// The same kernel for up to 128 experts, 16 tokens per workgroup (the FFN
// router's chunk), no override.
hipError_t launch_router_lds_wide(const RouterArgs& a, hipStream_t stream);
// Small-T router: partial logits over many single-wave blocks, then top-k.
// Same bits as launch_router_lds.  plog: router_small_plog_floats(T) floats.
int router_small_plog_floats(int T);
hipError_t launch_router_small(const RouterArgs& a, float* plog, hipStream_t stream);
// Its first kernel alone (the class partials, for a consumer that selects).
hipError_t launch_router_partial(const RouterArgs& a, float* plog, hipStream_t stream);
// The same partials for up to 128 experts (the FFN router): plog rows of 128
// floats, 4 * ceil(T / 16) * 16 rows.
hipError_t launch_router_partial_wide(const RouterArgs& a, float* plog, hipStream_t stream);

// Experts the dispatch kernels handle (the value router itself takes at most
// kMaxExperts; routing of wider layers comes from their own router).
constexpr int kMaxDispatchExperts = 128;

struct DispatchArgs {
  const int32_t* idx;     // [T, k] routing
  int32_t* chunk_counts;  // [C, E] in: per-chunk counts; out: per-chunk offsets
  int32_t* expert_off;    // [E + 1] out: first sorted pair of each expert
  int32_t* tile_base;     // [E + 1] out: first M-tile of each expert
  int32_t* perm;          // [T * k] out: pair ids (t * k + slot) grouped by expert, stable
  int T, E, k;
  int chunk_tokens;  // tokens per chunk (router block)
  int block_m;       // M-tile height of the grouped GEMM
};
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t stream);
// chunk_counts from idx (routing supplied by the caller rather than the router);
// ids outside [0, E) are not counted.
hipError_t launch_dispatch_count(const DispatchArgs& a, hipStream_t stream);

// Tile shape of the tiled GEMM: 352 x 256 (routed modes only), 256 x 256,
// 128 x 256 or 128 x 128 (rows x columns), on 8 waves (2 x 4) or, for
// 128 x 128, also 4 waves (2 x 2), with `stages` LDS buffers (2; 3 or 4 for
// 128 x 128).
struct GemmTile {
  int bm, bn, waves, stages;
};

// What the tiled GEMM computes (epilogues in grouped_gemm.hip).
enum GemmMode {
  kGemmRoutedSilu = 0,    // value experts: partial = w * SiLU(x W_e^T), fp16
  kGemmDense = 1,         // dense v_proj: out = x W^T, bf16
  kGemmRoutedSwiGLU = 2,  // FFN experts, gate/up: out[pair] = SiLU(gate) * up, bf16
  kGemmRoutedLinear = 3,  // FFN experts, down: partial = w * (h_pair W_e^T), fp16
  kGemmDenseSwiGLU = 4,   // shared FFN expert, gate/up, bf16
  kGemmDenseF16 = 5       // shared FFN expert, down: partial = x W^T, fp16
};

struct GemmArgs {
  const __bf16* x;         // A rows: [T, d] (or [T * k, d] for kGemmRoutedLinear)
  const __bf16* W;         // [E, N, d] (dense modes: [N, d])
  const int32_t* perm;     // [T * k]
  const float* topk_w;     // [T * k]
  const int32_t* expert_off;
  const int32_t* tile_base;  // M-tile bases for tile.bm (routed modes)
  f16_t* partial;          // fp16 results ([T * k, N] routed, [T, N] dense)
  __bf16* out;             // bf16 results ([T, N], or [T * k or T, N / 2] SwiGLU)
  int T, d, N, E, k;
  GemmTile tile;           // routed modes; dense modes choose their own
  int mode = kGemmRoutedSilu;
};
// Tile of the grouped GEMM for a call (the dispatch builds M-tiles of tile.bm rows).
GemmTile gemm_tile_grouped(int T, int k, int E, int N);
GemmTile gemm_tile_grouped_ffn(int T, int k, int E);  // the FFN's experts
// Upper bound on M-tiles of height bm for any routing of T tokens.
int gemm_max_mtiles(int T, int k, int E, int bm);
hipError_t launch_grouped_gemm(const GemmArgs& a, hipStream_t stream);
// Dense mode of the tiled GEMM: out = x W^T over T rows and one [N, d] weight
// (x, W, out, T, d, N are read; the routing fields are ignored).
GemmTile gemm_tile_dense(int T, int N);
hipError_t launch_dense_gemm(const GemmArgs& a, hipStream_t stream);

// Output of the split-k dense kernel's reduction.
enum DenseOut {
  kDenseOutBf16 = 0,   // out bf16 [T, N]
  kDenseOutF16 = 1,    // out_any fp16 [T, N]
  kDenseOutSwiGLU = 2  // out_any bf16 [T, N / 2]: SiLU(gate) * up of gate / up rows
                       // interleaved in blocks of 16 (as the SwiGLU GEMM modes)
};

struct DenseArgs {
  const __bf16* x;  // [T, d]
  const __bf16* W;  // [N, d]
  float* part;      // [dense_skinny_splits(d), T, N] fp32 scratch
  __bf16* out;      // [T, N] (kDenseOutBf16)
  int T, d, N;
  int out_mode = kDenseOutBf16;
  void* out_any = nullptr;  // kDenseOutF16 / kDenseOutSwiGLU output
};
// The split-k dense kernel handles at most this many tokens per call.
constexpr int kDenseSkinnyMaxT = 256;
int dense_skinny_splits(int d);
size_t dense_skinny_partial_floats(int T, int d, int N);
hipError_t launch_dense_skinny(const DenseArgs& a, hipStream_t stream);

struct DecodeArgs {
  const __bf16* x;      // A rows: tokens [T, d], or (kGemmRoutedLinear) one row per pair [T * k, d]
  const __bf16* W;      // [E, N, d]
  const int32_t* idx;   // [T, k]
  const float* topk_w;  // [T, k]
  f16_t* partial;       // [T * k, N] (kGemmRoutedSilu, kGemmRoutedLinear)
  int T, d, N, E, k;
  // Epilogue, as the grouped GEMM's mode of the same name: kGemmRoutedSilu,
  // kGemmRoutedSwiGLU (gate / up rows interleaved in blocks of 16, writes
  // out_h[pair, N / 2] bf16) or kGemmRoutedLinear.
  int mode = kGemmRoutedSilu;
  __bf16* out_h = nullptr;
};
// The decode path handles at most this many tokens per call.
constexpr int kDecodeMaxT = 256;
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Token-major small-T value experts with the k-way combine fused: writes the
// bf16 rows to out (if not null) and to cache row slot[t] (if cache is set
// and 0 <= slot[t] < num_slots).  decode_token_stages: 0 when the kernel does
// not take the call (by shape, the automatic choice or kOvDecodeChain).
struct DecodeTokenArgs {
  const __bf16* x;       // [T, d]
  const __bf16* W;       // [E, N, d]
  int32_t* idx;          // [T, k]; ids outside [0, E) add nothing (written when plog is set)
  float* topk_w;         // [T, k] (written when plog is set)
  __bf16* out;           // [T, N] or null
  const int64_t* slot = nullptr;
  long long num_slots = 0;
  __bf16* cache = nullptr;
  int T, d, N, E, k;
  // Set: the routing is selected in the kernel from the small-T router's
  // class partials (launch_router_partial; Tp rows per class plane), with
  // the selection bias and scale, instead of read from idx / topk_w.
  const float* plog = nullptr;
  int Tp = 0;
  const float* bias = nullptr;
  float scale = 1.f;
};
int decode_token_stages(int T, int d, int N, int E, int k);
hipError_t launch_decode_token(const DecodeTokenArgs& a, int stages, hipStream_t stream);

struct CombineArgs {
  const f16_t* partial;  // [T * k, N]
  __bf16* out;           // [T, N]; may be null when cache is set
  int T, N, k;
  // Paged store (cache null = none): row t also goes to cache row slot[t]
  // when 0 <= slot[t] < num_slots.
  const int64_t* slot = nullptr;
  long long num_slots = 0;
  __bf16* cache = nullptr;
  // Caller-supplied routing (null = router output): slot i of token t is
  // skipped when idx[t * k + i] is outside [0, E) (its partial row is never
  // written).
  const int32_t* idx = nullptr;
  int E = 0;
  // Optional [T, N] fp16 term added after the k slots (the FFN's shared expert).
  const f16_t* extra = nullptr;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

// Compact routing record (record.hip): k ids at kRecordIdBits bits each in
// one 32-bit word per token (k <= kRecordMaxK), k fp16 weights.
constexpr int kRecordIdBits = 6;
constexpr int kRecordMaxK = 32 / kRecordIdBits;
hipError_t launch_record_pack(const int32_t* idx, const float* w, int T, int k, uint32_t* ids,
                              f16_t* w16, hipStream_t stream);
hipError_t launch_record_unpack(const uint32_t* ids, const f16_t* w16, int T, int k, int32_t* idx,
                                float* w, hipStream_t stream);

// FFN mixture of experts (ffn.hip): router for E <= kMaxDispatchExperts
// (partial logits in plog, ffn_router_plog_floats(T) floats; selection in
// workgroups of ffn_router_chunk_tokens() tokens, which is also the dispatch
// chunk; chunk_counts [blocks, E]), and the gate/up row interleaving.
int ffn_router_chunk_tokens();
size_t ffn_router_plog_floats(int T);
hipError_t launch_ffn_router(const RouterArgs& a, float* plog, hipStream_t stream);
hipError_t launch_ffn_pack_gate_up(const __bf16* gate, const __bf16* up, __bf16* dst, int E,
                                   int inter, int d, hipStream_t stream);

}  // namespace mova
