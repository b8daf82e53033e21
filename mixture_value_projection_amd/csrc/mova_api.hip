// C ABI of the MoVA routed value projection: argument checks, workspace
// layout, path choice and launches.  Declarations and contracts: include/mova.h.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/mova.h"
#include "common.h"
#include "kernels.h"

namespace {

using namespace mova;

constexpr int kVersion = 200;  // 0.2.0
constexpr int kMaxT = 1 << 24;
// Token counts up to this take the weight-streaming decode path by default
// (measured faster than the grouped path for every T up to its limit).
constexpr int kDecodeAutoMaxT = kDecodeMaxT;

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shape check shared by every entry point; returns MOVA_OK or an error.
int check_shape(int T, int d, int E, int k) {
  if (T < 0 || d <= 0 || E <= 0 || k <= 0) return MOVA_ERR_INVALID_ARG;
  if (T > kMaxT) return MOVA_ERR_UNSUPPORTED;
  if (E > kMaxExperts || k > kMaxTopK || k > E) return MOVA_ERR_UNSUPPORTED;
  if (d % 64 != 0) return MOVA_ERR_UNSUPPORTED;
  return MOVA_OK;
}

int check_heads(int n_kv_heads, int head_dim) {
  if (n_kv_heads <= 0 || head_dim <= 0) return MOVA_ERR_INVALID_ARG;
  const long long N = (long long)n_kv_heads * head_dim;
  if (N % 64 != 0 || N > (1 << 14)) return MOVA_ERR_UNSUPPORTED;
  return MOVA_OK;
}

enum class Path { Decode, Grouped };

// Kernel-choice overrides (mova_debug_override); largest value per key.
std::atomic<int> g_override[kOvCount];
constexpr int kOverrideMax[kOvCount] = {2, 4, 7, 2, 3, 2, 1};

// Path forced by the kOvPath override: 1 the decode kernel (where T allows
// it), 2 dispatch and the grouped GEMM; 0 when none applies.
int forced_path(int T, Path* p) {
  const int v = override_value(kOvPath);
  if (v == 1 && T <= kDecodeMaxT) { *p = Path::Decode; return 1; }
  if (v == 2) { *p = Path::Grouped; return 1; }
  return 0;
}

Path choose_path(int T, int k) {
  (void)k;
  Path p;
  if (forced_path(T, &p)) return p;
  return T <= kDecodeAutoMaxT ? Path::Decode : Path::Grouped;
}

// The FFN's routed experts take the decode kernel up to 1024 pairs (T = 128
// at k = 8): measured at d = 2560, 100 experts of width 768, it is faster at
// T = 64, level at 128 and slower from 192 on, where the experts average more
// than 15 pairs.  The kOvPath override forces either path, as for the value
// path.
Path choose_ffn_path(int T, int k) {
  Path p;
  if (forced_path(T, &p)) return p;
  return (T <= kDecodeMaxT && (long long)T * k <= 1024) ? Path::Decode : Path::Grouped;
}

// Workspace layout (every region 256-byte aligned):
//   idx [T*k] i32 | w [T*k] f32 | chunk_counts [C*E] i32 | expert_off [E+1] i32 |
//   tile_base [E+1] i32 | plog (small-T router partial logits, T <= kDecodeMaxT
//   only) | perm [T*k] i32 | partial [T*k*N] f16
// C = dispatch chunks at the smallest router workgroup (16 tokens), so that
// the size depends on the shapes alone, whichever router kernel runs.
struct Layout {
  size_t idx, w, chunk, eoff, tbase, plog, perm, partial, total;
};

constexpr int kMinRouterChunk = 16;

Layout layout(int T, int E, int k, int N) {
  const size_t pairs = (size_t)T * k;
  const size_t C = (size_t)ceil_div(T, kMinRouterChunk);
  Layout L;
  size_t o = 0;
  L.idx = o;     o += align256(pairs * 4);
  L.w = o;       o += align256(pairs * 4);
  L.chunk = o;   o += align256(C * E * 4);
  L.eoff = o;    o += align256((size_t)(E + 1) * 4);
  L.tbase = o;   o += align256((size_t)(E + 1) * 4);
  L.plog = o;    o += align256(T <= kDecodeMaxT ? (size_t)router_small_plog_floats(T) * 4 : 0);
  L.perm = o;    o += align256(pairs * 4);
  L.partial = o; o += align256(pairs * N * 2);
  L.total = o;
  return L;
}

// Paged store of the value rows (mova_value_forward_paged).
struct PagedStore {
  void* cache;
  const int64_t* slot;
  int num_blocks, block_size;
};
// Largest pool, in slots, that the paged entry point accepts (a row index
// times N stays far inside 64-bit offsets).
constexpr long long kMaxSlots = 1ll << 40;

// Dense projection: the split-k kernel (with its fp32 partials in the
// workspace) up to kDenseSkinnyMaxT tokens, the tiled GEMM above.
enum class DensePath { Skinny, Tiled };

DensePath choose_dense_path(int T) {
  const bool skinny_ok = T <= kDenseSkinnyMaxT;
  const int v = override_value(kOvDensePath);  // 1 split-k, 2 tiled (tests, measurement)
  if (v == 1 && skinny_ok) return DensePath::Skinny;
  if (v == 2) return DensePath::Tiled;
  return skinny_ok ? DensePath::Skinny : DensePath::Tiled;
}

size_t dense_workspace(int T, int d, int N) {
  return T <= kDenseSkinnyMaxT ? align256(dense_skinny_partial_floats(T, d, N) * 4) : 0;
}

// FFN mixture of experts (mova_ffn_moe_forward).  Domain: 1 <= E <= 128,
// 1 <= k <= min(E, 8), d % 64 == 0 and d <= 16384 (d is also the output
// width), inter % 64 == 0 and 0 < inter <= 16384, inter_shared == 0 (no
// shared expert) or as inter.
int check_ffn(int T, int d, int E, int k, int inter, int inter_shared) {
  if (T < 0 || d <= 0 || E <= 0 || k <= 0 || inter <= 0 || inter_shared < 0)
    return MOVA_ERR_INVALID_ARG;
  if (T > kMaxT || E > kMaxDispatchExperts || k > kMaxTopK || k > E) return MOVA_ERR_UNSUPPORTED;
  if (d % 64 != 0 || d > (1 << 14) || inter % 64 != 0 || inter > (1 << 14))
    return MOVA_ERR_UNSUPPORTED;
  if (inter_shared % 64 != 0 || inter_shared > (1 << 14)) return MOVA_ERR_UNSUPPORTED;
  return MOVA_OK;
}

// FFN workspace (every region 256-byte aligned):
//   idx [T*k] i32 | w [T*k] f32 | chunk_counts [C*E] i32 | expert_off [E+1] |
//   tile_base [E+1] | router partial logits | perm [T*k] i32 |
//   h [T*k, inter] bf16 | partial [T*k, d] f16 |
//   shared h [T, inter_shared] bf16 | shared partial [T, d] f16 |
//   split-k fp32 partials of the shared expert (T <= kDenseSkinnyMaxT only)
// C = ceil(T / ffn_router_chunk_tokens()).
struct FfnLayout {
  size_t idx, w, chunk, eoff, tbase, plog, perm, h, partial, hs, ps, sk, total;
};

FfnLayout ffn_layout(int T, int d, int E, int k, int inter, int inter_shared) {
  const size_t pairs = (size_t)T * k;
  const size_t C = (size_t)ceil_div(T, ffn_router_chunk_tokens());
  FfnLayout L;
  size_t o = 0;
  L.idx = o;     o += align256(pairs * 4);
  L.w = o;       o += align256(pairs * 4);
  L.chunk = o;   o += align256(C * E * 4);
  L.eoff = o;    o += align256((size_t)(E + 1) * 4);
  L.tbase = o;   o += align256((size_t)(E + 1) * 4);
  L.plog = o;    o += align256(ffn_router_plog_floats(T) * 4);
  L.perm = o;    o += align256(pairs * 4);
  L.h = o;       o += align256(pairs * inter * 2);
  L.partial = o; o += align256(pairs * d * 2);
  L.hs = o;      o += align256((size_t)T * inter_shared * 2);
  L.ps = o;      o += align256(inter_shared > 0 ? (size_t)T * d * 2 : 0);
  L.sk = o;
  if (inter_shared > 0 && T <= kDenseSkinnyMaxT)
    o += align256(std::max(dense_skinny_partial_floats(T, d, 2 * inter_shared),
                           dense_skinny_partial_floats(T, inter_shared, d)) * 4);
  L.total = o;
  return L;
}

// ---- stage timing -------------------------------------------------------
constexpr int kStages = 5;
// Library-owned side stream of a device, for work that depends only on the
// call's inputs and can overlap the rest of the call (the FFN's shared
// expert).  It is forked from the caller's stream with an event and joined
// back with another before the results meet, so the call stays ordered on
// the caller's stream as a whole, also under graph capture.  Default
// priority, non-blocking; created on the device's first use and kept until
// the process ends.  The events are reused by every call, so forks and joins
// are enqueued under g_side_mu (enqueueing only: the work itself overlaps).
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
std::vector<SideStream> g_side;  // by device

// The side stream for work ordered after `stream`, or null (run on `stream`
// itself): the kOvSerial override set to 1, a stream of another device than
// the current one, a first use while `stream` is capturing, or a failure to
// create the stream.  Call with g_side_mu held.
SideStream* side_stream_for(hipStream_t stream) {
  if (override_value(kOvSerial) == 1) return nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
  if (stream != nullptr) {
    hipDevice_t sdev = 0;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess || (int)sdev != dev) return nullptr;
  }
  if ((int)g_side.size() <= dev) g_side.resize(dev + 1);
  SideStream& ss = g_side[dev];
  if (ss.s == nullptr) {
    // No stream creation while the caller's stream is being captured (it
    // may invalidate the capture): such a first call runs serially.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
      return nullptr;
    SideStream fresh;
    if (hipStreamCreateWithFlags(&fresh.s, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&fresh.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&fresh.join, hipEventDisableTiming) != hipSuccess) {
      if (fresh.fork != nullptr) (void)hipEventDestroy(fresh.fork);
      (void)hipStreamDestroy(fresh.s);
      return nullptr;
    }
    ss = fresh;
  }
  return &ss;
}

// One fork of side-stream work off the caller's stream, in three steps:
// begin() records the fork on the caller's stream and hands out the stream
// to launch on (the side stream, or the caller's own when there is none),
// end() records the join on it, join() makes the caller's stream wait for
// it.  join() also runs on destruction, so an early return never leaves the
// caller's stream (or a graph being captured) un-joined.  The side stream's
// lock is held from construction to the join.
class SideFork {
 public:
  SideFork(hipStream_t stream, bool wanted) : stream_(stream), lock_(g_side_mu, std::defer_lock) {
    if (!wanted) return;
    lock_.lock();
    side_ = side_stream_for(stream);
    if (side_ == nullptr) lock_.unlock();
  }
  SideFork(const SideFork&) = delete;
  SideFork& operator=(const SideFork&) = delete;
  ~SideFork() { (void)join(); }

  hipError_t begin(hipStream_t* launch_stream) {
    *launch_stream = stream_;
    if (side_ == nullptr) return hipSuccess;
    forked_ = true;
    hipError_t e = hipEventRecord(side_->fork, stream_);
    if (e == hipSuccess) e = hipStreamWaitEvent(side_->s, side_->fork, 0);
    *launch_stream = side_->s;
    return e;
  }
  hipError_t end() {
    return forked_ ? hipEventRecord(side_->join, side_->s) : hipSuccess;
  }
  hipError_t join() {
    if (side_ == nullptr) return hipSuccess;
    hipError_t e = hipSuccess;
    if (forked_) e = hipStreamWaitEvent(stream_, side_->join, 0);
    side_ = nullptr;
    lock_.unlock();
    return e;
  }

 private:
  hipStream_t stream_;
  std::unique_lock<std::mutex> lock_;
  SideStream* side_ = nullptr;
  bool forked_ = false;
};

struct Timing {
  std::mutex mu;
  int capacity = 0;
  unsigned mask = 0;
  std::vector<hipEvent_t> ev[kStages];  // pairs: start at 2i, stop at 2i+1
  int used[kStages] = {0, 0, 0, 0, 0};
} g_timing;

struct StageScope {
  int stage;
  hipStream_t s;
  hipEvent_t stop = nullptr;
  StageScope(int st, hipStream_t stream) : stage(st), s(stream) {
    if (g_timing.capacity <= 0 || !(g_timing.mask & (1u << st))) return;
    std::lock_guard<std::mutex> lk(g_timing.mu);
    const int u = g_timing.used[stage];
    if (u >= g_timing.capacity) return;
    (void)hipEventRecord(g_timing.ev[stage][2 * u], s);
    stop = g_timing.ev[stage][2 * u + 1];
    g_timing.used[stage] = u + 1;
  }
  ~StageScope() {
    if (stop != nullptr) (void)hipEventRecord(stop, s);
  }
};

void timing_free() {
  for (int s = 0; s < kStages; ++s) {
    for (hipEvent_t e : g_timing.ev[s])
      if (e != nullptr) (void)hipEventDestroy(e);
    g_timing.ev[s].clear();
    g_timing.used[s] = 0;
  }
  g_timing.capacity = 0;
  g_timing.mask = 0;
}

// ---- workspace of the entry point that allocates nothing -----------------
//
// mova_value_forward_noalloc takes its workspace from this array instead of
// the caller.  Each device the library runs on holds its own copy, allocated
// with the library's code object and kept until the process ends.  In host
// code `scratch` names a host-side stand-in, not a device address: its
// address on a device comes from hipGetSymbolAddress, taken once per device
// with that device current, and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[MOVA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // by device ordinal; null until first use

// This device's scratch address (looked up on the device's first call), or
// null when the lookup fails.  `dev` must be the current device.
void* device_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();  // clear the sticky error of the failed lookup
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

int mova::override_value(int key) {
  return (key >= 0 && key < kOvCount) ? g_override[key].load(std::memory_order_relaxed) : 0;
}

extern "C" {

int mova_version(void) { return kVersion; }

const char* mova_status_str(int status) {
  switch (status) {
    case MOVA_OK: return "MOVA_OK";
    case MOVA_ERR_INVALID_ARG: return "MOVA_ERR_INVALID_ARG: null/misaligned pointer or negative size";
    case MOVA_ERR_UNSUPPORTED: return "MOVA_ERR_UNSUPPORTED: shape outside the supported domain";
    case MOVA_ERR_WORKSPACE: return "MOVA_ERR_WORKSPACE: workspace missing or too small";
    case MOVA_ERR_HIP: return "MOVA_ERR_HIP: a HIP launch or runtime call failed";
    case MOVA_ERR_SCRATCH:
      return "MOVA_ERR_SCRATCH: the call needs more than the library's static scratch "
             "(MOVA_NOALLOC_SCRATCH_BYTES); use mova_value_forward with a workspace";
    default: return "MOVA: unknown status";
  }
}

size_t mova_workspace_bytes(int T, int d, int E, int k, int n_kv_heads, int head_dim) {
  if (check_shape(T, d, E, k) != MOVA_OK || check_heads(n_kv_heads, head_dim) != MOVA_OK)
    return (size_t)-1;
  if (T == 0) return 0;
  return layout(T, E, k, n_kv_heads * head_dim).total;
}

int mova_route(const void* x, const void* router_w, const float* router_b, int T, int d, int E,
               int k, float scale, int32_t* topk_idx, float* topk_w, hipStream_t stream) {
  int rc = check_shape(T, d, E, k);
  if (rc != MOVA_OK) return rc;
  if (!isfinite(scale)) return MOVA_ERR_UNSUPPORTED;
  if (T == 0) return MOVA_OK;
  if (x == nullptr || router_w == nullptr || topk_idx == nullptr || topk_w == nullptr)
    return MOVA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(router_w) || !aligned16(router_b) || !aligned16(topk_idx) ||
      !aligned16(topk_w))
    return MOVA_ERR_INVALID_ARG;
  RouterArgs ra{(const __bf16*)x, (const __bf16*)router_w, router_b, T, d, E, k, scale,
                topk_idx, topk_w, nullptr};
  // Routing alone has no workspace, so it uses the single-kernel router at
  // every T (same bits as the two-kernel small-T router of the decode path).
  return launch_router_lds(ra, stream) == hipSuccess ? MOVA_OK : MOVA_ERR_HIP;
}

// Shared body of mova_value_forward, mova_value_forward_paged and
// mova_value_from_routing.  `pg` set: the combine also stores each row at its
// slot of the paged pool, and `out` may be null.  `given` set: the routing
// is the caller's (no router; ids outside [0, E) are skipped), router_w,
// router_b and scale are unused.
struct GivenRouting {
  const int32_t* idx;
  const float* w;
};
static int value_forward_impl(const void* x, const void* router_w, const float* router_b,
                              const void* expert_w, int T, int d, int E, int k, float scale,
                              int n_kv_heads, int head_dim, void* out, const PagedStore* pg,
                              int32_t* topk_idx_out, float* topk_w_out, void* workspace,
                              size_t workspace_bytes, hipStream_t stream,
                              const GivenRouting* given = nullptr) {
  int rc = check_shape(T, d, E, k);
  if (rc != MOVA_OK) return rc;
  rc = check_heads(n_kv_heads, head_dim);
  if (rc != MOVA_OK) return rc;
  if (!isfinite(scale)) return MOVA_ERR_UNSUPPORTED;
  if (pg != nullptr && (pg->num_blocks < 0 || pg->block_size <= 0)) return MOVA_ERR_INVALID_ARG;
  if (pg != nullptr && (long long)pg->num_blocks * pg->block_size > kMaxSlots)
    return MOVA_ERR_UNSUPPORTED;
  if (T == 0) return MOVA_OK;
  if (given != nullptr && (given->idx == nullptr || given->w == nullptr)) return MOVA_ERR_INVALID_ARG;
  if (given != nullptr && (!aligned16(given->idx) || !aligned16(given->w)))
    return MOVA_ERR_INVALID_ARG;
  if (x == nullptr || (router_w == nullptr && given == nullptr) || expert_w == nullptr ||
      (out == nullptr && pg == nullptr))
    return MOVA_ERR_INVALID_ARG;
  if (pg != nullptr && (pg->cache == nullptr || pg->slot == nullptr)) return MOVA_ERR_INVALID_ARG;
  if (pg != nullptr && (!aligned16(pg->cache) || ((uintptr_t)pg->slot & 7u) != 0))
    return MOVA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(router_w) || !aligned16(router_b) || !aligned16(expert_w) ||
      !aligned16(out) || !aligned16(topk_idx_out) || !aligned16(topk_w_out))
    return MOVA_ERR_INVALID_ARG;
  const int N = n_kv_heads * head_dim;
  const Layout L = layout(T, E, k, N);
  if (workspace == nullptr || workspace_bytes < L.total) return MOVA_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return MOVA_ERR_INVALID_ARG;

  char* ws = (char*)workspace;
  int32_t* idx = given ? const_cast<int32_t*>(given->idx)
                       : (topk_idx_out ? topk_idx_out : (int32_t*)(ws + L.idx));
  float* w = given ? const_cast<float*>(given->w) : (topk_w_out ? topk_w_out : (float*)(ws + L.w));
  int32_t* chunk = (int32_t*)(ws + L.chunk);
  int32_t* eoff = (int32_t*)(ws + L.eoff);
  int32_t* tbase = (int32_t*)(ws + L.tbase);
  float* plog = (float*)(ws + L.plog);
  int32_t* perm = (int32_t*)(ws + L.perm);
  f16_t* partial = (f16_t*)(ws + L.partial);
  const __bf16* xb = (const __bf16*)x;
  const __bf16* wb = (const __bf16*)expert_w;

  const Path path = choose_path(T, k);
  const bool grouped = path == Path::Grouped;
  const int tok_stages = grouped ? 0 : decode_token_stages(T, d, N, E, k);
  hipError_t err = hipSuccess;
  if (given == nullptr) {
    StageScope sc(0, stream);
    RouterArgs ra{xb, (const __bf16*)router_w, router_b, T, d, E, k, scale, idx, w,
                  grouped ? chunk : nullptr};
    // The token-major kernel selects for its token itself from the partials.
    err = grouped      ? launch_router_lds(ra, stream)
          : tok_stages ? launch_router_partial(ra, plog, stream)
                       : launch_router_small(ra, plog, stream);
  }
  if (err != hipSuccess) return MOVA_ERR_HIP;

  if (path == Path::Decode) {
    StageScope sc(2, stream);
    if (const int stages = tok_stages) {
      // Token-major kernel: the top-k selection (router's partials) and the
      // k-way combine are fused into it.
      DecodeTokenArgs ta{xb, wb, idx, w, (__bf16*)out};
      ta.T = T; ta.d = d; ta.N = N; ta.E = E; ta.k = k;
      if (given == nullptr) {
        ta.plog = plog;
        ta.Tp = ceil_div(T, 16) * 16;
        ta.bias = router_b;
        ta.scale = scale;
      }
      if (pg != nullptr) {
        ta.slot = pg->slot;
        ta.num_slots = (long long)pg->num_blocks * pg->block_size;
        ta.cache = (__bf16*)pg->cache;
      }
      err = launch_decode_token(ta, stages, stream);
      return err == hipSuccess ? MOVA_OK : MOVA_ERR_HIP;
    }
    DecodeArgs da{xb, wb, idx, w, partial, T, d, N, E, k};
    err = launch_decode(da, stream);
  } else {
    const GemmTile tile = gemm_tile_grouped(T, k, E, N);
    {
      StageScope sc(1, stream);
      DispatchArgs dp{idx, chunk, eoff, tbase, perm, T, E, k, router_chunk_tokens(T), tile.bm};
      if (given != nullptr) err = launch_dispatch_count(dp, stream);
      if (err == hipSuccess) err = launch_dispatch(dp, stream);
    }
    if (err != hipSuccess) return MOVA_ERR_HIP;
    StageScope sc(2, stream);
    GemmArgs ga{xb, wb, perm, w, eoff, tbase, partial, nullptr, T, d, N, E, k, tile};
    err = launch_grouped_gemm(ga, stream);
  }
  if (err != hipSuccess) return MOVA_ERR_HIP;
  {
    StageScope sc(3, stream);
    CombineArgs ca{partial, (__bf16*)out, T, N, k};
    if (given != nullptr) {
      ca.idx = given->idx;
      ca.E = E;
    }
    if (pg != nullptr) {
      ca.slot = pg->slot;
      ca.num_slots = (long long)pg->num_blocks * pg->block_size;
      ca.cache = (__bf16*)pg->cache;
    }
    err = launch_combine(ca, stream);
  }
  return err == hipSuccess ? MOVA_OK : MOVA_ERR_HIP;
}

int mova_value_forward(const void* x, const void* router_w, const float* router_b,
                       const void* expert_w, int T, int d, int E, int k, float scale,
                       int n_kv_heads, int head_dim, void* out, int32_t* topk_idx_out,
                       float* topk_w_out, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  return value_forward_impl(x, router_w, router_b, expert_w, T, d, E, k, scale, n_kv_heads,
                            head_dim, out, nullptr, topk_idx_out, topk_w_out, workspace,
                            workspace_bytes, stream);
}

int mova_value_from_routing(const void* x, const int32_t* topk_idx, const float* topk_w,
                            const void* expert_w, int T, int d, int E, int k, int n_kv_heads,
                            int head_dim, void* out, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  const GivenRouting given{topk_idx, topk_w};
  return value_forward_impl(x, nullptr, nullptr, expert_w, T, d, E, k, 1.0f, n_kv_heads, head_dim,
                            out, nullptr, nullptr, nullptr, workspace, workspace_bytes, stream,
                            &given);
}

int mova_value_forward_record(const void* x, const void* router_w, const float* router_b,
                              const void* expert_w, int T, int d, int E, int k, float scale,
                              int n_kv_heads, int head_dim, void* out, uint32_t* record_ids,
                              void* record_w, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  int rc = check_shape(T, d, E, k);
  if (rc != MOVA_OK) return rc;
  if (k > kRecordMaxK) return MOVA_ERR_UNSUPPORTED;
  rc = check_heads(n_kv_heads, head_dim);
  if (rc != MOVA_OK) return rc;
  if (T > 0 && (record_ids == nullptr || record_w == nullptr)) return MOVA_ERR_INVALID_ARG;
  if (((uintptr_t)record_ids & 3u) != 0 || ((uintptr_t)record_w & 1u) != 0)
    return MOVA_ERR_INVALID_ARG;
  rc = value_forward_impl(x, router_w, router_b, expert_w, T, d, E, k, scale, n_kv_heads, head_dim,
                          out, nullptr, nullptr, nullptr, workspace, workspace_bytes, stream);
  if (rc != MOVA_OK || T == 0) return rc;
  // The routing the call used sits in the workspace (no routing outputs were
  // requested); pack it.
  const Layout L = layout(T, E, k, n_kv_heads * head_dim);
  char* ws = (char*)workspace;
  return launch_record_pack((const int32_t*)(ws + L.idx), (const float*)(ws + L.w), T, k,
                            record_ids, (f16_t*)record_w, stream) == hipSuccess
             ? MOVA_OK
             : MOVA_ERR_HIP;
}

int mova_value_from_record(const void* x, const uint32_t* record_ids, const void* record_w,
                           const void* expert_w, int T, int d, int E, int k, int n_kv_heads,
                           int head_dim, void* out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  int rc = check_shape(T, d, E, k);
  if (rc != MOVA_OK) return rc;
  if (k > kRecordMaxK) return MOVA_ERR_UNSUPPORTED;
  rc = check_heads(n_kv_heads, head_dim);
  if (rc != MOVA_OK) return rc;
  if (T == 0) return MOVA_OK;
  if (record_ids == nullptr || record_w == nullptr) return MOVA_ERR_INVALID_ARG;
  if (((uintptr_t)record_ids & 3u) != 0 || ((uintptr_t)record_w & 1u) != 0)
    return MOVA_ERR_INVALID_ARG;
  const Layout L = layout(T, E, k, n_kv_heads * head_dim);
  if (workspace == nullptr || workspace_bytes < L.total) return MOVA_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return MOVA_ERR_INVALID_ARG;
  if (x == nullptr || expert_w == nullptr || out == nullptr) return MOVA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(expert_w) || !aligned16(out)) return MOVA_ERR_INVALID_ARG;
  // Unpack into the workspace's routing regions (unused when the routing is
  // given), then rebuild as mova_value_from_routing does.
  char* ws = (char*)workspace;
  int32_t* idx = (int32_t*)(ws + L.idx);
  float* w = (float*)(ws + L.w);
  if (launch_record_unpack(record_ids, (const f16_t*)record_w, T, k, idx, w, stream) != hipSuccess)
    return MOVA_ERR_HIP;
  const GivenRouting given{idx, w};
  return value_forward_impl(x, nullptr, nullptr, expert_w, T, d, E, k, 1.0f, n_kv_heads, head_dim,
                            out, nullptr, nullptr, nullptr, workspace, workspace_bytes, stream,
                            &given);
}

int mova_value_forward_paged(const void* x, const void* router_w, const float* router_b,
                             const void* expert_w, int T, int d, int E, int k, float scale,
                             int n_kv_heads, int head_dim, void* v_cache, int num_blocks,
                             int block_size, const int64_t* slot_mapping, void* out,
                             int32_t* topk_idx_out, float* topk_w_out, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  const PagedStore pg{v_cache, slot_mapping, num_blocks, block_size};
  return value_forward_impl(x, router_w, router_b, expert_w, T, d, E, k, scale, n_kv_heads,
                            head_dim, out, &pg, topk_idx_out, topk_w_out, workspace,
                            workspace_bytes, stream);
}

int mova_value_forward_noalloc(const void* x, const void* router_w, const float* router_b,
                               const void* expert_w, int T, int d, int E, int k, float scale,
                               int n_kv_heads, int head_dim, void* out, int32_t* topk_idx_out,
                               float* topk_w_out, hipStream_t stream) {
  // Host-side checks first: nothing is looked up or enqueued for a call that
  // fails them.
  int rc = check_shape(T, d, E, k);
  if (rc != MOVA_OK) return rc;
  rc = check_heads(n_kv_heads, head_dim);
  if (rc != MOVA_OK) return rc;
  if (T == 0) return MOVA_OK;
  const size_t need = layout(T, E, k, n_kv_heads * head_dim).total;
  if (need > (size_t)MOVA_NOALLOC_SCRATCH_BYTES) return MOVA_ERR_SCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOVA_ERR_HIP;
  if (stream != nullptr) {
    hipDevice_t sdev = 0;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return MOVA_ERR_HIP;
    if ((int)sdev != dev) return MOVA_ERR_INVALID_ARG;
  }
  void* ws = device_scratch(dev);
  if (ws == nullptr) return MOVA_ERR_HIP;
  return value_forward_impl(x, router_w, router_b, expert_w, T, d, E, k, scale, n_kv_heads,
                            head_dim, out, nullptr, topk_idx_out, topk_w_out, ws,
                            (size_t)MOVA_NOALLOC_SCRATCH_BYTES, stream);
}

size_t mova_dense_workspace_bytes(int T, int d, int n_kv_heads, int head_dim) {
  if (T < 0 || d <= 0 || T > kMaxT || d % 64 != 0) return (size_t)-1;
  if (check_heads(n_kv_heads, head_dim) != MOVA_OK) return (size_t)-1;
  if (T == 0) return 0;
  return dense_workspace(T, d, n_kv_heads * head_dim);
}

int mova_dense_value_proj(const void* x, const void* w_v, int T, int d, int n_kv_heads,
                          int head_dim, void* out, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  if (T < 0 || d <= 0) return MOVA_ERR_INVALID_ARG;
  if (T > kMaxT || d % 64 != 0) return MOVA_ERR_UNSUPPORTED;
  int rc = check_heads(n_kv_heads, head_dim);
  if (rc != MOVA_OK) return rc;
  if (T == 0) return MOVA_OK;
  if (x == nullptr || w_v == nullptr || out == nullptr) return MOVA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_v) || !aligned16(out)) return MOVA_ERR_INVALID_ARG;
  const int N = n_kv_heads * head_dim;
  const DensePath path = choose_dense_path(T);
  hipError_t err;
  if (path == DensePath::Skinny) {
    if (workspace == nullptr || workspace_bytes < dense_workspace(T, d, N)) return MOVA_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return MOVA_ERR_INVALID_ARG;
    StageScope sc(4, stream);
    DenseArgs da{(const __bf16*)x, (const __bf16*)w_v, (float*)workspace, (__bf16*)out, T, d, N};
    err = launch_dense_skinny(da, stream);
  } else {
    StageScope sc(4, stream);
    GemmArgs ga{(const __bf16*)x, (const __bf16*)w_v, nullptr, nullptr, nullptr, nullptr,
                nullptr, (__bf16*)out, T, d, N, 1, 1, {0, 0, 0, 0}, kGemmDense};
    err = launch_dense_gemm(ga, stream);
  }
  return err == hipSuccess ? MOVA_OK : MOVA_ERR_HIP;
}

size_t mova_ffn_workspace_bytes(int T, int d, int E, int k, int inter, int inter_shared) {
  if (check_ffn(T, d, E, k, inter, inter_shared) != MOVA_OK) return (size_t)-1;
  if (T == 0) return 0;
  return ffn_layout(T, d, E, k, inter, inter_shared).total;
}

int mova_ffn_pack_gate_up(const void* gate_w, const void* up_w, int E, int inter, int d,
                          void* gate_up_w, hipStream_t stream) {
  if (E <= 0 || inter <= 0 || d <= 0) return MOVA_ERR_INVALID_ARG;
  if (E > kMaxDispatchExperts || inter % 64 != 0 || inter > (1 << 14) || d % 64 != 0 ||
      d > (1 << 14))
    return MOVA_ERR_UNSUPPORTED;
  if (gate_w == nullptr || up_w == nullptr || gate_up_w == nullptr) return MOVA_ERR_INVALID_ARG;
  if (!aligned16(gate_w) || !aligned16(up_w) || !aligned16(gate_up_w)) return MOVA_ERR_INVALID_ARG;
  return launch_ffn_pack_gate_up((const __bf16*)gate_w, (const __bf16*)up_w, (__bf16*)gate_up_w, E,
                                 inter, d, stream) == hipSuccess
             ? MOVA_OK
             : MOVA_ERR_HIP;
}

int mova_ffn_moe_forward(const void* x, const void* router_w, const float* router_b,
                         const void* gate_up_w, const void* down_w, int E, int k, int inter,
                         const void* shared_gate_up_w, const void* shared_down_w,
                         int inter_shared, int T, int d, float scale, void* out,
                         int32_t* topk_idx_out, float* topk_w_out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  int rc = check_ffn(T, d, E, k, inter, inter_shared);
  if (rc != MOVA_OK) return rc;
  if (!isfinite(scale)) return MOVA_ERR_UNSUPPORTED;
  if (T == 0) return MOVA_OK;
  if (x == nullptr || router_w == nullptr || gate_up_w == nullptr || down_w == nullptr ||
      out == nullptr)
    return MOVA_ERR_INVALID_ARG;
  if (inter_shared > 0 && (shared_gate_up_w == nullptr || shared_down_w == nullptr))
    return MOVA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(router_w) || !aligned16(router_b) || !aligned16(gate_up_w) ||
      !aligned16(down_w) || !aligned16(shared_gate_up_w) || !aligned16(shared_down_w) ||
      !aligned16(out) || !aligned16(topk_idx_out) || !aligned16(topk_w_out))
    return MOVA_ERR_INVALID_ARG;
  const FfnLayout L = ffn_layout(T, d, E, k, inter, inter_shared);
  if (workspace == nullptr || workspace_bytes < L.total) return MOVA_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return MOVA_ERR_INVALID_ARG;

  char* ws = (char*)workspace;
  int32_t* idx = topk_idx_out ? topk_idx_out : (int32_t*)(ws + L.idx);
  float* w = topk_w_out ? topk_w_out : (float*)(ws + L.w);
  int32_t* chunk = (int32_t*)(ws + L.chunk);
  int32_t* eoff = (int32_t*)(ws + L.eoff);
  int32_t* tbase = (int32_t*)(ws + L.tbase);
  int32_t* perm = (int32_t*)(ws + L.perm);
  __bf16* h = (__bf16*)(ws + L.h);
  f16_t* partial = (f16_t*)(ws + L.partial);
  __bf16* hs = (__bf16*)(ws + L.hs);
  f16_t* ps = (f16_t*)(ws + L.ps);
  const __bf16* xb = (const __bf16*)x;
  hipError_t err = hipSuccess;

  // The shared expert depends on x alone: it runs first, on the side stream
  // when there is one, overlapping the router and the routed experts.  Its
  // buffers (hs, ps, sk) are its own.
  SideFork fork(stream, inter_shared > 0);
  if (inter_shared > 0) {
    hipStream_t ss = stream;
    err = fork.begin(&ss);
    if (err == hipSuccess && T <= kDenseSkinnyMaxT) {
      // Few tokens: the weight-streaming split-k kernel, whose reduction
      // applies the SwiGLU (gate/up) or rounds to fp16 (down).
      float* sk = (float*)(ws + L.sk);
      DenseArgs sg{xb, (const __bf16*)shared_gate_up_w, sk, nullptr, T, d, 2 * inter_shared,
                   kDenseOutSwiGLU, hs};
      err = launch_dense_skinny(sg, ss);
      if (err == hipSuccess) {
        DenseArgs sd{hs, (const __bf16*)shared_down_w, sk, nullptr, T, inter_shared, d,
                     kDenseOutF16, ps};
        err = launch_dense_skinny(sd, ss);
      }
    } else if (err == hipSuccess) {
      GemmArgs sg{xb, (const __bf16*)shared_gate_up_w, nullptr, nullptr, nullptr, nullptr,
                  nullptr, hs, T, d, 2 * inter_shared, 1, 1, {0, 0, 0, 0}, kGemmDenseSwiGLU};
      err = launch_dense_gemm(sg, ss);
      if (err == hipSuccess) {
        GemmArgs sd{hs, (const __bf16*)shared_down_w, nullptr, nullptr, nullptr, nullptr, ps,
                    nullptr, T, inter_shared, d, 1, 1, {0, 0, 0, 0}, kGemmDenseF16};
        err = launch_dense_gemm(sd, ss);
      }
    }
    const hipError_t e = fork.end();
    if (err == hipSuccess) err = e;
  }
  if (err != hipSuccess) return MOVA_ERR_HIP;
  {
    StageScope sc(0, stream);
    RouterArgs ra{xb, (const __bf16*)router_w, router_b, T, d, E, k, scale, idx, w, chunk};
    err = launch_ffn_router(ra, (float*)(ws + L.plog), stream);
  }
  if (err != hipSuccess) return MOVA_ERR_HIP;
  const bool decode = choose_ffn_path(T, k) == Path::Decode;
  const GemmTile tile = gemm_tile_grouped_ffn(T, k, E);
  if (!decode) {
    StageScope sc(1, stream);
    DispatchArgs dp{idx, chunk, eoff, tbase, perm, T, E, k, ffn_router_chunk_tokens(), tile.bm};
    err = launch_dispatch(dp, stream);
  }
  if (err != hipSuccess) return MOVA_ERR_HIP;
  {
    StageScope sc(2, stream);
    // Routed experts: h[pair] = SiLU(gate x) * (up x), then partial[pair] =
    // w * (down h).  Few tokens: the weight-streaming decode kernel, which finds each
    // expert's pairs itself (no dispatch); else the grouped GEMM.
    if (decode) {
      DecodeArgs gu{xb, (const __bf16*)gate_up_w, idx, w, nullptr, T, d, 2 * inter, E, k};
      gu.mode = kGemmRoutedSwiGLU;
      gu.out_h = h;
      err = launch_decode(gu, stream);
      if (err == hipSuccess) {
        DecodeArgs dn{h, (const __bf16*)down_w, idx, w, partial, T, inter, d, E, k};
        dn.mode = kGemmRoutedLinear;
        err = launch_decode(dn, stream);
      }
    } else {
      GemmArgs gu{xb, (const __bf16*)gate_up_w, perm, w, eoff, tbase, nullptr, h,
                  T, d, 2 * inter, E, k, tile, kGemmRoutedSwiGLU};
      err = launch_grouped_gemm(gu, stream);
      if (err == hipSuccess) {
        GemmArgs dn{h, (const __bf16*)down_w, perm, w, eoff, tbase, partial, nullptr,
                    T, inter, d, E, k, tile, kGemmRoutedLinear};
        err = launch_grouped_gemm(dn, stream);
      }
    }
  }
  if (err == hipSuccess) err = fork.join();
  if (err != hipSuccess) return MOVA_ERR_HIP;
  {
    StageScope sc(3, stream);
    CombineArgs ca{partial, (__bf16*)out, T, d, k};
    ca.extra = inter_shared > 0 ? ps : nullptr;
    err = launch_combine(ca, stream);
  }
  return err == hipSuccess ? MOVA_OK : MOVA_ERR_HIP;
}

int mova_debug_override(int key, int value) {
  if (key < 0 || key >= kOvCount || value < 0 || value > kOverrideMax[key])
    return MOVA_ERR_INVALID_ARG;
  g_override[key].store(value, std::memory_order_relaxed);
  return MOVA_OK;
}

int mova_debug_override_get(int key) {
  return (key >= 0 && key < kOvCount) ? g_override[key].load(std::memory_order_relaxed) : -1;
}

int mova_timing_enable(int capacity, unsigned stage_mask) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  timing_free();
  stage_mask &= (1u << kStages) - 1;
  if (capacity <= 0 || stage_mask == 0) return MOVA_OK;
  for (int s = 0; s < kStages; ++s) {
    if (!(stage_mask & (1u << s))) continue;
    g_timing.ev[s].resize(2 * (size_t)capacity, nullptr);
    for (auto& e : g_timing.ev[s]) {
      // Timing-only events: no system-scope fence around the stage, so the
      // event pair brackets the kernels without a cache writeback of its own.
      if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
        e = nullptr;
        timing_free();
        return MOVA_ERR_HIP;
      }
    }
  }
  g_timing.capacity = capacity;
  g_timing.mask = stage_mask;
  return MOVA_OK;
}

int mova_timing_read(int n, double* total_ms, int* count) {
  if (n < 0 || (n > 0 && (total_ms == nullptr || count == nullptr))) return MOVA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_timing.mu);
  for (int s = 0; s < n; ++s) {
    total_ms[s] = 0.0;
    count[s] = 0;
    if (s >= kStages) continue;
    for (int u = 0; u < g_timing.used[s]; ++u) {
      hipEvent_t a = g_timing.ev[s][2 * u], b = g_timing.ev[s][2 * u + 1];
      if (hipEventSynchronize(b) != hipSuccess) return MOVA_ERR_HIP;
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, a, b) != hipSuccess) return MOVA_ERR_HIP;
      total_ms[s] += ms;
    }
    count[s] = g_timing.used[s];
  }
  return MOVA_OK;
}

}  // extern "C"
