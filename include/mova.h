/*
 * mova.h -- C ABI of the MoVA routed value projection for MI355X (gfx950).
 *
 * MoVA replaces an attention layer's value projection with a router and E
 * value experts (page "MoVA: routing the value vectors, and why the KV cache
 * does not notice", section "Where the routing happens"): per token, logits
 * = x Wr^T (router weight only), sigmoid scores, the k experts with the
 * highest selection score are kept, their scores are divided by their sum and
 * multiplied by `scale`, each kept expert's output goes through SiLU, and the
 * weighted sum is one [n_kv_heads, head_dim] value vector per token -- the
 * shape a plain GQA value projection produces.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers (HIP device memory), row-major
 *   and contiguous, 16-byte aligned.  The caller owns every buffer; the
 *   library never allocates, frees or synchronises device memory.
 * - bf16 means IEEE bfloat16 stored in 2 bytes; float means IEEE fp32.
 * - Work is enqueued asynchronously on `stream` (NULL = the null stream).
 *   Calls are stateless: concurrent calls need distinct outputs and
 *   workspaces.
 * - Return value: MOVA_OK or a negative mova_status.  Argument errors are
 *   detected on the host before anything is enqueued, so outputs are left
 *   untouched.  A failed kernel launch returns MOVA_ERR_HIP.
 * - T == 0 returns MOVA_OK and enqueues nothing.
 * - Supported domain: 1 <= E <= 64, 1 <= k <= min(E, 8), d > 0 and
 *   d % 64 == 0, N = n_kv_heads * head_dim with 0 < N <= 16384 and
 *   N % 64 == 0, 0 <= T <= 2^24, scale finite.
 *
 * Reading of the router bias (the pages pass it separately and do not show
 * where it enters): the bias is added to the sigmoid scores to choose the k
 * experts; the weights are computed from the unbiased scores.  Ties in the
 * selection score go to the lower expert index, and the k selected experts
 * are reported in order of (selection score desc, index asc).
 */
#ifndef MOVA_H
#define MOVA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t; /* identical to hip_runtime_api.h */

enum mova_status {
  MOVA_OK = 0,
  MOVA_ERR_INVALID_ARG = -1, /* null pointer, negative size, misaligned pointer */
  MOVA_ERR_UNSUPPORTED = -2, /* shape outside the supported domain */
  MOVA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than mova_workspace_bytes */
  MOVA_ERR_HIP = -4,         /* a HIP launch or runtime call failed */
  MOVA_ERR_SCRATCH = -5      /* mova_value_forward_noalloc: shapes need more than its scratch */
};

/* Version of this ABI (major * 10000 + minor * 100 + patch). */
int mova_version(void);

/* Human-readable name of a status code; never NULL, static storage. */
const char* mova_status_str(int status);

/*
 * Bytes of device workspace mova_value_forward needs for these sizes; 0 when
 * T == 0, and (size_t)-1 when the sizes are outside the supported domain.
 * Depends only on the sizes, never on the data.
 */
size_t mova_workspace_bytes(int T, int d, int E, int k, int n_kv_heads, int head_dim);

/*
 * Routing only: the router linear map, sigmoid, bias-for-selection, top-k,
 * renormalisation and scaling (section "Where the routing happens": the
 * router logits line and calc_router_weights with "sigmoid", top_k and
 * scaling_factor).
 *
 *   x        bf16  [T, d]   tokens
 *   router_w bf16  [E, d]   router weight (nn.Linear layout)
 *   router_b float [E]      router bias, NULL = zeros
 *   topk_idx int32 [T, k]   out: selected experts, ordered as above
 *   topk_w   float [T, k]   out: weights, sum over k equals `scale`
 *
 * Logits are accumulated in fp32 from the bf16 products.
 */
int mova_route(const void* x, const void* router_w, const float* router_b,
               int T, int d, int E, int k, float scale,
               int32_t* topk_idx, float* topk_w, hipStream_t stream);

/*
 * Full value projection (section "Where the routing happens": routing, then
 * combine_routed_experts with F.silu, then the view as heads of 128):
 *
 *   out[t, h, j] = sum_{i<k} w[t,i] * SiLU( sum_c x[t,c] * expert_w[idx[t,i], h*head_dim + j, c] )
 *
 *   x            bf16  [T, d]
 *   router_w     bf16  [E, d]
 *   router_b     float [E]          NULL = zeros
 *   expert_w     bf16  [E, N, d]    stacked bias-free experts, N = n_kv_heads*head_dim
 *   out          bf16  [T, n_kv_heads, head_dim]   (= [T, N] row-major)
 *   topk_idx_out int32 [T, k]       optional (NULL): the routing used
 *   topk_w_out   float [T, k]       optional (NULL)
 *   workspace    device scratch of at least mova_workspace_bytes(...) bytes,
 *                256-byte aligned; its contents on entry do not matter.
 *
 * Expert products accumulate in fp32; SiLU and the routing weight are applied
 * in fp32 and each slot's result is kept as fp16 (rounded to nearest even);
 * the k-way sum is fp32 in a fixed slot order (i = 0..k-1), rounded once to
 * bf16 (nearest even).  Range: the fp16 slot value holds |w * SiLU(z)| up to
 * 65504 (the largest finite fp16); a slot beyond it becomes +-inf, and so does
 * its token's output row element, although the sum itself would fit bf16.
 * The value layer's own scales stay far below (|out| < 8 on the workloads).  Results are bitwise reproducible for identical inputs and do not
 * depend on how the tokens are split across calls.
 */
int mova_value_forward(const void* x, const void* router_w, const float* router_b,
                       const void* expert_w, int T, int d, int E, int k, float scale,
                       int n_kv_heads, int head_dim, void* out,
                       int32_t* topk_idx_out, float* topk_w_out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The same value projection with the result stored straight into a paged
 * value cache: the routed vector of each token is what the cache keeps
 * (page "IFM K2 Horizon Deep Dive: Inside Mixture-of-Value Attention (MoVA)
 * ...", section "The Two Architectural Caching Strategies for MoVA", Option
 * A, the post-routing projected value cache in the ordinary paged-attention
 * pools; page "MoVA: routing the value vectors ...", section "Where the
 * routing happens", hands that [n_kv_heads, head_dim] vector to the cache
 * update).  The k-way combine writes each row once to the pool, and to `out`
 * as well when `out` is not NULL, so the cache store costs no extra pass.
 *
 *   v_cache      bf16  [num_blocks, block_size, n_kv_heads, head_dim]
 *                the pool; slot s is row s % block_size of block
 *                s / block_size, i.e. the s-th [n_kv_heads, head_dim] row
 *   slot_mapping int64 [T]  slot of each token; a slot outside
 *                [0, num_blocks * block_size) -- e.g. -1 for padding --
 *                stores nothing.  8-byte aligned.
 *   out          bf16  [T, n_kv_heads, head_dim] or NULL
 *   other arguments, workspace and numerics as for mova_value_forward (the
 *   pool rows get exactly the bits `out` gets).
 *
 * Rows of the pool that no token's slot names are left untouched.  Two
 * tokens naming the same slot race: that row's contents are unspecified.
 * Returns MOVA_ERR_INVALID_ARG for num_blocks < 0, block_size <= 0, a NULL
 * or misaligned v_cache or slot_mapping (T > 0), MOVA_ERR_UNSUPPORTED for a
 * pool of more than 2^40 slots; otherwise as mova_value_forward.
 */
int mova_value_forward_paged(const void* x, const void* router_w, const float* router_b,
                             const void* expert_w, int T, int d, int E, int k, float scale,
                             int n_kv_heads, int head_dim, void* v_cache, int num_blocks,
                             int block_size, const int64_t* slot_mapping, void* out,
                             int32_t* topk_idx_out, float* topk_w_out,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Value vectors rebuilt from stored routing: the expert projection, SiLU,
 * weighting and k-way combine of mova_value_forward, with the routing given
 * instead of computed (no router).  This is the reconstruction step of the
 * compact cache of page "IFM K2 Horizon Deep Dive: Inside Mixture-of-Value
 * Attention (MoVA) ...", section "The Two Architectural Caching Strategies
 * for MoVA", Option B, which keeps a token's input x_t with its top-4 expert
 * ids and 4 weights and materialises the value vector when it is needed:
 *
 *   out[t, h, j] = sum over i < k with 0 <= topk_idx[t,i] < E of
 *                  topk_w[t,i] * SiLU( sum_c x[t,c] * expert_w[topk_idx[t,i], h*head_dim + j, c] )
 *
 *   x        bf16  [T, d]    the stored inputs
 *   topk_idx int32 [T, k]    stored expert ids; an id outside [0, E) marks an
 *                            unused slot, which adds nothing (so does a 0 weight)
 *   topk_w   float [T, k]    stored weights (widen fp16 weights to float)
 *   expert_w, out, workspace (mova_workspace_bytes) as for mova_value_forward.
 *
 * Ids may repeat within a token (each slot counts).  Numerics as for
 * mova_value_forward; fed the routing that mova_value_forward reported, it
 * returns the same bits.  Errors as for mova_value_forward (topk_idx and
 * topk_w are required, 16-byte aligned).
 */
int mova_value_from_routing(const void* x, const int32_t* topk_idx, const float* topk_w,
                            const void* expert_w, int T, int d, int E, int k, int n_kv_heads,
                            int head_dim, void* out, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * mova_value_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, kernels, numerics and results (bit for bit) as
 * mova_value_forward, without the workspace: the call takes its scratch from
 * a static device array of MOVA_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on each device it runs on, from that device's first use until the
 * process ends.  It calls no allocating routine.
 *
 * - Size limit: shapes whose mova_workspace_bytes(...) exceeds
 *   MOVA_NOALLOC_SCRATCH_BYTES return MOVA_ERR_SCRATCH before anything is
 *   enqueued (at d = 2560, E = 64, k = 4, N = 1024 that is T up to about
 *   6100 tokens; the scratch is 48 MiB).
 * - The scratch's contents on entry do not matter (each call writes what it
 *   reads); it keeps the last call's contents.
 * - Calls that overlap on one device share its one scratch array and race:
 *   the caller orders them (one stream, or events between streams).
 * - `stream` must belong to the current device (else MOVA_ERR_INVALID_ARG);
 *   NULL is the current device's null stream.
 * - Other errors as for mova_value_forward (MOVA_ERR_HIP also when the
 *   scratch's device address cannot be looked up).
 */
#define MOVA_NOALLOC_SCRATCH_BYTES (48u << 20)

int mova_value_forward_noalloc(const void* x, const void* router_w, const float* router_b,
                               const void* expert_w, int T, int d, int E, int k, float scale,
                               int n_kv_heads, int head_dim, void* out,
                               int32_t* topk_idx_out, float* topk_w_out, hipStream_t stream);

/*
 * Compact routing record of the compact value cache (page "IFM K2 Horizon
 * Deep Dive: Inside Mixture-of-Value Attention (MoVA) ...", section "The Two
 * Architectural Caching Strategies for MoVA", Option B, which keeps a token's
 * x_t with its top-4 expert ids and four fp16 weights and rebuilds v_t from
 * them).  Layout, per token t:
 *
 *   record_ids uint32 [T]     slot j's expert id in bits [6j, 6j + 6), j < k
 *                             (k <= 5; E <= 64 ids fit 6 bits); higher bits 0
 *   record_w   fp16   [T, k]  slot j's routing weight, IEEE binary16, rounded
 *                             to nearest even from the fp32 weight
 *
 * 4 + 2k bytes per token (12 at k = 4), stored beside the token's x_t.  The
 * page's "16-bit mask" cannot hold four ids out of 64, so the ids take one
 * 32-bit word.  record_ids must be 4-byte aligned, record_w 2-byte aligned.
 */

/*
 * mova_value_forward that also writes each token's compact routing record
 * (the routing the call used, packed as above).  Same arguments, workspace,
 * numerics and outputs as mova_value_forward otherwise.  k > 5 returns
 * MOVA_ERR_UNSUPPORTED; a NULL or misaligned record pointer (T > 0) returns
 * MOVA_ERR_INVALID_ARG, before anything is enqueued.
 */
int mova_value_forward_record(const void* x, const void* router_w, const float* router_b,
                              const void* expert_w, int T, int d, int E, int k, float scale,
                              int n_kv_heads, int head_dim, void* out, uint32_t* record_ids,
                              void* record_w, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * Value vectors rebuilt from stored x_t and stored compact records: the
 * records unpacked (ids, fp16 weights widened exactly to fp32), then exactly
 * mova_value_from_routing -- the same kernels, the same bits as
 * mova_value_from_routing given the unpacked routing.  An id >= E (possible
 * only when E < 64) marks an unused slot; so does a zero weight.
 *
 *   x          bf16 [T, d]; record_ids, record_w as above; expert_w, out,
 *   workspace (mova_workspace_bytes) as for mova_value_forward.
 *
 * k > 5 returns MOVA_ERR_UNSUPPORTED; otherwise errors as for
 * mova_value_from_routing.
 */
int mova_value_from_record(const void* x, const uint32_t* record_ids, const void* record_w,
                           const void* expert_w, int T, int d, int E, int k, int n_kv_heads,
                           int head_dim, void* out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Bytes of device workspace mova_dense_value_proj needs for these sizes: 0
 * when T == 0 or T > 256, (size_t)-1 outside the supported domain (that of
 * mova_value_forward without the router's E and k).
 */
size_t mova_dense_workspace_bytes(int T, int d, int n_kv_heads, int head_dim);

/*
 * Plain (dense) GQA value projection, the matched baseline of the routed
 * projection: the model's first dense layers keep an ordinary v_proj, a
 * single bias-free d -> n_kv_heads*head_dim linear map (page "MoVA: routing
 * the value vectors ...", section "So what does it cost?", which sets the
 * 2.62M-parameter v_proj (2560 x 1024) against the routed experts; its
 * section "The take" lists a decode kernel measured against a matched GQA
 * baseline on the same hardware among the things wanted next):
 *
 *   out[t, h, j] = sum_c x[t, c] * w_v[h*head_dim + j, c]
 *
 *   x          bf16 [T, d]
 *   w_v        bf16 [N, d]     nn.Linear layout, N = n_kv_heads*head_dim
 *   out        bf16 [T, n_kv_heads, head_dim]
 *   workspace  device scratch of at least mova_dense_workspace_bytes(...)
 *              bytes, 256-byte aligned (may be NULL when that is 0).
 *
 * Products accumulate in fp32 and each output is rounded once to bf16
 * (nearest even).  Up to 256 tokens the weight is split over d among many
 * workgroups (fp32 partials in the workspace, added in a fixed order);
 * larger T runs the tiled MFMA GEMM.  Results are bitwise reproducible for
 * identical inputs.  Errors as for mova_value_forward.
 */
int mova_dense_value_proj(const void* x, const void* w_v, int T, int d, int n_kv_heads,
                          int head_dim, void* out, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * FFN mixture of experts on the same kernels as the value path (the
 * weight-streaming decode kernel up to T * k = 1024 pairs, else dispatch and
 * the tiled GEMM; both give the same bits): the
 * sparse FFN the model runs beside its routed value projection, 100 experts
 * with top-8 routing plus one shared expert (the thevalue.engineering page
 * on the MoVA architecture, section "Dual sparsity").  The pages give neither
 * the FFN expert shape nor its routing function; readings taken here:
 *   - SwiGLU experts, down( SiLU(gate x) * (up x) ), bias-free, of width
 *     `inter` (routed) and `inter_shared` (shared; 0 = no shared expert);
 *   - routing by the value router's function (sigmoid scores, bias added for
 *     selection, top-k, scores renormalised and multiplied by `scale`);
 *   - out = sum_i w_i * expert_{idx_i}(x) + shared(x), one [d] row per token.
 *
 *   x                bf16  [T, d]
 *   router_w         bf16  [E, d];  router_b float [E] or NULL
 *   gate_up_w        bf16  [E, 2*inter, d]  gate and up rows interleaved in
 *                    blocks of 16 (see mova_ffn_pack_gate_up)
 *   down_w           bf16  [E, d, inter]
 *   shared_gate_up_w bf16  [2*inter_shared, d] (interleaved the same way)
 *   shared_down_w    bf16  [d, inter_shared]
 *   out              bf16  [T, d]
 *   topk_idx_out / topk_w_out  int32 / float [T, k], optional
 *   workspace        >= mova_ffn_workspace_bytes(...) bytes, 256-byte aligned
 *
 * Domain: 1 <= E <= 128, 1 <= k <= min(E, 8), d % 64 == 0 and d <= 16384,
 * inter and inter_shared multiples of 64 up to 16384 (inter > 0), T <= 2^24.
 * Numerics: products accumulate in fp32; SiLU(gate) * up is rounded once to
 * bf16 (the down projection's MFMA operand); each routed slot's w * down(h)
 * and the shared expert's output are kept as fp16; the sum is fp32 in slot
 * order, the shared term last, rounded once to bf16.  Logits for the top-k
 * are fp32: four MFMA chains per (token, expert) over the k steps of each
 * residue class mod 4, in order, added in class order.  Results are bitwise
 * reproducible for identical inputs.  A token's row does not depend on the
 * other tokens of the call, except that the shared expert runs a split-k
 * kernel up to T = 256 and the tiled GEMM above, which sum in different
 * orders (rows agree to rounding across that boundary).  Errors as for
 * mova_value_forward.
 * Streams: the shared expert depends on x alone and runs on a stream the
 * library owns for the current device (created on first use, default
 * priority, kept until the process ends), forked from `stream` with an event
 * at the start of the call and joined back before the results are combined.
 * The call is therefore ordered on `stream` as a whole, also when `stream` is
 * being captured into a graph.  The side stream is not used when `stream`
 * belongs to another device than the current one, when its first use would
 * fall inside a capture, or while MOVA_OVERRIDE_SERIAL is set.  Calls
 * from several host threads are safe; their shared experts share the one
 * side stream.
 */
size_t mova_ffn_workspace_bytes(int T, int d, int E, int k, int inter, int inter_shared);

/*
 * gate_up_w[e, 32b + j] = gate_w[e, 16b + j] and gate_up_w[e, 32b + 16 + j] =
 * up_w[e, 16b + j] for j < 16: the row order the FFN forward reads.  gate_w
 * and up_w are bf16 [E, inter, d] (nn.Linear layout); gate_up_w is bf16
 * [E, 2*inter, d] and must not overlap them.  Pass E = 1 for the shared
 * expert.  Domain as mova_ffn_moe_forward; returns MOVA_OK or an error.
 */
int mova_ffn_pack_gate_up(const void* gate_w, const void* up_w, int E, int inter, int d,
                          void* gate_up_w, hipStream_t stream);

int mova_ffn_moe_forward(const void* x, const void* router_w, const float* router_b,
                         const void* gate_up_w, const void* down_w, int E, int k, int inter,
                         const void* shared_gate_up_w, const void* shared_down_w,
                         int inter_shared, int T, int d, float scale, void* out,
                         int32_t* topk_idx_out, float* topk_w_out, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * Kernel-choice overrides, for tests and measurements only.  A production
 * call chooses its kernels from the shapes alone and reads no environment
 * variable; an override set here forces one choice instead, for every later
 * call in the process (all devices, all threads) until it is set back to 0
 * (automatic).  A forced choice that a call's shape cannot take falls back
 * to the automatic one.  Every choice computes the same results: the
 * overrides exist so that tests can compare the kernels bit for bit and
 * measurements can time each one.
 */
enum mova_override {
  MOVA_OVERRIDE_PATH = 0,          /* 1: decode kernel (T <= 256), 2: dispatch + grouped GEMM */
  MOVA_OVERRIDE_ROUTER = 1,        /* tokens per router workgroup: 1: 16, 2: 32 (4 LDS
                                      stages), 3: 32 (3 stages), 4: 64 */
  MOVA_OVERRIDE_GEMM_TILE = 2,     /* 1: 256x256, 2: 128x256, 3: 128x128, 4: 128x128 with 3
                                      stages, 5: with 4 stages, 6: 128x128 on 4 waves,
                                      7: 352x256 (routed GEMMs only) */
  MOVA_OVERRIDE_DENSE_PATH = 3,    /* 1: split-k kernel (T <= 256), 2: tiled GEMM */
  MOVA_OVERRIDE_DECODE_CHAIN = 4,  /* small-T expert kernel: 1: the chain kernel wherever it
                                      fits, 2: neither it nor the token-major kernel, 3: the
                                      token-major kernel (combine fused) wherever it fits */
  MOVA_OVERRIDE_DECODE_GROUPS = 5, /* 1 or 2: 16-column groups per wave in the decode kernel */
  MOVA_OVERRIDE_SERIAL = 6,        /* 1: the FFN's shared expert on the caller's stream */
  MOVA_OVERRIDE_COUNT = 7
};

/* Sets an override; MOVA_OK, or MOVA_ERR_INVALID_ARG for an unknown key or a
 * value outside the key's range (nothing changes then). */
int mova_debug_override(int key, int value);

/* The current value of an override (0 = automatic), -1 for an unknown key. */
int mova_debug_override_get(int key);

/*
 * Stage timing (profiling aid).  While enabled, each mova_value_forward call
 * records a HIP event pair on the call's stream around each stage selected
 * by `stage_mask` (bit s = stage s), for up to `capacity` calls.  Stages:
 * 0 router, 1 dispatch, 2 expert projection (grouped GEMM or decode stream),
 * 3 combine; 4 is the whole of a mova_dense_value_proj call.
 *
 * mova_timing_enable(capacity, stage_mask) starts a new collection
 * (capacity <= 0 or stage_mask == 0 turns timing off); it creates host-side
 * HIP events (timing-only: created without a system-scope fence, so they add
 * no cache writeback around the stage), no device memory.
 * mova_timing_read waits for the recorded events and writes, for stage s < n,
 * the summed milliseconds to total_ms[s] and the number of recorded launches
 * to count[s].  Returns MOVA_OK, MOVA_ERR_INVALID_ARG or MOVA_ERR_HIP.
 * Not thread-safe with concurrent forward calls.
 */
int mova_timing_enable(int capacity, unsigned stage_mask);
int mova_timing_read(int n, double* total_ms, int* count);

#ifdef __cplusplus
}
#endif

#endif /* MOVA_H */
