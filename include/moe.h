/* moe.h -- C-ABI of libmoe.so: the routed mixture-of-experts layer on gfx950.
 *
 * The layer (GLM-5.3-Flash class): each token picks the top-K of E experts
 * (K = 8 of E = 288 per layer in that model; page "GLM-5.3-Flash EXL3 3.05bpw on
 * 1x RTX 3090 -- RAM/NVMe expert tiering", field summary), the picks are grouped
 * by expert, each picked expert runs a SwiGLU FFN (gate, up, down matrices, each
 * reached through a per-layer pointer table that can be rewritten in place; page
 * "GLM-5.3-Flash EXL3 3.05bpw on 1x RTX PRO 6000 - GPU expert cache, host-RAM
 * streaming", field config.expert_cache.mechanism), and the expert outputs are
 * summed with the routing weights, plus an optional always-on shared expert
 * (page "0xSero/glm53-flash-offload", paragraph "Decode kernels (fast mode)").
 *
 * Conventions.  Unless stated otherwise every pointer is DEVICE memory, owned by
 * the caller, and every call is stream-ordered on `stream` (a hipStream_t; NULL =
 * the null stream), returns without waiting for the device, makes no device
 * allocation and no host<->device copy except where stated, and can be captured
 * in a HIP graph.  Status codes report host-side argument checks; faults inside
 * kernels surface at the caller's next synchronisation.  No C++ exception crosses
 * this boundary.  One host thread may use a context at a time; calls that run
 * concurrently on different streams need distinct workspaces and contexts (a
 * context with a shared expert owns a second stream and two events: moe_forward
 * runs the shared expert there, forked from and joined back into `stream`; the
 * fork and join are stream-ordered and can be captured).
 *
 * Packed weight format (v1).  A matrix W[N][Kd] (N outputs, Kd reduction; N % 64
 * == 0, Kd % G == 0) stores unsigned codes c with W[n][k] = (c - 2^(bits-1)) *
 * s[n][k/G], one 16-bit scale (bf16 or fp16) per row and group of G consecutive
 * reduction elements.  Supported (bits, G): (3, 128), (4, 32), (2, 128), (4, 128).
 *   codes region: tiles t = (n/64)*(Kd/G) + g, one per 64 rows and one group.  A
 *     tile holds 64 units, unit u = row 64*(n/64) + u, each bits*G/8 bytes split
 *     into C = bits*G/128 chunks of 16 bytes; chunk j of tile t starts at byte
 *     (t*C + j)*1024 and unit u's part of it at +16u (one wave64 16-byte load per
 *     chunk reads 1024 contiguous bytes).  A unit's 32-bit little-endian words
 *     are its chunks' words in order.
 *   code i of a unit (reduction index g*G + i), P = i/2, half h = i%2:
 *     4-bit, G = 32 or 128, 4 or 16 words: c = (w[P/4] >> (16h + 4*(P%4))) & 15
 *     2-bit, G = 128, 8 words:  c = (w[P/8] >> (16h + 2*(P%8))) & 3
 *     3-bit, G = 128, 12 words: P < 60: c = (w[P/5] >> (16h + off[P%5])) & 7,
 *                               off = {1, 4, 7, 10, 13};
 *                               P >= 60, m = P - 60: bit b of c is bit 16h of
 *                               w[3m + b].
 *   scales region: at the next 256-byte boundary after the codes, in the codes'
 *     tile order: tile t = (n/64)*(Kd/G) + g holds the 64 16-bit scales of its
 *     rows, scale s[n][g] at index t*64 + n%64 (one wave's scales of a tile are
 *     128 contiguous bytes); the matrix blob ends at the following 256-byte
 *     boundary.  Blobs must be 256-byte aligned.
 * An expert is three blobs: gate [I][H], up [I][H], down [H][I].  At H = 5120,
 * I = 1536, 3-bit G = 128 an expert is 9,216,000 bytes (3.125 bits per weight).
 * The shared expert is three row-major bfloat16 matrices gate [Is][H], up [Is][H],
 * down [H][Is].
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_ctx moe_ctx;
typedef void* moe_stream_t; /* a hipStream_t */

/* The workspace's error word: an int32 at this byte offset of the workspace.
 * moe_forward sets MOE_ERR_ROUTING in it (atomically; the bit stays set) when it
 * finds caller-supplied routing inconsistent, and MOE_ERR_RANGE (below) when the
 * matrix-core path meets a value outside fp16's exact range.  moe_workspace_init
 * clears it; so may the caller (stream-ordered write of 0). */
#define MOE_WS_ERROR_OFFSET 4
/* The workspace's first MOE_WS_COUNTER_BYTES bytes hold its cross-block
 * counters, the one/two-token combine's accumulators, the error word and the
 * current call's routing verdict; every call leaves them zero again, apart from
 * the error word. */
#define MOE_WS_COUNTER_BYTES 167936
#define MOE_ERR_ROUTING 1
/* Set by a call on the matrix-core path (T > 64) that met a value fp16 does not
 * hold exactly: a group scale s with |s| < 2^-14 or |s| > 8188 (so q*s, |q| <= 8,
 * is not exact), or h = silu(g)*u with |h| >= 65504 (or not finite).  That call's
 * outputs are then not to be trusted; the GEMV path (T <= 64) has no such limit. */
#define MOE_ERR_RANGE 4
/* Set by a call of one or two tokens whose combine met a pair term w*y with
 * |w*y| >= 2^21 (or not finite): that token's affected outputs are NaN.  The
 * combine of these calls sums the terms exactly in 28-bit fixed point. */
#define MOE_ERR_COMBINE 8

typedef enum {
  MOE_OK = 0,
  MOE_E_ARG = 1,          /* invalid argument (null, misaligned, out of range)    */
  MOE_E_UNSUPPORTED = 2,  /* unsupported shape or format                          */
  MOE_E_NOMEM = 3,        /* host or device allocation failed (moe_create only)   */
  MOE_E_HIP = 4,          /* a HIP call or kernel launch failed                   */
  MOE_E_STATE = 5         /* context not ready (e.g. expert table never set)      */
} moe_status;

typedef struct {
  int32_t hidden;        /* H                                                     */
  int32_t inter;         /* I, routed expert intermediate size                    */
  int32_t n_experts;     /* E, routed experts per layer (<= 1024)                 */
  int32_t top_k;         /* K (1 <= K <= min(E, 16))                              */
  int32_t bits;          /* 2, 3 or 4                                             */
  int32_t group;         /* 128 (2, 3 or 4 bits) or 32 (4 bits)                   */
  int32_t scale_f16;     /* 1: fp16 scales, 0: bf16 scales                        */
  int32_t shared_inter;  /* Is, 0 = no shared expert                              */
  int32_t max_tokens;    /* largest T accepted by moe_route / moe_forward         */
} moe_cfg;

/* One expert's three packed blobs (device pointers, 256-byte aligned). */
typedef struct {
  const void* gate;
  const void* up;
  const void* down;
} moe_expert_ref;

/* Create a context for n_layers layers of shape *cfg (the layer of the page
 * "GLM-5.3-Flash EXL3 3.05bpw on 1x RTX 3090 -- RAM/NVMe expert tiering", field
 * summary: top-8 of 288 experts per token and layer).  Allocates only the device
 * pointer tables (3 pointers per expert per layer), the shared-expert pointer
 * slots and, when shared_inter > 0, the shared expert's stream and two events.  H and I must be multiples of 64 and of G; Is a multiple of 64.
 * Returns MOE_E_UNSUPPORTED for other shapes, MOE_E_NOMEM on allocation failure. */
moe_status moe_create(const moe_cfg* cfg, int32_t n_layers, moe_ctx** out);

/* Free the context's tables.  Waits for the device to finish with them. */
moe_status moe_destroy(moe_ctx* ctx);

/* Workspace bytes that moe_route and moe_forward need for any T <= n_tokens
 * tokens (0 if n_tokens is out of range).  One workspace serves both calls.
 * Batches of T <= 64 tokens run the GEMV kernels; larger ones the matrix-core
 * kernels (when H and I are multiples of 128), whose activation copies are fp16
 * scaled by a per-token power of two and whose h = silu(g)*u is held in fp16
 * (|h| must stay below 65504). */
size_t moe_workspace_bytes(const moe_ctx* ctx, int32_t n_tokens);

/* Zero the workspace's counters and its error word; must run once on a new
 * workspace before its first use (zero-filled memory also qualifies).  Every
 * later call leaves the counters zero again.  Uses a fill kernel, not a memset. */
moe_status moe_workspace_init(const moe_ctx* ctx, void* ws, size_t ws_bytes,
                              moe_stream_t stream);

/* Set one layer's pointer table (page "GLM-5.3-Flash EXL3 3.05bpw on 1x RTX PRO
 * 6000 - GPU expert cache, host-RAM streaming", field config.expert_cache.mechanism:
 * per-layer gate, up and down pointer tables rewritten in place): host_table[e]
 * (HOST array of E entries, logical expert order) gives expert e's three blobs.
 * The entries reach the device as arguments of a stream-ordered kernel (up to
 * 128 entries per launch): the host array may be reused as soon as the call
 * returns, the call does not wait for the device, and a captured HIP graph keeps
 * its own copy of the entries.  Only pointers are set, so the blobs must outlive
 * their table entries.  A remap to other physical slots is another call; results
 * depend only on the logical ids, never on where the bytes are (page
 * "0xSero/glm53-flash-offload", paragraph "Elastic CLOCK expert cache").
 * MOE_E_ARG for a null or misaligned blob (checked on the host first). */
moe_status set_expert_table(moe_ctx* ctx, int32_t layer, const moe_expert_ref* host_table,
                            moe_stream_t stream);

/* Device address of a layer's table (E entries of moe_expert_ref, logical
 * order), for in-place rewrites by device code (the cache manager of the RTX PRO
 * 6000 page rewrites the tables on the device, field
 * config.expert_cache.mechanism).  The context owns the table; writes must be
 * stream-ordered before the moe_forward calls that read them.  NULL on a bad
 * layer. */
void* moe_expert_table_device(moe_ctx* ctx, int32_t layer);

/* Set a layer's shared expert (row-major bfloat16 gate [Is][H], up [Is][H],
 * down [H][Is]), the always-on expert beside the routed ones (page
 * "0xSero/glm53-flash-offload", paragraph "Decode kernels (fast mode)"); NULLs
 * clear it.  Only pointers are kept; host-side call, no device work. */
moe_status moe_set_shared(moe_ctx* ctx, int32_t layer, const void* gate, const void* up,
                          const void* down);

/* Route T tokens: top-K of E experts per token and the grouping of the picks by
 * expert (pages "GLM-5.3-Flash EXL3 3.05bpw on 1x RTX 3090 -- RAM/NVMe expert
 * tiering", field summary; "0xSero/glm53-flash-offload", paragraphs "Elastic
 * CLOCK expert cache" and "Batched decode": the picks deduplicated into the
 * layer's expert union with each expert's tokens).  The pages do not print the
 * router function; it is read as a softmax over the logits below, renormalised
 * over the picks.
 *   x_bf16    [T][H] bfloat16 activations
 *   w_router  [E][H] fp32 router matrix; bias [E] fp32 or NULL
 *   logits l[t][e] = sum_h x[t][h] * w_router[e][h] + bias[e], accumulated in fp64
 *   (every product is exact in fp64), so the selection is the exact-arithmetic one
 *   up to summation-order rounding;
 *   topk_ids  [T][K] int32: the K largest logits, descending, ties to the lower id
 *   topk_w    [T][K] fp32: softmax over all experts restricted to the K picks and
 *             renormalised, w_k = exp(l_k - l_0) / sum_j exp(l_j - l_0)
 *   expert_offsets [E+1] int32, sorted_pairs [T*K] int32, pair_pos [T*K] int32:
 *             pairs p = t*K + k grouped by logical expert (ascending), stable by p:
 *             expert e owns positions expert_offsets[e] .. expert_offsets[e+1]-1,
 *             sorted_pairs[i] is the pair at position i, pair_pos[p] its position.
 *   ws        workspace of at least moe_workspace_bytes(ctx, T) bytes, 256-aligned.
 * T = 0 returns MOE_OK and launches nothing. */
moe_status moe_route(moe_ctx* ctx, const void* x_bf16, int32_t T, const float* w_router,
                     const float* bias, int32_t* topk_ids, float* topk_w,
                     int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* pair_pos,
                     void* ws, size_t ws_bytes, moe_stream_t stream);

/* Expert FFNs and combine for one layer (page "GLM-5.3-Flash EXL3 3.05bpw on 1x
 * RTX PRO 6000 - GPU expert cache, host-RAM streaming", field
 * config.expert_cache.mechanism: each expert's gate, up and down reached through
 * the layer's tables; page "0xSero/glm53-flash-offload", paragraph "Decode
 * kernels (fast mode)": the shared expert beside the routed ones), given routing
 * (topk_ids, topk_w, expert_offsets, sorted_pairs from moe_route, or from the
 * caller in the same layout; pair_pos is not needed here).
 *   out       [T][H] fp32: out[t] = sum_{k=0..K-1} topk_w[t][k] * y(t,k) + shared(x_t)
 *             if set, bit-reproducible: a fixed-order fp32 sum (k ascending), or
 *             for one and two tokens an exact fixed-point sum (MOE_ERR_COMBINE)
 *   pair_out  [T*K][H] fp32 or NULL: row t*K + k is the unweighted expert output
 *             y(t,k); rows of pairs left out of the grouping are not written
 *   y(t,k) = down . (silu(gate . x_t) * (up . x_t)) of expert topk_ids[t][k],
 *   accumulated in fp32 from exact integer codes and bf16 activations with the
 *   group scale applied per group.
 * A pair whose id is outside [0, E) must be left out of the grouping and then
 * contributes nothing.  The routing is checked on the device, in the call's own
 * kernels (the host never waits): offsets[0] == 0, offsets non-decreasing,
 * offsets[E] equal to the number of pairs with an id in [0, E), and each grouped
 * position i < offsets[E] holding a pair p in [0, T*K) whose id e has
 * offsets[e] <= i < offsets[e+1], ascending within an expert.  Inconsistent
 * routing makes the call write neither out nor pair_out and set MOE_ERR_ROUTING
 * in the workspace's error word; every read stays inside the buffers' documented
 * extents ([T][K] ids, [E+1] offsets, [T*K] sorted pairs) whatever their values.
 * Returns MOE_E_STATE if the layer's table was never set. */
moe_status moe_forward(moe_ctx* ctx, int32_t layer, const void* x_bf16, int32_t T,
                       const int32_t* topk_ids, const float* topk_w,
                       const int32_t* expert_offsets, const int32_t* sorted_pairs, float* out,
                       float* pair_out, void* ws, size_t ws_bytes, moe_stream_t stream);

/* moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels and results, with the workspace taken from a scratch array inside the
 * library (MOE_NOALLOC_SCRATCH_BYTES of device memory per GPU, held from the
 * first moe_create on that GPU until the process ends) instead of a caller
 * buffer.  The call itself allocates nothing.  Arguments, layout and routing
 * check as moe_forward; MOE_E_ARG (with a message) when T needs more scratch than
 * the array holds (more than MOE_NOALLOC_SCRATCH_BYTES of workspace: at H = 5120,
 * I = 1536, K = 8 with a shared expert, batches of up to 15 tokens fit).  Every call on
 * one GPU, from any context, shares that GPU's array, which keeps the last
 * call's contents (its counters are left zero): calls that overlap on one GPU,
 * e.g. on two streams, race and must not be issued.  The array's error word is
 * not exposed; inconsistent routing still leaves the outputs untouched. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
moe_status moe_forward_noalloc(moe_ctx* ctx, int32_t layer, const void* x_bf16, int32_t T,
                               const int32_t* topk_ids, const float* topk_w,
                               const int32_t* expert_offsets, const int32_t* sorted_pairs,
                               float* out, float* pair_out, moe_stream_t stream);

/* Host home for experts (page "0xSero/glm53-flash-offload", paragraph "Zero-copy
 * home": every routed expert in a pinned host arena, the pointer tables holding
 * its device alias, read by the expert kernels with no copy).  Allocates `bytes`
 * of pinned host memory mapped into the device's address space; *host is the
 * host address (fill the expert blobs there), *device the address to put in
 * pointer tables (256-byte aligned).  Blocking host call; not for use under
 * capture.  MOE_E_NOMEM when the allocation fails. */
moe_status moe_host_arena_create(size_t bytes, void** host, void** device);
moe_status moe_host_arena_destroy(void* host);

/* Device-side expert cache over one layer's table (page "GLM-5.3-Flash EXL3
 * 3.05bpw on 1x RTX PRO 6000 - GPU expert cache, host-RAM streaming", field
 * config.expert_cache.mechanism; page "0xSero/glm53-flash-offload", paragraph
 * "Elastic CLOCK expert cache").  Every expert has a home copy (device memory or
 * a host arena); `slots` copies fit in a caller-owned device slot arena
 * (slot_bytes apart, each >= the three blobs of an expert laid out gate, up,
 * down).  moe_cache_init points the layer's table at the home copies and resets
 * the cache state (a caller-owned device buffer of moe_cache_state_bytes bytes,
 * 256-byte aligned; one per layer).  moe_cache_step, called after the routing of
 * a step (expert_offsets as moe_route writes them) and before moe_forward, runs
 * one block that marks the step's experts, counts hits and misses, picks a
 * victim slot for each miss (MOE_CACHE_LFU: scores decay by `decay` per step and
 * gain one per use, the lowest score among the slots the step does not use is
 * evicted; MOE_CACHE_CLOCK: reference bits and a hand), rewrites the table in
 * place (admitted experts at their slot, evicted ones back at home), then a
 * gather kernel copies the admitted experts into their slots.  Stream-ordered;
 * nothing waits for the host; capturable.  Results of moe_forward do not change:
 * the bytes are the same wherever they are read from.  The state begins with
 * int64 steps, hits, misses (totals) and int32 hits, misses of the last step.
 * The home copies and the arena must outlive the cache's use of the table. */
#define MOE_CACHE_LFU 0
#define MOE_CACHE_CLOCK 1
size_t moe_cache_state_bytes(const moe_ctx* ctx, int32_t slots);
moe_status moe_cache_init(moe_ctx* ctx, int32_t layer, int32_t slots, int32_t policy, double decay,
                          const moe_expert_ref* home_table, void* slot_arena, size_t slot_bytes,
                          void* state, size_t state_bytes, moe_stream_t stream);
moe_status moe_cache_step(moe_ctx* ctx, int32_t layer, const int32_t* expert_offsets, void* state,
                          moe_stream_t stream);

/* Stack glue between the MoE layers of a stack (42 of them in the pages' model;
 * page "GLM-5.3-Flash EXL3 2.05bpw on 2x RTX 5090 - TabbyAPI hot-expert swaps,
 * 262K ctx, vision": MoE layers 3-44; the norm itself is not on the pages, it is
 * read as a unit-gain RMSNorm): y_bf16[t] = bf16(x[t] / sqrt(mean(x[t]^2) + eps))
 * (unit gain, round to nearest even) for fp32 x [T][H]; and, if resid is not
 * NULL, resid[t][h] += add[t][h] first (fp32), normalising the updated resid. */
moe_status moe_rmsnorm_bf16(const moe_ctx* ctx, float* resid, const float* add, int32_t T,
                            float eps, void* y_bf16, moe_stream_t stream);

/* One MoE layer in one call (page "0xSero/glm53-flash-offload", bullet "Decode
 * kernels (fast mode)": a decode layer's launches fused): the routing of x_bf16
 * into the routing buffers exactly as moe_route, then the expert FFNs and combine
 * exactly as moe_forward on that routing, with the same results bit for bit.
 * Because no caller code can run between the two, batches of one or two tokens
 * let the routing kernel hand each active expert's table entry to the expert
 * kernels, which then skip their own lookup.  Arguments, layouts, alignment and
 * workspace as for moe_route and moe_forward; stream-ordered, capturable.
 * Returns MOE_E_STATE if the layer's table was never set. */
moe_status moe_layer_forward(moe_ctx* ctx, int32_t layer, const void* x_bf16, int32_t T,
                             const float* w_router, const float* bias, int32_t* topk_ids,
                             float* topk_w, int32_t* expert_offsets, int32_t* sorted_pairs,
                             int32_t* pair_pos, float* out, float* pair_out, void* ws,
                             size_t ws_bytes, moe_stream_t stream);

/* One MoE layer of a stack on its residual stream, in one call:
 *   xn_bf16 = bf16(RMSNorm(resid))    (exactly as moe_rmsnorm_bf16 with add NULL)
 *   routing of xn_bf16                (as moe_route, into the routing buffers)
 *   out = MoE_layer(xn_bf16)          (as moe_forward; pair_out not written)
 *   resid += out                      (fp32, elementwise)
 * so that repeated over the layers it computes x <- x + MoE(bf16(RMSNorm(x)))
 * (the stack glue named beside moe_rmsnorm_bf16 below).  The normalisation is
 * done inside the routing kernels of batches up to 32 tokens (one launch fewer
 * per layer) and the residual update inside the combine; the results are bit for
 * bit those of moe_rmsnorm_bf16(resid, NULL) + moe_route + moe_forward followed by
 * resid += out.  resid fp32 [T][H] (read and written), xn_bf16 [T][H] and out fp32
 * [T][H] caller-owned device buffers, 16-byte aligned; eps in [0, 1]; workspace as
 * for moe_forward.  Stream-ordered, nothing waits for the host, capturable. */
moe_status moe_stack_layer(moe_ctx* ctx, int32_t layer, float* resid, int32_t T, float eps,
                           const float* w_router, const float* bias, int32_t* topk_ids,
                           float* topk_w, int32_t* expert_offsets, int32_t* sorted_pairs,
                           int32_t* pair_pos, void* xn_bf16, float* out, void* ws,
                           size_t ws_bytes, moe_stream_t stream);

/* Kernel timing (measurement aid, not part of the layer).  While enabled
 * (process-wide), every kernel the library
 * launches carries two HIP events that the launch timestamps at the kernel's
 * start and end (the kernel's own duration, without the dispatch latency).
 * moe_profile_read waits for the recorded events, writes up to max_kernels
 * entries (names: max_kernels x 32 chars, NUL-terminated, HOST memory; total_ms
 * and launches: HOST arrays) for the kernels launched since the last read, and
 * returns the number of entries.  Not for use while a stream is being captured. */
moe_status moe_profile_enable(int32_t on);
int32_t moe_profile_read(int32_t max_kernels, char* names, double* total_ms, int64_t* launches);
/* The same, also giving each kernel's median launch duration and the mean of its
 * launches within twice that median (median_ms, typical_mean_ms: HOST arrays, or
 * NULL).  A launch's start event is occasionally held back by the host side of
 * the launch by hundreds of microseconds; these two figures are not moved by
 * such outliers. */
int32_t moe_profile_read_stats(int32_t max_kernels, char* names, double* total_ms,
                               double* median_ms, double* typical_mean_ms, int64_t* launches);

/* Streaming-read probe (measurement aid, not part of the layer): reads `bytes`
 * (a multiple of 16) of device memory at src (16-byte aligned) once, with the
 * access pattern of the decode kernels' weight stream (16-byte loads, each wave
 * instruction covering 1,024 contiguous bytes, eight loads in flight per thread,
 * up to 4,096 blocks of 256 threads walking the buffer).  sink: device memory of
 * 4,096 x 256 words that the kernel may write (it writes nothing in practice).
 * Timed with moe_profile_* (kernel "stream_read") it gives the practical HBM
 * read rate of one launch of that size.  MOE_E_ARG for bad arguments. */
moe_status moe_stream_read(const void* src, size_t bytes, void* sink, moe_stream_t stream);

/* Detail string of the last non-OK status on this thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
