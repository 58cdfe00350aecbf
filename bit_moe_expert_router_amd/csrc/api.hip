// api.hip -- the extern "C" boundary of libmoe.so (declared in include/moe.h):
// argument checks, the device pointer tables, workspace geometry and dispatch.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <new>
#include <vector>

#include "common.h"

// Scratch of moe_forward_noalloc: the workspace of callers that cannot allocate,
// in the library's own device memory (each GPU the library runs on holds one copy
// until the process ends).  Host code never passes this name to a kernel or a
// copy: it is a host-side stand-in, not a device address.  moe_create looks up
// the device address once per device (hipGetSymbolAddress, with that device
// current) and keeps it in s_scratch_dev; only that address is used.
constexpr size_t kNoAllocBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex s_scratch_mu;
void* s_scratch_dev[kMaxDevices];  // per device: scratch's device address, or null
}  // namespace


struct moe_ctx {
  moe_cfg cfg;
  int n_layers;
  moe_expert_ref* d_tables;       // [n_layers][E] on the device
  std::vector<char> table_set;    // per layer
  struct Shared {
    const void *g, *u, *d;
  };
  std::vector<Shared> shared;     // per layer
  uint8_t* scratch = nullptr;     // this device's copy of the no-allocation scratch
  // the shared expert runs on a second stream (default priority) between a fork
  // event recorded on the caller's stream and a join event the combine waits for
  hipStream_t side = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
};

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

moe_status ok() {
  g_err[0] = 0;
  return MOE_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

moe_status check_cfg(const moe_cfg& c) {
  if (c.hidden <= 0 || c.inter <= 0 || c.n_experts <= 0 || c.top_k <= 0 || c.max_tokens <= 0)
    return fail(MOE_E_ARG, "cfg: sizes must be positive");
  if (moe::codec_of(c.bits, c.group) < 0)
    return fail(MOE_E_UNSUPPORTED,
                "cfg: (bits, group) = (%d, %d) unsupported; use (3,128), (4,32), (2,128) or (4,128)",
                c.bits, c.group);
  if (c.hidden % 64 || c.inter % 64 || c.hidden % c.group || c.inter % c.group)
    return fail(MOE_E_UNSUPPORTED, "cfg: hidden and inter must be multiples of 64 and of the group");
  if (c.n_experts > 1024) return fail(MOE_E_UNSUPPORTED, "cfg: at most 1024 experts");
  if (c.hidden / c.group > 64 || c.inter / c.group > 32 || c.hidden > 8192 || c.inter > 8192)
    return fail(MOE_E_UNSUPPORTED,
                "cfg: at most 64 groups along hidden, 32 along inter, and sizes <= 8192");
  if (c.top_k > 16 || c.top_k > c.n_experts) return fail(MOE_E_UNSUPPORTED, "cfg: top_k must be <= min(16, E)");
  if (c.shared_inter < 0) return fail(MOE_E_ARG, "cfg: shared_inter < 0");
  if (c.shared_inter > 0 && (c.shared_inter % 256 || c.hidden % 256))
    return fail(MOE_E_UNSUPPORTED, "cfg: shared expert needs hidden and shared_inter multiples of 256");
  if ((int64_t)c.max_tokens * c.top_k > (1 << 30)) return fail(MOE_E_UNSUPPORTED, "cfg: max_tokens too large");
  if (c.scale_f16 != 0 && c.scale_f16 != 1) return fail(MOE_E_ARG, "cfg: scale_f16 must be 0 or 1");
  return ok();
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err; }

moe_status moe_create(const moe_cfg* cfg, int32_t n_layers, moe_ctx** out) {
  if (!cfg || !out) return fail(MOE_E_ARG, "moe_create: null argument");
  *out = nullptr;
  if (n_layers <= 0) return fail(MOE_E_ARG, "moe_create: n_layers must be positive");
  moe_status st = check_cfg(*cfg);
  if (st != MOE_OK) return st;
  moe_ctx* c = new (std::nothrow) moe_ctx();
  if (!c) return fail(MOE_E_NOMEM, "moe_create: host allocation");
  c->cfg = *cfg;
  c->n_layers = n_layers;
  c->table_set.assign(n_layers, 0);
  c->shared.assign(n_layers, moe_ctx::Shared{nullptr, nullptr, nullptr});
  size_t tb = sizeof(moe_expert_ref) * (size_t)n_layers * cfg->n_experts;
  if (hipMalloc(&c->d_tables, tb) != hipSuccess) {
    delete c;
    return fail(MOE_E_NOMEM, "moe_create: device tables (%zu bytes)", tb);
  }
  {  // the no-allocation scratch of this device: its address, and zero counters
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    std::lock_guard<std::mutex> lk(s_scratch_mu);
    if (e == hipSuccess && dev >= 0 && dev < kMaxDevices && !s_scratch_dev[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e == hipSuccess) e = moe::launch_zero_i32((int32_t*)p, moe::kCounters, nullptr);
      if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
      if (e == hipSuccess) s_scratch_dev[dev] = p;
    }
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
      (void)hipFree(c->d_tables);
      delete c;
      return fail(MOE_E_HIP, "moe_create: device scratch lookup: %s",
                  e != hipSuccess ? hipGetErrorString(e) : "device id out of range");
    }
    c->scratch = (uint8_t*)s_scratch_dev[dev];
  }
  if (cfg->shared_inter > 0 &&
      (hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking) != hipSuccess ||
       hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming) != hipSuccess ||
       hipEventCreateWithFlags(&c->ev_join, hipEventDisableTiming) != hipSuccess)) {
    if (c->ev_fork) (void)hipEventDestroy(c->ev_fork);
    if (c->side) (void)hipStreamDestroy(c->side);
    (void)hipFree(c->d_tables);
    delete c;
    return fail(MOE_E_HIP, "moe_create: shared-expert stream or events");
  }
  *out = c;
  return ok();
}

moe_status moe_destroy(moe_ctx* ctx) {
  if (!ctx) return ok();
  (void)hipDeviceSynchronize();
  (void)hipFree(ctx->d_tables);
  if (ctx->ev_join) (void)hipEventDestroy(ctx->ev_join);
  if (ctx->ev_fork) (void)hipEventDestroy(ctx->ev_fork);
  if (ctx->side) (void)hipStreamDestroy(ctx->side);
  delete ctx;
  return ok();
}

size_t moe_workspace_bytes(const moe_ctx* ctx, int32_t n_tokens) {
  if (!ctx || n_tokens < 0 || n_tokens > ctx->cfg.max_tokens) return 0;
  // enough for every T <= n_tokens: the decode layout grows with T up to the mode
  // switch, the prefill layout from there on
  const int64_t dec = moe::ws_layout(ctx->cfg, n_tokens < moe::kDecodeMaxTokens ? n_tokens
                                                                                : moe::kDecodeMaxTokens).total;
  const int64_t all = moe::ws_layout(ctx->cfg, n_tokens).total;
  return (size_t)(dec > all ? dec : all);
}

moe_status moe_workspace_init(const moe_ctx* ctx, void* ws, size_t ws_bytes, moe_stream_t stream) {
  if (!ctx || !ws) return fail(MOE_E_ARG, "moe_workspace_init: null argument");
  if (ws_bytes < (size_t)moe::kCounters * 4) return fail(MOE_E_ARG, "moe_workspace_init: workspace too small");
  hipStream_t s = (hipStream_t)stream;
  return hip_status(moe::launch_zero_i32((int32_t*)ws, moe::kCounters, s), "moe_workspace_init");
}

moe_status set_expert_table(moe_ctx* ctx, int32_t layer, const moe_expert_ref* host_table,
                            moe_stream_t stream) {
  if (!ctx || !host_table) return fail(MOE_E_ARG, "set_expert_table: null argument");
  if (layer < 0 || layer >= ctx->n_layers) return fail(MOE_E_ARG, "set_expert_table: bad layer %d", layer);
  const int E = ctx->cfg.n_experts;
  for (int e = 0; e < E; ++e) {
    const moe_expert_ref& r = host_table[e];
    if (!r.gate || !r.up || !r.down)
      return fail(MOE_E_ARG, "set_expert_table: expert %d has a null blob", e);
    if (!aligned(r.gate, 256) || !aligned(r.up, 256) || !aligned(r.down, 256))
      return fail(MOE_E_ARG, "set_expert_table: expert %d blob not 256-byte aligned", e);
  }
  // the entries travel as kernel arguments: the host table may be reused right
  // after return, nothing waits, and a captured graph holds its own copy
  const hipError_t err = moe::launch_set_table(ctx->d_tables + (size_t)layer * E, host_table, E,
                                               (hipStream_t)stream);
  if (err != hipSuccess) return hip_status(err, "set_expert_table");
  ctx->table_set[layer] = 1;
  return ok();
}

void* moe_expert_table_device(moe_ctx* ctx, int32_t layer) {
  if (!ctx || layer < 0 || layer >= ctx->n_layers) return nullptr;
  return ctx->d_tables + (size_t)layer * ctx->cfg.n_experts;
}

moe_status moe_set_shared(moe_ctx* ctx, int32_t layer, const void* gate, const void* up,
                          const void* down) {
  if (!ctx) return fail(MOE_E_ARG, "moe_set_shared: null context");
  if (layer < 0 || layer >= ctx->n_layers) return fail(MOE_E_ARG, "moe_set_shared: bad layer %d", layer);
  const bool any = gate || up || down, all = gate && up && down;
  if (any && !all) return fail(MOE_E_ARG, "moe_set_shared: give all three matrices or none");
  if (any && ctx->cfg.shared_inter <= 0)
    return fail(MOE_E_STATE, "moe_set_shared: context created without a shared expert");
  if (any && (!aligned(gate, 16) || !aligned(up, 16) || !aligned(down, 16)))
    return fail(MOE_E_ARG, "moe_set_shared: matrices must be 16-byte aligned");
  ctx->shared[layer] = moe_ctx::Shared{gate, up, down};
  return ok();
}

moe_status moe_route(moe_ctx* ctx, const void* x_bf16, int32_t T, const float* w_router,
                     const float* bias, int32_t* topk_ids, float* topk_w,
                     int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* pair_pos,
                     void* ws, size_t ws_bytes, moe_stream_t stream) {
  if (!ctx) return fail(MOE_E_ARG, "moe_route: null context");
  const moe_cfg& c = ctx->cfg;
  if (T < 0 || T > c.max_tokens) return fail(MOE_E_ARG, "moe_route: T=%d outside [0, %d]", T, c.max_tokens);
  if (T == 0) return ok();
  if (!x_bf16 || !w_router || !topk_ids || !topk_w || !expert_offsets || !sorted_pairs || !pair_pos || !ws)
    return fail(MOE_E_ARG, "moe_route: null pointer argument");
  if (!aligned(x_bf16, 16) || !aligned(w_router, 16) || !aligned(ws, 256))
    return fail(MOE_E_ARG, "moe_route: x and w_router must be 16-byte aligned, ws 256-byte aligned");
  const moe::WsLayout L = moe::ws_layout(c, T);
  if (ws_bytes < (size_t)L.total)
    return fail(MOE_E_ARG, "moe_route: workspace %zu bytes < %lld needed", ws_bytes, (long long)L.total);
  uint8_t* w8 = (uint8_t*)ws;
  const moe::RouteIn in{(const uint16_t*)x_bf16, nullptr, 0.f, nullptr};
  hipError_t e = moe::launch_route(c, in, T, w_router, bias, topk_ids, topk_w, expert_offsets,
                                   sorted_pairs, pair_pos, (double*)(w8 + L.logits),
                                   (int32_t*)(w8 + L.ghist), (int32_t*)(w8 + L.counters),
                                   (hipStream_t)stream);
  return hip_status(e, "moe_route launch");
}

}  // extern "C"

namespace {

moe_status forward_impl(const char* who, moe_ctx* ctx, int32_t layer, const void* x_bf16,
                        int32_t T, const int32_t* topk_ids, const float* topk_w,
                        const int32_t* expert_offsets, const int32_t* sorted_pairs, float* out,
                        float* pair_out, void* ws, size_t ws_bytes, moe_stream_t stream,
                        float* resid = nullptr, int pre_entries = 0) {
  if (!ctx) return fail(MOE_E_ARG, "%s: null context", who);
  const moe_cfg& c = ctx->cfg;
  if (layer < 0 || layer >= ctx->n_layers) return fail(MOE_E_ARG, "%s: bad layer %d", who, layer);
  if (T < 0 || T > c.max_tokens) return fail(MOE_E_ARG, "%s: T=%d outside [0, %d]", who, T, c.max_tokens);
  if (!ctx->table_set[layer]) return fail(MOE_E_STATE, "%s: expert table of layer %d never set", who, layer);
  if (T == 0) return ok();
  if (!x_bf16 || !topk_ids || !topk_w || !expert_offsets || !sorted_pairs || !out || !ws)
    return fail(MOE_E_ARG, "%s: null pointer argument", who);
  if (!aligned(x_bf16, 16) || !aligned(out, 16) || !aligned(ws, 256) || (pair_out && !aligned(pair_out, 16)))
    return fail(MOE_E_ARG, "%s: x, out, pair_out must be 16-byte aligned, ws 256-byte aligned", who);
  const moe::WsLayout L = moe::ws_layout(c, T);
  if (ws_bytes < (size_t)L.total)
    return fail(MOE_E_ARG, "%s: workspace %zu bytes < %lld needed", who, ws_bytes, (long long)L.total);
  const moe_ctx::Shared& sh = ctx->shared[layer];
  moe::FwdArgs f{&c, ctx->d_tables + (size_t)layer * c.n_experts, sh.g, sh.u, sh.d,
                 (const uint16_t*)x_bf16, T, topk_ids, topk_w, expert_offsets, sorted_pairs,
                 out, pair_out, resid, (uint8_t*)ws, ctx->side, ctx->ev_fork, ctx->ev_join};
  f.pre_entries = pre_entries;
  return hip_status(moe::launch_forward(f, (hipStream_t)stream), who);
}

}  // namespace

extern "C" {

moe_status moe_forward(moe_ctx* ctx, int32_t layer, const void* x_bf16, int32_t T,
                       const int32_t* topk_ids, const float* topk_w,
                       const int32_t* expert_offsets, const int32_t* sorted_pairs, float* out,
                       float* pair_out, void* ws, size_t ws_bytes, moe_stream_t stream) {
  return forward_impl("moe_forward", ctx, layer, x_bf16, T, topk_ids, topk_w, expert_offsets,
                      sorted_pairs, out, pair_out, ws, ws_bytes, stream);
}

moe_status moe_forward_noalloc(moe_ctx* ctx, int32_t layer, const void* x_bf16, int32_t T,
                               const int32_t* topk_ids, const float* topk_w,
                               const int32_t* expert_offsets, const int32_t* sorted_pairs,
                               float* out, float* pair_out, moe_stream_t stream) {
  if (!ctx) return fail(MOE_E_ARG, "moe_forward_noalloc: null context");
  if (T > 0 && T <= ctx->cfg.max_tokens) {
    const int64_t need = moe::ws_layout(ctx->cfg, T).total;
    if ((size_t)need > kNoAllocBytes)
      return fail(MOE_E_ARG,
                  "moe_forward_noalloc: T=%d needs %lld bytes of scratch, more than the "
                  "library's %zu; use moe_forward with a workspace",
                  T, (long long)need, kNoAllocBytes);
  }
  return forward_impl("moe_forward_noalloc", ctx, layer, x_bf16, T, topk_ids, topk_w,
                      expert_offsets, sorted_pairs, out, pair_out, ctx->scratch, kNoAllocBytes,
                      stream);
}

moe_status moe_stack_layer(moe_ctx* ctx, int32_t layer, float* resid, int32_t T, float eps,
                           const float* w_router, const float* bias, int32_t* topk_ids,
                           float* topk_w, int32_t* expert_offsets, int32_t* sorted_pairs,
                           int32_t* pair_pos, void* xn_bf16, float* out, void* ws,
                           size_t ws_bytes, moe_stream_t stream) {
  if (!ctx) return fail(MOE_E_ARG, "moe_stack_layer: null context");
  const moe_cfg& c = ctx->cfg;
  if (layer < 0 || layer >= ctx->n_layers) return fail(MOE_E_ARG, "moe_stack_layer: bad layer %d", layer);
  if (T < 0 || T > c.max_tokens)
    return fail(MOE_E_ARG, "moe_stack_layer: T=%d outside [0, %d]", T, c.max_tokens);
  if (!ctx->table_set[layer])
    return fail(MOE_E_STATE, "moe_stack_layer: expert table of layer %d never set", layer);
  if (!(eps >= 0.f) || eps > 1.f) return fail(MOE_E_ARG, "moe_stack_layer: eps must be in [0, 1]");
  if (T == 0) return ok();
  if (!resid || !w_router || !topk_ids || !topk_w || !expert_offsets || !sorted_pairs || !pair_pos ||
      !xn_bf16 || !out || !ws)
    return fail(MOE_E_ARG, "moe_stack_layer: null pointer argument");
  if (!aligned(resid, 16) || !aligned(w_router, 16) || !aligned(xn_bf16, 16) || !aligned(out, 16) ||
      !aligned(ws, 256))
    return fail(MOE_E_ARG,
                "moe_stack_layer: resid, w_router, xn_bf16, out must be 16-byte aligned, ws 256-byte aligned");
  const moe::WsLayout L = moe::ws_layout(c, T);
  if (ws_bytes < (size_t)L.total)
    return fail(MOE_E_ARG, "moe_stack_layer: workspace %zu bytes < %lld needed", ws_bytes,
                (long long)L.total);
  uint8_t* w8 = (uint8_t*)ws;
  moe::RouteIn in{nullptr, resid, eps, (uint16_t*)xn_bf16};
  int pre = 0;
  if (!moe::prefill_eligible(c, T)) {  // the routing may do the experts' lookup and plan
    in.table = ctx->d_tables + (size_t)layer * c.n_experts;
    in.entries = moe::act_entries(w8, L);
    in.wrote_entries = &pre;
    in.act_hdr = (int32_t*)(w8 + L.act);
    in.osx = (float*)(w8 + L.osx);
    in.ctr0 = (int32_t*)(w8 + L.counters);
    in.codec = moe::codec_of(c.bits, c.group);
  }
  const hipError_t e = moe::launch_route(c, in, T, w_router, bias, topk_ids, topk_w, expert_offsets,
                                         sorted_pairs, pair_pos, (double*)(w8 + L.logits),
                                         (int32_t*)(w8 + L.ghist), (int32_t*)(w8 + L.counters),
                                         (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, "moe_stack_layer routing");
  return forward_impl("moe_stack_layer", ctx, layer, xn_bf16, T, topk_ids, topk_w, expert_offsets,
                      sorted_pairs, out, nullptr, ws, ws_bytes, stream, resid, pre);
}

moe_status moe_layer_forward(moe_ctx* ctx, int32_t layer, const void* x_bf16, int32_t T,
                             const float* w_router, const float* bias, int32_t* topk_ids,
                             float* topk_w, int32_t* expert_offsets, int32_t* sorted_pairs,
                             int32_t* pair_pos, float* out, float* pair_out, void* ws,
                             size_t ws_bytes, moe_stream_t stream) {
  if (!ctx) return fail(MOE_E_ARG, "moe_layer_forward: null context");
  const moe_cfg& c = ctx->cfg;
  if (layer < 0 || layer >= ctx->n_layers) return fail(MOE_E_ARG, "moe_layer_forward: bad layer %d", layer);
  if (T < 0 || T > c.max_tokens)
    return fail(MOE_E_ARG, "moe_layer_forward: T=%d outside [0, %d]", T, c.max_tokens);
  if (!ctx->table_set[layer])
    return fail(MOE_E_STATE, "moe_layer_forward: expert table of layer %d never set", layer);
  if (T == 0) return ok();
  if (!x_bf16 || !w_router || !topk_ids || !topk_w || !expert_offsets || !sorted_pairs || !pair_pos ||
      !out || !ws)
    return fail(MOE_E_ARG, "moe_layer_forward: null pointer argument");
  if (!aligned(x_bf16, 16) || !aligned(w_router, 16) || !aligned(out, 16) || !aligned(ws, 256) ||
      (pair_out && !aligned(pair_out, 16)))
    return fail(MOE_E_ARG,
                "moe_layer_forward: x, w_router, out, pair_out must be 16-byte aligned, ws 256-byte aligned");
  const moe::WsLayout L = moe::ws_layout(c, T);
  if (ws_bytes < (size_t)L.total)
    return fail(MOE_E_ARG, "moe_layer_forward: workspace %zu bytes < %lld needed", ws_bytes,
                (long long)L.total);
  uint8_t* w8 = (uint8_t*)ws;
  moe::RouteIn in{(const uint16_t*)x_bf16, nullptr, 0.f, nullptr};
  int pre = 0;
  if (!moe::prefill_eligible(c, T)) {  // the routing may do the experts' lookup and plan
    in.table = ctx->d_tables + (size_t)layer * c.n_experts;
    in.entries = moe::act_entries(w8, L);
    in.wrote_entries = &pre;
    in.act_hdr = (int32_t*)(w8 + L.act);
    in.osx = (float*)(w8 + L.osx);
    in.ctr0 = (int32_t*)(w8 + L.counters);
    in.codec = moe::codec_of(c.bits, c.group);
  }
  const hipError_t e = moe::launch_route(c, in, T, w_router, bias, topk_ids, topk_w, expert_offsets,
                                         sorted_pairs, pair_pos, (double*)(w8 + L.logits),
                                         (int32_t*)(w8 + L.ghist), (int32_t*)(w8 + L.counters),
                                         (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, "moe_layer_forward routing");
  return forward_impl("moe_layer_forward", ctx, layer, x_bf16, T, topk_ids, topk_w, expert_offsets,
                      sorted_pairs, out, pair_out, ws, ws_bytes, stream, nullptr, pre);
}

moe_status moe_host_arena_create(size_t bytes, void** host, void** device) {
  if (!host || !device || bytes == 0) return fail(MOE_E_ARG, "moe_host_arena_create: bad argument");
  *host = *device = nullptr;
  void* h = nullptr;
  hipError_t e = hipHostMalloc(&h, bytes, hipHostMallocMapped);
  if (e != hipSuccess) return fail(MOE_E_NOMEM, "moe_host_arena_create: %zu bytes: %s", bytes,
                                   hipGetErrorString(e));
  void* d = nullptr;
  e = hipHostGetDevicePointer(&d, h, 0);
  if (e != hipSuccess || !aligned(d, 256)) {
    (void)hipHostFree(h);
    return fail(MOE_E_HIP, "moe_host_arena_create: device address: %s",
                e != hipSuccess ? hipGetErrorString(e) : "not 256-byte aligned");
  }
  *host = h;
  *device = d;
  return ok();
}

moe_status moe_host_arena_destroy(void* host) {
  if (!host) return ok();
  return hip_status(hipHostFree(host), "moe_host_arena_destroy");
}

size_t moe_cache_state_bytes(const moe_ctx* ctx, int32_t slots) {
  if (!ctx || slots < 0 || slots > 1024) return 0;
  return (size_t)moe::cache_state_bytes(ctx->cfg.n_experts, slots);
}

moe_status moe_cache_init(moe_ctx* ctx, int32_t layer, int32_t slots, int32_t policy, double decay,
                          const moe_expert_ref* home_table, void* slot_arena, size_t slot_bytes,
                          void* state, size_t state_bytes, moe_stream_t stream) {
  if (!ctx || !home_table || !state) return fail(MOE_E_ARG, "moe_cache_init: null argument");
  const moe_cfg& c = ctx->cfg;
  if (layer < 0 || layer >= ctx->n_layers) return fail(MOE_E_ARG, "moe_cache_init: bad layer %d", layer);
  if (slots < 0 || slots > 1024 || slots > c.n_experts)
    return fail(MOE_E_ARG, "moe_cache_init: slots %d outside [0, min(E, 1024)]", slots);
  if (policy != MOE_CACHE_LFU && policy != MOE_CACHE_CLOCK)
    return fail(MOE_E_ARG, "moe_cache_init: unknown policy %d", policy);
  if (!(decay > 0.0 && decay <= 1.0)) return fail(MOE_E_ARG, "moe_cache_init: decay outside (0, 1]");
  const moe::MatGeom gu{c.inter, c.hidden, c.bits, c.group}, dn{c.hidden, c.inter, c.bits, c.group};
  const int64_t need = 2 * gu.bytes() + dn.bytes();
  if (slots > 0 && (!slot_arena || !aligned(slot_arena, 256) || slot_bytes < (size_t)need ||
                    slot_bytes % 256))
    return fail(MOE_E_ARG,
                "moe_cache_init: slot arena must be 256-byte aligned with slot_bytes >= %lld, a "
                "multiple of 256", (long long)need);
  if (!aligned(state, 256) || state_bytes < moe_cache_state_bytes(ctx, slots))
    return fail(MOE_E_ARG, "moe_cache_init: state must be 256-byte aligned, %zu bytes",
                moe_cache_state_bytes(ctx, slots));
  for (int e = 0; e < c.n_experts; ++e) {
    const moe_expert_ref& r = home_table[e];
    if (!r.gate || !r.up || !r.down || !aligned(r.gate, 256) || !aligned(r.up, 256) ||
        !aligned(r.down, 256))
      return fail(MOE_E_ARG, "moe_cache_init: home copy of expert %d null or misaligned", e);
  }
  const hipError_t e = moe::launch_cache_init(
      (uint8_t*)state, c.n_experts, slots, policy, decay, (uint64_t)slot_arena, (int64_t)slot_bytes,
      gu.bytes(), dn.bytes(), home_table, ctx->d_tables + (size_t)layer * c.n_experts,
      (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, "moe_cache_init");
  ctx->table_set[layer] = 1;
  return ok();
}

moe_status moe_cache_step(moe_ctx* ctx, int32_t layer, const int32_t* expert_offsets, void* state,
                          moe_stream_t stream) {
  if (!ctx || !expert_offsets || !state) return fail(MOE_E_ARG, "moe_cache_step: null argument");
  if (layer < 0 || layer >= ctx->n_layers) return fail(MOE_E_ARG, "moe_cache_step: bad layer %d", layer);
  return hip_status(moe::launch_cache_step(expert_offsets,
                                           ctx->d_tables + (size_t)layer * ctx->cfg.n_experts,
                                           (uint8_t*)state, (hipStream_t)stream),
                    "moe_cache_step");
}

moe_status moe_rmsnorm_bf16(const moe_ctx* ctx, float* resid, const float* add, int32_t T,
                            float eps, void* y_bf16, moe_stream_t stream) {
  if (!ctx) return fail(MOE_E_ARG, "moe_rmsnorm_bf16: null context");
  if (T < 0 || T > ctx->cfg.max_tokens) return fail(MOE_E_ARG, "moe_rmsnorm_bf16: bad T=%d", T);
  if (T == 0) return ok();
  if (!resid || !y_bf16) return fail(MOE_E_ARG, "moe_rmsnorm_bf16: null pointer argument");
  if (!(eps >= 0.f)) return fail(MOE_E_ARG, "moe_rmsnorm_bf16: eps must be >= 0");
  return hip_status(moe::launch_rmsnorm(resid, add, T, ctx->cfg.hidden, eps, (uint16_t*)y_bf16,
                                        (hipStream_t)stream),
                    "moe_rmsnorm_bf16 launch");
}

}  // extern "C"
