// C ABI of libmoe.so: argument validation, workspace layout and the launch
// sequence of the MoE layer forward.  Declarations and the contract of every
// entry point are in include/moe.h.

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "kernels.h"
#include "moe.h"

namespace {

thread_local std::string g_error;

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

moe_status ok() {
  g_error.clear();
  return MOE_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Byte layout of the workspace for one configuration.
struct Plan {
  int64_t T, P;
  int H, E, k, I, Is;
  int S;         // partials per logit: k splits, or 3 weight planes (router GEMM form)
  int rgemm;     // router logits as one GEMM over the weight planes
  int Np;        // router GEMM: rows of the plane matrix (3E rounded up to the column tile)
  int64_t zld;   // partial logits per token (E S, or Np for the plane GEMM)
  int C;         // permutation chunks, padded to a multiple of 4
  int shape;     // expert GEMM tile shape (kTileBig / kTileSmall)
  int tile_cap;  // capacity of the GEMM tile list
  size_t zpart, wsplit, ids, w, rank, hist, base, offsets, sorted, pos, wsorted, tiles, ntiles,
      queue, h, o, ctl, total;
};

moe_status validate(const moe_config* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "config is NULL");
  if (c->tokens < 0) return fail(MOE_ERR_INVALID_ARG, "tokens < 0 (%lld)", (long long)c->tokens);
  if (c->hidden <= 0 || c->num_experts <= 0 || c->inter <= 0 || c->inter_shared < 0)
    return fail(MOE_ERR_INVALID_ARG, "non-positive size (hidden %d, experts %d, inter %d, shared %d)",
                c->hidden, c->num_experts, c->inter, c->inter_shared);
  if (c->top_k < 1 || c->top_k > c->num_experts)
    return fail(MOE_ERR_INVALID_ARG, "top_k %d outside [1, num_experts=%d]", c->top_k,
                c->num_experts);
  if (c->num_experts > moe::kMaxExperts)
    return fail(MOE_ERR_UNSUPPORTED, "num_experts %d > %d", c->num_experts, moe::kMaxExperts);
  if (c->top_k > moe::kMaxTopK)
    return fail(MOE_ERR_UNSUPPORTED, "top_k %d > %d", c->top_k, moe::kMaxTopK);
  if (c->hidden % 128)
    return fail(MOE_ERR_UNSUPPORTED, "hidden %d is not a multiple of 128", c->hidden);
  if (c->inter % 64 || c->inter_shared % 64)
    return fail(MOE_ERR_UNSUPPORTED, "inter %d / inter_shared %d not multiples of 64", c->inter,
                c->inter_shared);
  if (c->tokens * static_cast<int64_t>(c->top_k) >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "tokens * top_k must be < 2^31");
  if (c->tokens * static_cast<int64_t>(c->top_k) *
          std::max<int64_t>(c->hidden, std::max(c->inter, c->inter_shared)) >= (int64_t(1) << 32))
    return fail(MOE_ERR_UNSUPPORTED, "tokens * top_k * max(hidden, inter) must be < 2^32");
  return MOE_OK;
}

void make_plan(const moe_config* c, Plan* p) {
  p->T = c->tokens;
  p->P = c->tokens * c->top_k;
  p->H = c->hidden;
  p->E = c->num_experts;
  p->k = c->top_k;
  p->I = c->inter;
  p->Is = c->inter_shared;
  const int T = static_cast<int>(p->T);
  p->rgemm = p->T >= moe::kRouterGemmTokens;
  p->Np = (3 * p->E + moe::kRouterGemmTileN - 1) / moe::kRouterGemmTileN * moe::kRouterGemmTileN;
  p->S = p->rgemm ? 3 : (p->T > 0 ? moe::router_split(T, p->H, p->E) : 1);
  p->zld = p->rgemm ? p->Np : static_cast<int64_t>(p->E) * p->S;
  p->C = moe::permute_hist_stride(static_cast<int>(p->P));  // padded chunk count
  p->shape = moe::experts_pick_shape(p->T, static_cast<int>(p->P), p->E, p->H, p->I, p->Is);
  p->tile_cap = moe::experts_tile_capacity(p->T, static_cast<int>(p->P), p->E, p->Is > 0, p->shape);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  const size_t P = static_cast<size_t>(p->P), T64 = static_cast<size_t>(p->T);
  // The single-launch path's control words first, at the same offset for
  // every configuration, so that a workspace reused across batch sizes
  // keeps them where the previous call left them (zero).
  p->ctl = take(static_cast<size_t>(moe::kCtlWords) * 4);
  p->zpart = take(static_cast<size_t>(p->zld) * T64 * 4);
  p->wsplit = take(p->rgemm ? static_cast<size_t>(p->Np) * p->H * 2 : 0);
  p->ids = take(P * 4);
  p->w = take(P * 4);
  p->rank = take(P * 4);
  p->hist = take(static_cast<size_t>(p->E) * p->C * 4);
  p->base = take(static_cast<size_t>(p->E) * p->C * 4);
  p->offsets = take((static_cast<size_t>(p->E) + 1) * 4);
  p->sorted = take(P * 4);
  p->pos = take(P * 4);
  p->wsorted = take(P * 4);
  p->tiles = take(static_cast<size_t>(p->tile_cap) * 8);
  p->ntiles = take(16);
  p->queue = take(moe::kQueueWords * 4);
  p->h = take((P * p->I + T64 * p->Is) * 2);
  p->o = take((P + (p->Is > 0 ? T64 : 0)) * p->H * 2);
  p->total = off;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

moe_status hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define MOE_CHECK_LAUNCH(expr, what)           \
  do {                                         \
    hipError_t e_ = (expr);                    \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

moe_status check_ws(const Plan& p, const void* ws, size_t ws_bytes) {
  if (!ws) return fail(MOE_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned16(ws)) return fail(MOE_ERR_UNSUPPORTED, "workspace not 16-byte aligned");
  if (ws_bytes < p.total)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, p.total);
  return MOE_OK;
}

// Split-k partials are planes [S][T][E]; the plane GEMM's are rows [T][Np]
// with the three planes of expert e in columns 3e .. 3e+2.
moe::PartialLayout partial_layout(const Plan& p) {
  if (p.rgemm) return {3, p.Np, 3, 1};
  return {p.S, p.E, 1, p.T * p.E};
}

moe_status route_impl(const Plan& p, const moe_config* c, const uint16_t* x, const float* rw,
                      const float* rb, int32_t* ids, float* w, void* ws, hipStream_t stream,
                      hipEvent_t* ev) {
  float* zpart = at<float>(ws, p.zpart);
  const int T = static_cast<int>(p.T);
  if (ev) hipEventRecord(ev[0], stream);
  if (p.rgemm) {
    uint16_t* wsplit = at<uint16_t>(ws, p.wsplit);
    MOE_CHECK_LAUNCH(moe::launch_router_split(rw, p.E, p.H, p.Np, wsplit, stream), "router split");
    moe::ExpertArgs g{};
    g.x = x;
    g.T = p.T;
    g.H = p.H;
    g.wsplit = wsplit;
    g.zout = zpart;
    g.Np = p.Np;
    MOE_CHECK_LAUNCH(moe::launch_router_logits(g, stream), "router gemm");
  } else {
    MOE_CHECK_LAUNCH(moe::launch_router_gemm(x, rw, zpart, T, p.H, p.E, p.S, stream),
                     "router gemm");
  }
  if (ev) hipEventRecord(ev[1], stream);
  MOE_CHECK_LAUNCH(moe::launch_topk(zpart, partial_layout(p), rb, T, p.E, p.k, c->routed_scaling,
                                    c->renormalize ? 1 : 0, ids, w, stream),
                   "top-k");
  return MOE_OK;
}

// w (may be NULL): gating weights in pair order, gathered into expert order
// in the workspace for the down GEMM's epilogue.
moe_status permute_impl(const Plan& p, const int32_t* ids, int32_t* offsets, int32_t* sorted,
                        int32_t* pos, const float* w, void* ws, hipStream_t stream,
                        hipEvent_t* ev) {
  MOE_CHECK_LAUNCH(
      moe::launch_permute(ids, static_cast<int>(p.P), p.E, p.T, moe::experts_tile_rows(p.shape),
                          p.Is > 0, at<int32_t>(ws, p.rank), at<int32_t>(ws, p.hist),
                          at<int32_t>(ws, p.base), offsets, sorted, pos, at<int2>(ws, p.tiles),
                          at<int32_t>(ws, p.ntiles), at<uint32_t>(ws, p.queue), w,
                          w ? at<float>(ws, p.wsorted) : nullptr,
                          stream, ev),
      "permute");
  return MOE_OK;
}

// Arguments of the expert GEMMs over the workspace of plan p.
moe::ExpertArgs expert_args(const Plan& p, const moe_config* c, const uint16_t* x,
                            const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                            const uint16_t* ws_gate, const uint16_t* ws_up,
                            const uint16_t* ws_down, void* ws) {
  uint16_t* h_routed = at<uint16_t>(ws, p.h);
  uint16_t* o_routed = at<uint16_t>(ws, p.o);
  moe::ExpertArgs g{};
  g.x = x;
  g.sorted = at<int32_t>(ws, p.sorted);
  g.w_sorted = at<float>(ws, p.wsorted);
  g.k = p.k;
  g.T = p.T;
  g.H = p.H;
  g.I = p.I;
  g.Is = p.Is;
  g.E = p.E;
  g.w_gate = w_gate;
  g.w_up = w_up;
  g.w_down = w_down;
  g.ws_gate = ws_gate;
  g.ws_up = ws_up;
  g.ws_down = ws_down;
  g.limit = c->swiglu_limit;
  g.limit_shared = c->swiglu_limit_shared;
  g.tiles = at<int2>(ws, p.tiles);
  g.ntiles = at<int32_t>(ws, p.ntiles);
  g.offsets = at<int32_t>(ws, p.offsets);
  g.queue = at<uint32_t>(ws, p.queue);
  g.h_routed = h_routed;
  g.h_shared = h_routed + static_cast<size_t>(p.P) * p.I;
  g.o_routed = o_routed;
  g.o_shared = p.Is > 0 ? o_routed + static_cast<size_t>(p.P) * p.H : nullptr;
  return g;
}

// Routed-expert weights as e4m3 codes with per-output-row scales.
struct Fp8Weights {
  const uint8_t *gate, *up, *down;
  const float *s_gate, *s_up, *s_down;
};

// The configuration and the pointers of a layer forward (bf16 or, with f8,
// e4m3 routed weights), before anything else.
moe_status check_forward_args(const moe_config* c, const uint16_t* x, const float* router_w,
                              const float* router_bias, const uint16_t* w_gate,
                              const uint16_t* w_up, const uint16_t* w_down,
                              const uint16_t* ws_gate, const uint16_t* ws_up,
                              const uint16_t* ws_down, const uint16_t* y,
                              const int32_t* topk_ids_out, const float* topk_w_out,
                              const Fp8Weights* f8) {
  moe_status st = validate(c);
  if (st) return st;
  const bool routed_ok = f8 ? (f8->gate && f8->up && f8->down && f8->s_gate && f8->s_up &&
                               f8->s_down)
                            : (w_gate && w_up && w_down);
  if (!router_w || !routed_ok || (c->tokens > 0 && (!x || !y)))
    return fail(MOE_ERR_INVALID_ARG, "a required pointer is NULL");
  if (c->inter_shared > 0 && (!ws_gate || !ws_up || !ws_down))
    return fail(MOE_ERR_INVALID_ARG, "inter_shared > 0 but a shared-expert weight is NULL");
  const void* ptrs[] = {x, router_w, router_bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
                        y, topk_ids_out, topk_w_out,
                        f8 ? f8->gate : nullptr, f8 ? f8->up : nullptr, f8 ? f8->down : nullptr,
                        f8 ? f8->s_gate : nullptr, f8 ? f8->s_up : nullptr,
                        f8 ? f8->s_down : nullptr};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(MOE_ERR_UNSUPPORTED, "pointer %p not 16-byte aligned", q);
  return MOE_OK;
}

moe_status forward_impl(const moe_config* c, const uint16_t* x, const float* router_w,
                        const float* router_bias, const uint16_t* w_gate, const uint16_t* w_up,
                        const uint16_t* w_down, const uint16_t* ws_gate, const uint16_t* ws_up,
                        const uint16_t* ws_down, uint16_t* y, int32_t* topk_ids_out,
                        float* topk_w_out, void* ws, size_t ws_bytes, hipStream_t stream,
                        hipEvent_t* ev, const Fp8Weights* f8 = nullptr) {
  moe_status st = check_forward_args(c, x, router_w, router_bias, w_gate, w_up, w_down, ws_gate,
                                     ws_up, ws_down, y, topk_ids_out, topk_w_out, f8);
  if (st) return st;
  Plan p;
  make_plan(c, &p);
  if ((st = check_ws(p, ws, ws_bytes))) return st;
  if (p.T == 0) return ok();

  int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(ws, p.ids);
  float* w = topk_w_out ? topk_w_out : at<float>(ws, p.w);
  int32_t* offsets = at<int32_t>(ws, p.offsets);
  int32_t* sorted = at<int32_t>(ws, p.sorted);
  int32_t* pos = at<int32_t>(ws, p.pos);

  if ((st = route_impl(p, c, x, router_w, router_bias, ids, w, ws, stream, ev))) return st;
  if ((st = permute_impl(p, ids, offsets, sorted, pos, w, ws, stream, ev ? ev + 2 : nullptr)))
    return st;

  moe::ExpertArgs g = expert_args(p, c, x, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, ws);
  if (f8) {
    g.w8_gate = f8->gate;
    g.w8_up = f8->up;
    g.w8_down = f8->down;
    g.s_gate = f8->s_gate;
    g.s_up = f8->s_up;
    g.s_down = f8->s_down;
  }
  // FP8: the e4m3 kernels; their blocks on shared-expert tiles run the bf16 body.
  if (ev) hipEventRecord(ev[5], stream);
  MOE_CHECK_LAUNCH(moe::launch_gateup(g, p.shape, p.tile_cap, stream, f8 ? 1 : 0), "gate/up gemm");
  if (ev) hipEventRecord(ev[6], stream);
  MOE_CHECK_LAUNCH(moe::launch_down(g, p.shape, p.tile_cap, stream, f8 ? 1 : 0), "down gemm");

  if (ev) hipEventRecord(ev[7], stream);
  MOE_CHECK_LAUNCH(moe::launch_combine(g.o_routed, g.o_shared, pos, p.k, p.T, p.H, y, stream),
                   "combine");
  if (ev) hipEventRecord(ev[8], stream);
  return ok();
}

// ---- single launch (small batches): the same steps in one persistent grid.

moe_status forward_fused_impl(const moe_config* c, const uint16_t* x, const float* router_w,
                              const float* router_bias, const uint16_t* w_gate,
                              const uint16_t* w_up, const uint16_t* w_down,
                              const uint16_t* ws_gate, const uint16_t* ws_up,
                              const uint16_t* ws_down, uint16_t* y, int32_t* topk_ids_out,
                              float* topk_w_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = validate(c);
  if (st) return st;
  if (!router_w || !w_gate || !w_up || !w_down || (c->tokens > 0 && (!x || !y)))
    return fail(MOE_ERR_INVALID_ARG, "a required pointer is NULL");
  if (c->inter_shared > 0 && (!ws_gate || !ws_up || !ws_down))
    return fail(MOE_ERR_INVALID_ARG, "inter_shared > 0 but a shared-expert weight is NULL");
  const void* ptrs[] = {x, router_w, router_bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
                        y, topk_ids_out, topk_w_out};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(MOE_ERR_UNSUPPORTED, "pointer %p not 16-byte aligned", q);
  if (c->tokens > moe::kFusedMaxTokens || c->tokens * c->top_k > moe::kFusedMaxPairs)
    return fail(MOE_ERR_UNSUPPORTED,
                "single-launch path takes tokens <= %d and tokens * top_k <= %d (got %lld, %lld)",
                moe::kFusedMaxTokens, moe::kFusedMaxPairs, (long long)c->tokens,
                (long long)(c->tokens * c->top_k));
  Plan p;
  make_plan(c, &p);
  if ((st = check_ws(p, ws, ws_bytes))) return st;
  if (p.T == 0) return ok();

  moe::FusedArgs f{};
  f.g = expert_args(p, c, x, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, ws);
  f.wg = router_w;
  f.bias = router_bias;
  f.zpart = at<float>(ws, p.zpart);
  f.S = p.S;
  f.pl = partial_layout(p);
  f.scaling = c->routed_scaling;
  f.renorm = c->renormalize ? 1 : 0;
  f.ids = topk_ids_out ? topk_ids_out : at<int32_t>(ws, p.ids);
  f.w = topk_w_out ? topk_w_out : at<float>(ws, p.w);
  f.offsets = at<int32_t>(ws, p.offsets);
  f.sorted = at<int32_t>(ws, p.sorted);
  f.w_sorted = at<float>(ws, p.wsorted);
  f.pos = at<int32_t>(ws, p.pos);
  f.tiles = at<int2>(ws, p.tiles);
  f.tile_cap = p.tile_cap;
  f.y = y;
  f.ctl = at<uint32_t>(ws, p.ctl);
  MOE_CHECK_LAUNCH(moe::launch_fused(f, stream), "fused forward");
  return ok();
}

// ---- dense SwiGLU FFN: the expert GEMMs with one group of all T rows.
struct DensePlan {
  int64_t T;
  int H, I;
  int shape, tile_cap;
  size_t tiles, ntiles, queue, h, total;
};

moe_status validate_dense(const moe_dense_config* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "config is NULL");
  if (c->tokens < 0) return fail(MOE_ERR_INVALID_ARG, "tokens < 0 (%lld)", (long long)c->tokens);
  if (c->hidden <= 0 || c->inter <= 0)
    return fail(MOE_ERR_INVALID_ARG, "non-positive size (hidden %d, inter %d)", c->hidden, c->inter);
  if (c->reserved != 0) return fail(MOE_ERR_INVALID_ARG, "reserved field must be 0");
  if (c->hidden % 128)
    return fail(MOE_ERR_UNSUPPORTED, "hidden %d is not a multiple of 128", c->hidden);
  if (c->inter % 64) return fail(MOE_ERR_UNSUPPORTED, "inter %d not a multiple of 64", c->inter);
  if (c->tokens * static_cast<int64_t>(std::max(c->hidden, c->inter)) >= (int64_t(1) << 32))
    return fail(MOE_ERR_UNSUPPORTED, "tokens * max(hidden, inter) must be < 2^32");
  return MOE_OK;
}

void make_dense_plan(const moe_dense_config* c, DensePlan* p) {
  p->T = c->tokens;
  p->H = c->hidden;
  p->I = c->inter;
  // One group of T rows: big tiles once the rows outnumber a few tiles.
  const bool fits = p->H % 256 == 0 && p->I % 128 == 0;
  p->shape = (fits && p->T >= 1024) ? moe::kTileBig : moe::kTileSmall;
  const int bm = moe::experts_tile_rows(p->shape);
  p->tile_cap = static_cast<int>(std::max<int64_t>(1, (p->T + bm - 1) / bm));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  p->tiles = take(static_cast<size_t>(p->tile_cap) * 8);
  p->ntiles = take(16);
  p->queue = take(moe::kQueueWords * 4);
  p->h = take(static_cast<size_t>(p->T) * p->I * 2);
  p->total = off;
}

// ---- fixed scratch of moe_forward_noalloc.
// The workspace of moe_forward (router partials, permutation, GEMM tile
// lists and queue counters, h and o) lives in this file-scope device array
// instead of caller memory.  Each device holds its own copy, allocated by the
// runtime when the library's code object is loaded there, for the life of the
// process.  Host code never names the array for its memory: its device
// address is taken once per device with hipGetSymbolAddress and kept here.
static_assert(MOE_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on its first use).
moe_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "device %d beyond the %d devices with a scratch slot", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_dense_workspace_size(const moe_dense_config* cfg) {
  if (validate_dense(cfg) != MOE_OK) return 0;
  DensePlan p;
  make_dense_plan(cfg, &p);
  return p.total;
}

moe_status moe_dense_forward(const moe_dense_config* cfg, const uint16_t* x,
                             const uint16_t* w_gate, const uint16_t* w_up,
                             const uint16_t* w_down, uint16_t* y, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  moe_status st = validate_dense(cfg);
  if (st) return st;
  if (!w_gate || !w_up || !w_down || (cfg->tokens > 0 && (!x || !y)))
    return fail(MOE_ERR_INVALID_ARG, "a required pointer is NULL");
  const void* ptrs[] = {x, w_gate, w_up, w_down, y};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(MOE_ERR_UNSUPPORTED, "pointer %p not 16-byte aligned", q);
  DensePlan p;
  make_dense_plan(cfg, &p);
  if (!ws) return fail(MOE_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned16(ws)) return fail(MOE_ERR_UNSUPPORTED, "workspace not 16-byte aligned");
  if (ws_bytes < p.total)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, p.total);
  if (p.T == 0) return ok();

  // The MLP is the expert GEMMs' shared group (group index E = 0): no routed
  // experts, weight 1.0, its output written straight into y.
  moe::ExpertArgs g{};
  g.x = x;
  g.k = 1;
  g.T = p.T;
  g.H = p.H;
  g.I = 0;
  g.Is = p.I;
  g.E = 0;
  g.ws_gate = w_gate;
  g.ws_up = w_up;
  g.ws_down = w_down;
  g.limit_shared = cfg->swiglu_limit;
  g.tiles = at<int2>(ws, p.tiles);
  g.ntiles = at<int32_t>(ws, p.ntiles);
  g.queue = at<uint32_t>(ws, p.queue);
  g.h_shared = at<uint16_t>(ws, p.h);
  g.o_shared = y;
  MOE_CHECK_LAUNCH(moe::launch_dense_tiles(at<int2>(ws, p.tiles), at<int32_t>(ws, p.ntiles),
                                           g.queue, p.T, moe::experts_tile_rows(p.shape), 0,
                                           stream),
                   "dense tile list");
  MOE_CHECK_LAUNCH(moe::launch_gateup(g, p.shape, p.tile_cap, stream), "dense gate/up gemm");
  MOE_CHECK_LAUNCH(moe::launch_down(g, p.shape, p.tile_cap, stream), "dense down gemm");
  return ok();
}

size_t moe_workspace_size(const moe_config* cfg) {
  if (validate(cfg) != MOE_OK) return 0;
  Plan p;
  make_plan(cfg, &p);
  return p.total;
}

const char* moe_last_error(void) { return g_error.c_str(); }

moe_status moe_route(const moe_config* cfg, const uint16_t* x, const float* router_w,
                     const float* router_bias, int32_t* topk_ids, float* topk_w, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  moe_status st = validate(cfg);
  if (st) return st;
  if (!router_w || (cfg->tokens > 0 && (!x || !topk_ids || !topk_w)))
    return fail(MOE_ERR_INVALID_ARG, "a required pointer is NULL");
  const void* ptrs[] = {x, router_w, router_bias, topk_ids, topk_w};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(MOE_ERR_UNSUPPORTED, "pointer %p not 16-byte aligned", q);
  Plan p;
  make_plan(cfg, &p);
  if ((st = check_ws(p, ws, ws_bytes))) return st;
  if (p.T == 0) return ok();
  if ((st = route_impl(p, cfg, x, router_w, router_bias, topk_ids, topk_w, ws, stream, nullptr)))
    return st;
  return ok();
}

moe_status moe_permute(const moe_config* cfg, const int32_t* topk_ids, int32_t* expert_offsets,
                       int32_t* sorted_pairs, int32_t* pair_pos, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  moe_status st = validate(cfg);
  if (st) return st;
  if (!expert_offsets || (cfg->tokens > 0 && (!topk_ids || !sorted_pairs || !pair_pos)))
    return fail(MOE_ERR_INVALID_ARG, "a required pointer is NULL");
  const void* ptrs[] = {topk_ids, expert_offsets, sorted_pairs, pair_pos};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(MOE_ERR_UNSUPPORTED, "pointer %p not 16-byte aligned", q);
  Plan p;
  make_plan(cfg, &p);
  if ((st = check_ws(p, ws, ws_bytes))) return st;
  if (p.T == 0) {
    // Offsets of an empty batch are all zero; nothing else to write.
    MOE_CHECK_LAUNCH(moe::launch_fill_zero(expert_offsets, p.E + 1, stream), "zero offsets");
    return ok();
  }
  if ((st = permute_impl(p, topk_ids, expert_offsets, sorted_pairs, pair_pos, nullptr, ws, stream,
                         nullptr)))
    return st;
  return ok();
}

moe_status moe_forward(const moe_config* cfg, const uint16_t* x, const float* router_w,
                       const float* router_bias, const uint16_t* w_gate, const uint16_t* w_up,
                       const uint16_t* w_down, const uint16_t* ws_gate, const uint16_t* ws_up,
                       const uint16_t* ws_down, uint16_t* y, int32_t* topk_ids_out,
                       float* topk_w_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return forward_impl(cfg, x, router_w, router_bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
                      y, topk_ids_out, topk_w_out, ws, ws_bytes, stream, nullptr);
}

moe_status moe_forward_timed(const moe_config* cfg, const uint16_t* x, const float* router_w,
                             const float* router_bias, const uint16_t* w_gate,
                             const uint16_t* w_up, const uint16_t* w_down,
                             const uint16_t* ws_gate, const uint16_t* ws_up,
                             const uint16_t* ws_down, uint16_t* y, int32_t* topk_ids_out,
                             float* topk_w_out, void* ws, size_t ws_bytes, hipStream_t stream,
                             hipEvent_t* events, int n_events) {
  if (!events || n_events != MOE_NUM_STAGES + 1)
    return fail(MOE_ERR_INVALID_ARG, "moe_forward_timed needs %d events", MOE_NUM_STAGES + 1);
  for (int i = 0; i < n_events; ++i)
    if (!events[i]) return fail(MOE_ERR_INVALID_ARG, "event %d is NULL", i);
  return forward_impl(cfg, x, router_w, router_bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
                      y, topk_ids_out, topk_w_out, ws, ws_bytes, stream, events);
}

moe_status moe_forward_fp8(const moe_config* cfg, const uint16_t* x, const float* router_w,
                           const float* router_bias, const uint8_t* w8_gate, const uint8_t* w8_up,
                           const uint8_t* w8_down, const float* scale_gate,
                           const float* scale_up, const float* scale_down,
                           const uint16_t* ws_gate, const uint16_t* ws_up,
                           const uint16_t* ws_down, uint16_t* y, int32_t* topk_ids_out,
                           float* topk_w_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  const Fp8Weights f8{w8_gate, w8_up, w8_down, scale_gate, scale_up, scale_down};
  return forward_impl(cfg, x, router_w, router_bias, nullptr, nullptr, nullptr, ws_gate, ws_up,
                      ws_down, y, topk_ids_out, topk_w_out, ws, ws_bytes, stream, nullptr, &f8);
}

moe_status moe_forward_fused(const moe_config* cfg, const uint16_t* x, const float* router_w,
                             const float* router_bias, const uint16_t* w_gate,
                             const uint16_t* w_up, const uint16_t* w_down,
                             const uint16_t* ws_gate, const uint16_t* ws_up,
                             const uint16_t* ws_down, uint16_t* y, int32_t* topk_ids_out,
                             float* topk_w_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return forward_fused_impl(cfg, x, router_w, router_bias, w_gate, w_up, w_down, ws_gate, ws_up,
                            ws_down, y, topk_ids_out, topk_w_out, ws, ws_bytes, stream);
}

moe_status moe_forward_noalloc(const moe_config* cfg, const uint16_t* x, const float* router_w,
                               const float* router_bias, const uint16_t* w_gate,
                               const uint16_t* w_up, const uint16_t* w_down,
                               const uint16_t* ws_gate, const uint16_t* ws_up,
                               const uint16_t* ws_down, uint16_t* y, int32_t* topk_ids_out,
                               float* topk_w_out, hipStream_t stream) {
  moe_status st = check_forward_args(cfg, x, router_w, router_bias, w_gate, w_up, w_down, ws_gate,
                                     ws_up, ws_down, y, topk_ids_out, topk_w_out, nullptr);
  if (st) return st;
  Plan p;
  make_plan(cfg, &p);
  if (p.total > static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES))
    return fail(MOE_ERR_WORKSPACE,
                "moe_forward_noalloc: this batch needs %zu bytes of workspace, the fixed scratch "
                "holds %zu (use moe_forward with a caller workspace)",
                p.total, static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES));
  if (p.T == 0) return ok();
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  return forward_impl(cfg, x, router_w, router_bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down,
                      y, topk_ids_out, topk_w_out, ws, MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

moe_status moe_workspace_view(const moe_config* cfg, int which, size_t* offset, size_t* bytes) {
  moe_status st = validate(cfg);
  if (st) return st;
  if (!offset || !bytes) return fail(MOE_ERR_INVALID_ARG, "offset/bytes is NULL");
  Plan p;
  make_plan(cfg, &p);
  const size_t P = static_cast<size_t>(p.P), T = static_cast<size_t>(p.T);
  switch (which) {
    case MOE_WS_TOPK_IDS: *offset = p.ids; *bytes = P * 4; break;
    case MOE_WS_TOPK_W: *offset = p.w; *bytes = P * 4; break;
    case MOE_WS_EXPERT_OFFSETS: *offset = p.offsets; *bytes = (static_cast<size_t>(p.E) + 1) * 4; break;
    case MOE_WS_SORTED_PAIRS: *offset = p.sorted; *bytes = P * 4; break;
    case MOE_WS_PAIR_POS: *offset = p.pos; *bytes = P * 4; break;
    case MOE_WS_H: *offset = p.h; *bytes = (P * p.I + T * p.Is) * 2; break;
    case MOE_WS_O: *offset = p.o; *bytes = (P + (p.Is > 0 ? T : 0)) * p.H * 2; break;
    case MOE_WS_FUSED_CTL: *offset = p.ctl; *bytes = static_cast<size_t>(moe::kCtlWords) * 4; break;
    case MOE_WS_FUSED_STATUS: *offset = p.ctl + moe::kCtlStatus * 4; *bytes = 4; break;
    default: return fail(MOE_ERR_INVALID_ARG, "unknown workspace buffer id %d", which);
  }
  return ok();
}

}  // extern "C"
