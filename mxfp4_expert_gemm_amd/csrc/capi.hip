// C ABI of the MXFP4 Stable-LatentMoE layer: argument checks, workspace layout and
// the order of kernels on the caller's stream.  No device memory is allocated here.
#include <stdint.h>
#include <string.h>

#include "common.h"
#include "kernels.h"

using namespace moe;

namespace {

constexpr int MAX_K = 64;
constexpr int MAX_E = 1024;    // experts held in registers by the routing wave
constexpr int MAX_DIM = 8192;  // columns a GEMV wave holds in registers

struct Layout {
  size_t logits_fast, xnorm2, wnorm2, idx, w, counts, offsets, perm, active, nact, stats, permws, h, a, y, z;
  size_t total;
};

Layout layout(const moe_config& c, int k) {
  Layout l;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  const size_t T = (size_t)c.num_tokens, E = (size_t)c.num_experts, L = (size_t)c.d_latent,
               F = (size_t)c.d_ffn, K = (size_t)k;
  l.logits_fast = take(T * E * 4);
  l.xnorm2 = take(T * 4);
  l.wnorm2 = take(E * 4);
  l.idx = take(T * K * 4);
  l.w = take(T * K * 4);
  l.counts = take(E * 4);
  l.offsets = take((E + 1) * 4);
  l.perm = take(T * K * 4);
  l.active = take(E * 4);
  l.nact = take(4);
  l.stats = take(16);
  l.permws = take(permute_ws_bytes((int64_t)(T * K), (int32_t)E));
  l.h = take(T * L * 2);
  l.a = take(T * K * F * 2);
  l.y = take(T * K * L * 4);
  l.z = take(T * L * 2);
  l.total = off;
  return l;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na && nb && x < y + nb && y < x + na;
}

moe_status check_config(const moe_config* c, int32_t k) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->num_tokens < 0 || c->d_model <= 0 || c->d_latent <= 0 || c->d_ffn <= 0 || c->num_experts <= 0)
    return MOE_ERR_INVALID_ARG;
  if (c->d_model % 32 || c->d_latent % 32 || c->d_ffn % 32) return MOE_ERR_INVALID_ARG;
  if (k < 1 || k > c->num_experts || k > MAX_K) return MOE_ERR_INVALID_ARG;
  if (c->act != MOE_ACT_SILU && c->act != MOE_ACT_SITU) return MOE_ERR_INVALID_ARG;
  if (c->renormalize != 0 && c->renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (c->bias_row_stride != 0 && c->bias_row_stride != c->num_experts) return MOE_ERR_INVALID_ARG;
  if (c->act == MOE_ACT_SITU) return MOE_ERR_UNSUPPORTED;  // formula not defined on the pages
  // sizes this build's kernels hold in registers; the expert GEMV also needs 128-column multiples
  if (c->num_experts > MAX_E || c->d_model > MAX_DIM || c->d_latent > MAX_DIM || c->d_ffn > MAX_DIM ||
      c->d_latent % 128 || c->d_ffn % 128)
    return MOE_ERR_UNSUPPORTED;
  if (c->num_tokens > (int64_t)1 << 24 || c->num_tokens * k > (int64_t)INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status dev(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

#define MOE_TRY(expr)                 \
  do {                                \
    moe_status _s = (expr);           \
    if (_s != MOE_OK) return _s;      \
  } while (0)

__global__ void fill_i32_kernel(int32_t* p, int n, int32_t v) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

moe_status zero_i32(int32_t* p, int n, hipStream_t st) {
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, st, p, n, 0);
  return dev(hipGetLastError());
}

// router logits (fast, with norms) and optionally the latent down projection, in one launch
moe_status run_router_and_down(const moe_config& c, const void* x, const void* router_w, const void* latent_down,
                               void* ws, const Layout& l, hipStream_t st) {
  DenseSeg segs[2];
  segs[0].W = static_cast<const uint16_t*>(router_w);
  segs[0].rows = c.num_experts;
  segs[0].router = 1;
  segs[0].out = at<float>(ws, l.logits_fast);
  segs[0].wnorm2 = at<float>(ws, l.wnorm2);
  segs[0].xnorm2 = at<float>(ws, l.xnorm2);
  int nseg = 1;
  if (latent_down) {
    segs[1].W = static_cast<const uint16_t*>(latent_down);
    segs[1].rows = c.d_latent;
    segs[1].router = 0;
    segs[1].out = at<uint16_t>(ws, l.h);
    segs[1].wnorm2 = nullptr;
    segs[1].xnorm2 = nullptr;
    nseg = 2;
  }
  return dev(launch_dense_gemv(static_cast<const uint16_t*>(x), c.num_tokens, c.d_model, segs, nseg, st));
}

moe_status run_route(const moe_config& c, int k, int flags, const void* x, const void* router_w,
                     const float* bias, int32_t* idx, float* w, float* logits_out, void* ws, const Layout& l,
                     hipStream_t st) {
  RouteArgs a;
  a.logits_fast = at<float>(ws, l.logits_fast);
  a.xnorm2 = at<float>(ws, l.xnorm2);
  a.wnorm2 = at<float>(ws, l.wnorm2);
  a.gamma = GEMV_ROUTER_GAMMA;
  a.exact_logits = nullptr;
  a.bias = bias;
  a.bias_stride = c.bias_row_stride;
  a.x = static_cast<const uint16_t*>(x);
  a.router_w = static_cast<const uint16_t*>(router_w);
  a.d = c.d_model;
  a.T = c.num_tokens;
  a.E = c.num_experts;
  a.k = k;
  a.renormalize = c.renormalize;
  a.flags = flags;
  a.idx = idx;
  a.w = w;
  a.logits_out = logits_out;
  a.stats = at<int32_t>(ws, l.stats);
  MOE_TRY(zero_i32(a.stats, 4, st));
  return dev(launch_route(a, st));
}

ExpertArgs expert_args(const moe_config& c, int k, const void* h, const uint8_t* blob, void* ws, const Layout& l,
                       const int32_t* counts, const int32_t* offsets, const int32_t* perm, float* y) {
  ExpertArgs e;
  e.h = static_cast<const uint16_t*>(h);
  e.blob = blob;
  e.L = c.d_latent;
  e.F = c.d_ffn;
  e.k = k;
  e.T = c.num_tokens;
  e.counts = counts;
  e.offsets = offsets;
  e.perm = perm;
  e.active = at<int32_t>(ws, l.active);
  e.n_active = at<int32_t>(ws, l.nact);
  int64_t rows = c.num_tokens * k;
  e.max_active = (int32_t)(rows < c.num_experts ? rows : c.num_experts);
  e.a = at<uint16_t>(ws, l.a);
  e.y = y;
  return e;
}

}  // namespace

extern "C" {

size_t moe_expert_bytes(int32_t d_latent, int32_t d_ffn) {
  if (d_latent <= 0 || d_ffn <= 0 || d_latent % 32 || d_ffn % 32) return 0;
  size_t wts = (size_t)3 * (size_t)d_latent * (size_t)d_ffn;
  return wts / 2 + wts / 32;
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
  }
  return "MOE_ERR_UNKNOWN";
}

moe_status moe_workspace_size(const moe_config* cfg, int32_t k, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_config(cfg, k));
  *bytes = layout(*cfg, k).total;
  return MOE_OK;
}

static moe_status forward_impl(const void* x, const void* router_w, const void* latent_down, const void* latent_up,
                               const uint8_t* expert_blob, int32_t k, const moe_config* cfg, const float* router_bias,
                               void* out, moe_routing_out* routing, void* workspace, size_t workspace_bytes,
                               const moe_stage_events* ev, moe_stream_t stream) {
  MOE_TRY(check_config(cfg, k));
  const moe_config& c = *cfg;
  if (c.num_tokens == 0) return MOE_OK;  // nothing to do; pointers may be NULL
  if (!x || !router_w || !latent_down || !latent_up || !expert_blob || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(router_w) || !aligned16(latent_down) || !aligned16(latent_up) ||
      !aligned16(expert_blob) || !aligned16(out))
    return MOE_ERR_INVALID_ARG;
  if (router_bias && (reinterpret_cast<uintptr_t>(router_bias) & 3u)) return MOE_ERR_INVALID_ARG;
  const size_t xbytes = (size_t)c.num_tokens * c.d_model * 2;
  if (overlap(x, xbytes, out, xbytes)) return MOE_ERR_INVALID_ARG;
  const Layout l = layout(c, k);
  if (!workspace || workspace_bytes < l.total) return MOE_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MOE_ERR_INVALID_ARG;
  if (overlap(workspace, l.total, x, xbytes) || overlap(workspace, l.total, out, xbytes)) return MOE_ERR_INVALID_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  void* ws = workspace;
  auto mark = [&](int stage, bool begin) -> moe_status {
    if (!ev) return MOE_OK;
    moe_event_t e = begin ? ev->begin[stage] : ev->end[stage];
    return e ? dev(hipEventRecord(reinterpret_cast<hipEvent_t>(e), st)) : MOE_OK;
  };

  int32_t* idx = routing && routing->topk_idx ? routing->topk_idx : at<int32_t>(ws, l.idx);
  float* w = routing && routing->topk_w ? routing->topk_w : at<float>(ws, l.w);
  int32_t* counts = routing && routing->expert_counts ? routing->expert_counts : at<int32_t>(ws, l.counts);
  int32_t* offsets = routing && routing->expert_offsets ? routing->expert_offsets : at<int32_t>(ws, l.offsets);
  int32_t* perm = routing && routing->perm ? routing->perm : at<int32_t>(ws, l.perm);
  float* logits_out = routing ? routing->logits : nullptr;

  MOE_TRY(mark(MOE_STAGE_ROUTER_DOWN, true));
  MOE_TRY(run_router_and_down(c, x, router_w, latent_down, ws, l, st));
  MOE_TRY(mark(MOE_STAGE_ROUTER_DOWN, false));
  MOE_TRY(mark(MOE_STAGE_ROUTE, true));
  MOE_TRY(run_route(c, k, 0, x, router_w, router_bias, idx, w, logits_out, ws, l, st));
  MOE_TRY(mark(MOE_STAGE_ROUTE, false));
  MOE_TRY(mark(MOE_STAGE_PERMUTE, true));
  MOE_TRY(dev(launch_permute(idx, c.num_tokens * k, c.num_experts, counts, offsets, perm, at<int32_t>(ws, l.active),
                             at<int32_t>(ws, l.nact), at<void>(ws, l.permws), st)));
  MOE_TRY(mark(MOE_STAGE_PERMUTE, false));
  ExpertArgs ea = expert_args(c, k, at<uint16_t>(ws, l.h), expert_blob, ws, l, counts, offsets, perm,
                              at<float>(ws, l.y));
  MOE_TRY(mark(MOE_STAGE_GATE_UP, true));
  MOE_TRY(dev(launch_expert_gateup(ea, st)));
  MOE_TRY(mark(MOE_STAGE_GATE_UP, false));
  MOE_TRY(mark(MOE_STAGE_DOWN, true));
  MOE_TRY(dev(launch_expert_down(ea, st)));
  MOE_TRY(mark(MOE_STAGE_DOWN, false));
  MOE_TRY(mark(MOE_STAGE_COMBINE, true));
  MOE_TRY(dev(launch_combine(at<float>(ws, l.y), w, c.num_tokens, k, c.d_latent, at<uint16_t>(ws, l.z), st)));
  MOE_TRY(mark(MOE_STAGE_COMBINE, false));
  DenseSeg up;
  up.W = static_cast<const uint16_t*>(latent_up);
  up.rows = c.d_model;
  up.router = 0;
  up.out = out;
  up.wnorm2 = nullptr;
  up.xnorm2 = nullptr;
  MOE_TRY(mark(MOE_STAGE_UP, true));
  MOE_TRY(dev(launch_dense_gemv(at<uint16_t>(ws, l.z), c.num_tokens, c.d_latent, &up, 1, st)));
  return mark(MOE_STAGE_UP, false);
}

moe_status moe_layer_forward(const void* x, const void* router_w, const void* latent_down, const void* latent_up,
                             const uint8_t* expert_blob, int32_t k, const moe_config* cfg,
                             const float* router_bias, void* out, moe_routing_out* routing, void* workspace,
                             size_t workspace_bytes, moe_stream_t stream) {
  return forward_impl(x, router_w, latent_down, latent_up, expert_blob, k, cfg, router_bias, out, routing,
                      workspace, workspace_bytes, nullptr, stream);
}

moe_status moe_layer_forward_profiled(const void* x, const void* router_w, const void* latent_down,
                                      const void* latent_up, const uint8_t* expert_blob, int32_t k,
                                      const moe_config* cfg, const float* router_bias, void* out,
                                      moe_routing_out* routing, void* workspace, size_t workspace_bytes,
                                      const moe_stage_events* events, moe_stream_t stream) {
  return forward_impl(x, router_w, latent_down, latent_up, expert_blob, k, cfg, router_bias, out, routing,
                      workspace, workspace_bytes, events, stream);
}

moe_status moe_dequant_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t cols, float* out,
                             moe_stream_t stream) {
  if (!codes || !scales || !out || rows < 0 || cols <= 0 || cols % 32) return MOE_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(out) & 7u) return MOE_ERR_INVALID_ARG;
  return dev(launch_dequant(codes, scales, rows, cols, out, reinterpret_cast<hipStream_t>(stream)));
}

moe_status moe_route(const void* x, const void* router_w, const float* router_bias, const moe_config* cfg,
                     int32_t k, int32_t flags, moe_routing_out* routing, void* workspace, size_t workspace_bytes,
                     moe_stream_t stream) {
  MOE_TRY(check_config(cfg, k));
  const moe_config& c = *cfg;
  if (flags & ~MOE_ROUTE_EXACT_ALL) return MOE_ERR_INVALID_ARG;
  if (c.num_tokens == 0) return MOE_OK;
  if (!x || !router_w || !routing || !routing->logits || !routing->topk_idx || !routing->topk_w)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(router_w)) return MOE_ERR_INVALID_ARG;
  const Layout l = layout(c, k);
  if (!workspace || workspace_bytes < l.total) return MOE_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  MOE_TRY(run_router_and_down(c, x, router_w, nullptr, workspace, l, st));
  return run_route(c, k, flags, x, router_w, router_bias, routing->topk_idx, routing->topk_w, routing->logits,
                   workspace, l, st);
}

moe_status moe_topk(const float* logits, int64_t num_tokens, int32_t num_experts, int32_t k, int32_t renormalize,
                    int32_t* topk_idx, float* topk_w, moe_stream_t stream) {
  if (!logits || !topk_idx || !topk_w || num_tokens < 0 || num_experts < 1 || k < 1 || k > num_experts ||
      k > MAX_K || (renormalize != 0 && renormalize != 1))
    return MOE_ERR_INVALID_ARG;
  if (num_experts > MAX_E) return MOE_ERR_UNSUPPORTED;
  if (num_tokens == 0) return MOE_OK;
  RouteArgs a;
  memset(&a, 0, sizeof a);
  a.exact_logits = logits;
  a.T = num_tokens;
  a.E = num_experts;
  a.k = k;
  a.renormalize = renormalize;
  a.idx = topk_idx;
  a.w = topk_w;
  return dev(launch_route(a, reinterpret_cast<hipStream_t>(stream)));
}

moe_status moe_permute(const int32_t* topk_idx, int64_t num_tokens, int32_t k, int32_t num_experts,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm, void* workspace,
                       size_t workspace_bytes, moe_stream_t stream) {
  if (!topk_idx || !expert_counts || !expert_offsets || !perm || num_tokens < 0 || k < 1 || k > MAX_K ||
      num_experts < 1 || k > num_experts)
    return MOE_ERR_INVALID_ARG;
  if (num_experts > MAX_E) return MOE_ERR_UNSUPPORTED;
  const int64_t rows = num_tokens * k;
  if (rows == 0) return MOE_OK;
  const size_t need = align_up(permute_ws_bytes(rows, num_experts), 256) + align_up((size_t)num_experts * 4, 256) + 256;
  if (!workspace || workspace_bytes < need) return MOE_ERR_WORKSPACE;
  void* pws = workspace;
  int32_t* active = at<int32_t>(workspace, align_up(permute_ws_bytes(rows, num_experts), 256));
  int32_t* nact = at<int32_t>(workspace, align_up(permute_ws_bytes(rows, num_experts), 256) +
                                             align_up((size_t)num_experts * 4, 256));
  return dev(launch_permute(topk_idx, rows, num_experts, expert_counts, expert_offsets, perm, active, nact, pws,
                            reinterpret_cast<hipStream_t>(stream)));
}

moe_status moe_expert_ffn(const void* h, const uint8_t* expert_blob, int32_t k, const moe_config* cfg,
                          const moe_routing_out* routing, float* y, void* a_out, void* workspace,
                          size_t workspace_bytes, moe_stream_t stream) {
  MOE_TRY(check_config(cfg, k));
  const moe_config& c = *cfg;
  if (c.num_tokens == 0) return MOE_OK;
  if (!h || !expert_blob || !routing || !routing->topk_idx || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(expert_blob) || !aligned16(y) || (a_out && !aligned16(a_out)))
    return MOE_ERR_INVALID_ARG;
  const Layout l = layout(c, k);
  if (!workspace || workspace_bytes < l.total) return MOE_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  void* ws = workspace;
  int32_t* counts = at<int32_t>(ws, l.counts);
  int32_t* offsets = at<int32_t>(ws, l.offsets);
  int32_t* perm = at<int32_t>(ws, l.perm);
  MOE_TRY(dev(launch_permute(routing->topk_idx, c.num_tokens * k, c.num_experts, counts, offsets, perm,
                             at<int32_t>(ws, l.active), at<int32_t>(ws, l.nact), at<void>(ws, l.permws), st)));
  ExpertArgs ea = expert_args(c, k, h, expert_blob, ws, l, counts, offsets, perm, y);
  MOE_TRY(dev(launch_expert_gateup(ea, st)));
  MOE_TRY(dev(launch_expert_down(ea, st)));
  if (a_out)
    MOE_TRY(dev(launch_unpermute_rows(ea.a, perm, c.num_tokens * k, c.d_ffn, static_cast<uint16_t*>(a_out), st)));
  return MOE_OK;
}

moe_status moe_combine(const float* y, const float* topk_w, int64_t num_tokens, int32_t k, int32_t d_latent,
                       void* z, moe_stream_t stream) {
  if (!y || !topk_w || !z || num_tokens < 0 || k < 1 || d_latent <= 0 || d_latent % 32) return MOE_ERR_INVALID_ARG;
  if (!aligned16(y) || (reinterpret_cast<uintptr_t>(z) & 7u)) return MOE_ERR_INVALID_ARG;
  return dev(launch_combine(y, topk_w, num_tokens, k, d_latent, static_cast<uint16_t*>(z),
                            reinterpret_cast<hipStream_t>(stream)));
}

moe_status moe_linear_bf16(const void* in, const void* W, int64_t num_tokens, int32_t n_in, int32_t n_out, void* out,
                           moe_stream_t stream) {
  if (!in || !W || !out || num_tokens < 0 || n_in <= 0 || n_out <= 0 || n_in % 32) return MOE_ERR_INVALID_ARG;
  if (!aligned16(in) || !aligned16(W) || (reinterpret_cast<uintptr_t>(out) & 1u)) return MOE_ERR_INVALID_ARG;
  if (n_in > MAX_DIM) return MOE_ERR_UNSUPPORTED;
  if (num_tokens == 0) return MOE_OK;
  DenseSeg s;
  s.W = static_cast<const uint16_t*>(W);
  s.rows = n_out;
  s.router = 0;
  s.out = out;
  s.wnorm2 = nullptr;
  s.xnorm2 = nullptr;
  return dev(launch_dense_gemv(static_cast<const uint16_t*>(in), num_tokens, n_in, &s, 1,
                               reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
