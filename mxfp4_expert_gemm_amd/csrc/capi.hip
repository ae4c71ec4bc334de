// C ABI of the MXFP4 Stable-LatentMoE layer: argument checks, workspace layout and
// the order of kernels on the caller's stream.  No device memory is allocated here.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "common.h"
#include "kernels.h"

using namespace moe;

namespace {

constexpr int MAX_K = 64;
constexpr int MAX_E = 1024;    // experts held in registers by the routing wave
constexpr int MAX_DIM = 8192;  // columns a GEMV wave holds in registers
constexpr int MAX_EXPERT_DIM = 7168;  // latent / FFN width whose staged activation rows fit LDS
constexpr int MAX_SHARED = 8;

// Experts run as grouped GEMMs over 64-row tiles once they hold 8 routed rows on
// average; below that, the streaming kernels that read each expert once per 4 rows.
bool use_gemm(int64_t rows, int32_t E) { return rows >= 8 * (int64_t)E; }

// REAP partials per routed row: the latent-row blocks of the down kernel the batch runs
int32_t sal_chunks(const moe_config& c, int k) {
  if (down_combine_fits(c.num_tokens, k)) return down_combine_sal_chunks(c.d_latent);
  if (use_gemm(c.num_tokens * k, c.num_experts)) return down_gemm_sal_chunks(c.d_latent);
  return down_mx_sal_chunks(c.d_latent);
}

struct Layout {
  size_t logits_fast, xnorm, wnorm, idx, w, counts, offsets, perm, tiles, nact, permws, h, y, z, gtiles, salp;
  // the grouping renumbered to HBM slots (experts fetched from host memory)
  size_t tiles_s, counts_s, offsets_s, idx_s;
  // shared experts: x split for the matrix cores, their grouping, GLU rows, outputs
  size_t xq_hi, xq_lo, xq_shi, xq_slo, s_counts, s_offsets, s_perm, s_tiles, s_nact, sq_hi, sq_lo, sq_shi, sq_slo, s_y,
      s_gtiles;
  size_t hq_hi, hq_lo, hq_shi, hq_slo, aq_hi, aq_lo, aq_shi, aq_slo;
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
  l.xnorm = take(T * 4);
  l.wnorm = take(E * 4);
  l.idx = take(T * K * 4);
  l.w = take(T * K * 4);
  l.counts = take(E * 4);
  l.offsets = take((E + 1) * 4);
  l.perm = take(T * K * 4);
  l.tiles = take(E * 16);
  l.nact = take(4);
  l.permws = take(permute_ws_bytes((int64_t)(T * K), (int32_t)E));
  l.h = take(T * L * 2);
  l.hq_hi = take(T * L);
  l.hq_lo = take(T * L);
  l.hq_shi = take(T * L / 32);
  l.hq_slo = take(T * L / 32);
  l.aq_hi = take(T * K * F);
  l.aq_lo = take(T * K * F);
  l.aq_shi = take(T * K * F / 32);
  l.aq_slo = take(T * K * F / 32);
  l.y = take(T * K * L * 4);
  l.z = take(T * L * 2);
  l.gtiles = take(gemm_tiles_bytes((int64_t)(T * K), (int32_t)E));
  l.salp = take(T * K * (size_t)sal_chunks(c, k) * 8);
  l.tiles_s = take(E * 16);
  l.counts_s = take(E * 4);
  l.offsets_s = take((E + 1) * 4);
  l.idx_s = take(T * K * 4);
  const size_t S = (size_t)c.num_shared, D = (size_t)c.d_model, FS = (size_t)c.d_ffn_shared;
  l.xq_hi = l.xq_lo = l.xq_shi = l.xq_slo = l.s_counts = l.s_offsets = l.s_perm = l.s_tiles = l.s_nact = l.sq_hi =
      l.sq_lo = l.sq_shi = l.sq_slo = l.s_y = l.s_gtiles = 0;
  if (S > 0) {
    l.xq_hi = take(T * D);
    l.xq_lo = take(T * D);
    l.xq_shi = take(T * D / 32);
    l.xq_slo = take(T * D / 32);
    l.s_counts = take(S * 4);
    l.s_offsets = take((S + 1) * 4);
    l.s_perm = take(T * S * 4);
    l.s_tiles = take(S * 16);
    l.s_nact = take(4);
    l.sq_hi = take(T * S * FS);
    l.sq_lo = take(T * S * FS);
    l.sq_shi = take(T * S * FS / 32);
    l.sq_slo = take(T * S * FS / 32);
    l.s_y = take(T * S * D * 4);
    l.s_gtiles = take(gemm_tiles_bytes((int64_t)(T * S), (int32_t)S));
  }
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
  if (c->expert_layout != MOE_LAYOUT_RECORD && c->expert_layout != MOE_LAYOUT_PACKED) return MOE_ERR_INVALID_ARG;
  if (c->act_format != MOE_ACT_FMT_BF16 && c->act_format != MOE_ACT_FMT_MXFP8) return MOE_ERR_INVALID_ARG;
  if (c->num_shared < 0 || c->num_shared > MAX_SHARED || c->d_ffn_shared < 0 || c->d_ffn_shared % 32 ||
      (c->num_shared > 0 && c->d_ffn_shared == 0))
    return MOE_ERR_INVALID_ARG;
  // shared experts run the expert kernels at the full width d
  if (c->num_shared > 0 && (c->d_model > MAX_EXPERT_DIM || c->d_model % 128 || c->d_ffn_shared > MAX_EXPERT_DIM ||
                            c->d_ffn_shared % 128))
    return MOE_ERR_UNSUPPORTED;
  if (c->act == MOE_ACT_SITU) return MOE_ERR_UNSUPPORTED;  // formula not defined on the pages
  // sizes this build's kernels hold in registers; the expert GEMV also needs 128-column multiples
  if (c->num_experts > MAX_E || c->d_model > MAX_DIM || c->d_latent > MAX_EXPERT_DIM || c->d_ffn > MAX_EXPERT_DIM ||
      c->d_latent % 128 || c->d_ffn % 128)
    return MOE_ERR_UNSUPPORTED;
  if (c->num_tokens > (int64_t)1 << 24 || c->num_tokens * k > (int64_t)INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int32_t max_tiles(int64_t rows, int32_t E) { return (int32_t)(rows < E ? rows : E); }


moe_status dev(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

#define MOE_TRY(expr)                 \
  do {                                \
    moe_status _s = (expr);           \
    if (_s != MOE_OK) return _s;      \
  } while (0)

// gate/up then down (y fp32 by routed row) with the kernel family the batch calls for
moe_status run_experts_on(const MxArgs& mx, int64_t rows, int32_t E, const int32_t* counts, const int32_t* offsets,
                          int4* gt, hipStream_t st) {
  if (use_gemm(rows, E)) {
    const int64_t mt = gemm_max_tiles(rows, E);
    MOE_TRY(dev(launch_gemm_tiles(counts, offsets, E, gt, mt, st)));
    MOE_TRY(dev(launch_gateup_gemm(mx, gt, mt, st)));
    return dev(launch_down_gemm(mx, gt, mt, st));
  }
  MOE_TRY(dev(launch_gateup_mx(mx, st)));
  return dev(launch_down_mx(mx, st));
}
moe_status run_experts(const MxArgs& mx, const moe_config& c, int k, const int32_t* counts, const int32_t* offsets,
                       void* ws, const Layout& l, hipStream_t st) {
  return run_experts_on(mx, c.num_tokens * k, c.num_experts, counts, offsets, at<int4>(ws, l.gtiles), st);
}

// The grouping of the shared experts' rows, known in closed form: every token t has row
// t*S + s for every shared expert s, so expert s owns rows s*T .. s*T + T-1 of perm
// (tokens ascending), counts T and offset s*T; its tile is {s, s*T, T, s}.
__global__ void shared_group_kernel(int32_t* counts, int32_t* offsets, int32_t* perm, int4* tiles, int32_t* nact,
                                    int64_t T, int32_t S) {
  const int64_t n = T * S;
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < n; r += (int64_t)gridDim.x * blockDim.x) {
    const int64_t s = r / T, t = r - s * T;
    perm[r] = (int32_t)(t * S + s);
  }
  if (blockIdx.x == 0) {
    for (int s = threadIdx.x; s <= S; s += blockDim.x) {
      offsets[s] = (int32_t)(s * T);
      if (s < S) {
        counts[s] = (int32_t)T;
        tiles[s] = make_int4(s, (int)(s * T), (int)T, s);
      }
    }
    if (threadIdx.x == 0) *nact = S;
  }
}

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
  segs[0].wnorm = at<float>(ws, l.wnorm);
  segs[0].xnorm = at<float>(ws, l.xnorm);
  int nseg = 1;
  if (latent_down) {
    segs[1].W = static_cast<const uint16_t*>(latent_down);
    segs[1].rows = c.d_latent;
    segs[1].router = 0;
    segs[1].out = at<uint16_t>(ws, l.h);
    segs[1].wnorm = nullptr;
    segs[1].xnorm = nullptr;
    nseg = 2;
  }
  return dev(launch_dense(static_cast<const uint16_t*>(x), c.num_tokens, c.d_model, segs, nseg, st));
}

RouteArgs route_args(const moe_config& c, int k, int flags, const void* x, const void* router_w, const float* bias,
                     int32_t* idx, float* w, float* logits_out, void* ws, const Layout& l) {
  RouteArgs a;
  a.logits_fast = at<float>(ws, l.logits_fast);
  a.xnorm = at<float>(ws, l.xnorm);
  a.wnorm = at<float>(ws, l.wnorm);
  a.gamma = dense_router_gamma(c.num_tokens, c.d_model);
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
  a.stats = nullptr;
  a.h = nullptr;
  a.L = c.d_latent;
  a.mxfp8 = c.act_format == MOE_ACT_FMT_MXFP8;
  a.hq = QRows{nullptr, nullptr, nullptr, nullptr};
  return a;
}

QRows hq_rows(void* ws, const Layout& l) {
  return QRows{at<uint8_t>(ws, l.hq_hi), at<uint8_t>(ws, l.hq_lo), at<uint8_t>(ws, l.hq_shi), at<uint8_t>(ws, l.hq_slo)};
}
QRows aq_rows(void* ws, const Layout& l) {
  return QRows{at<uint8_t>(ws, l.aq_hi), at<uint8_t>(ws, l.aq_lo), at<uint8_t>(ws, l.aq_shi), at<uint8_t>(ws, l.aq_slo)};
}

MxArgs mx_args(const moe_config& c, int k, const uint8_t* blob, void* ws, const Layout& l, const int32_t* perm,
               float* y) {
  MxArgs m;
  m.blob = blob;
  m.packed = c.expert_layout == MOE_LAYOUT_PACKED;
  m.L = c.d_latent;
  m.F = c.d_ffn;
  m.k = k;
  m.T = c.num_tokens;
  m.tiles = at<int4>(ws, l.tiles);
  m.max_active = max_tiles(c.num_tokens * k, c.num_experts);
  m.perm = perm;
  m.hq = hq_rows(ws, l);
  m.aq = aq_rows(ws, l);
  m.mxfp8 = c.act_format == MOE_ACT_FMT_MXFP8;
  m.a_bf16 = nullptr;
  m.y = y;
  m.clock = nullptr;
  m.sal = nullptr;
  m.sal_chunks = 0;
  return m;
}

// ---- scratch of the entry point without a workspace argument
// One file-scope device array: each GPU the library runs on holds its own copy until the
// process ends.  On the host its name is only a stand-in, not the device address: the
// address comes from hipGetSymbolAddress, once per device with that device current, and
// only that address is ever passed to kernels.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mutex;
void* scratch_addr[MAX_DEVICES];

// the scratch's device address on the device that owns `stream`, which must be current
moe_status scratch_for(hipStream_t stream, void** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur < 0 || cur >= MAX_DEVICES) return MOE_ERR_DEVICE;
  if (stream) {
    hipDevice_t sd = -1;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return MOE_ERR_DEVICE;
    if (sd != cur) return MOE_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_addr[cur]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_DEVICE;
    scratch_addr[cur] = p;
  }
  *out = scratch_addr[cur];
  return MOE_OK;
}

// ---- the second stream the shared experts run on
// One per device, created at the first call that needs it while the caller's stream is not
// being captured, and kept until the process ends: default priority, no implicit
// synchronisation with the null stream.  The caller's stream records `fork`, the side
// stream waits on it, runs the shared experts and records `join`, and the caller's stream
// waits on `join` before the latent-up projection: an event fork and join, which stream
// capture records as graph edges.  `use` is held from the fork to the join's wait, so
// calls on one device from several host threads take the side stream one at a time.
struct SideStream {
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex use;
};
std::mutex side_mutex;
SideStream side_streams[MAX_DEVICES];

// the side stream of the device that owns `st`; *out stays null when there is none and
// none may be made now (the caller's stream is being captured): the shared experts then
// run on the caller's stream
moe_status side_for(hipStream_t st, SideStream** out) {
  *out = nullptr;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return MOE_ERR_DEVICE;
  int device = cur;
  if (st) {
    hipDevice_t sd = -1;
    if (hipStreamGetDevice(st, &sd) != hipSuccess) return MOE_ERR_DEVICE;
    device = sd;
  }
  if (device < 0 || device >= MAX_DEVICES) return MOE_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(side_mutex);
  SideStream& s = side_streams[device];
  if (!s.side) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) return MOE_ERR_DEVICE;
    if (cs != hipStreamCaptureStatusNone) return MOE_OK;
    if (device != cur && hipSetDevice(device) != hipSuccess) return MOE_ERR_DEVICE;
    hipStream_t side = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    bool ok = hipStreamCreateWithFlags(&side, hipStreamNonBlocking) == hipSuccess &&
              hipEventCreateWithFlags(&fork, hipEventDisableTiming) == hipSuccess &&
              hipEventCreateWithFlags(&join, hipEventDisableTiming) == hipSuccess;
    if (device != cur && hipSetDevice(cur) != hipSuccess) ok = false;
    if (!ok) {
      if (join) (void)hipEventDestroy(join);
      if (fork) (void)hipEventDestroy(fork);
      if (side) (void)hipStreamDestroy(side);
      return MOE_ERR_DEVICE;
    }
    s.fork = fork;
    s.join = join;
    s.side = side;
  }
  *out = &s;
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_expert_bytes(int32_t d_latent, int32_t d_ffn) {
  if (d_latent <= 0 || d_ffn <= 0 || d_latent % 32 || d_ffn % 32) return 0;
  size_t wts = (size_t)3 * (size_t)d_latent * (size_t)d_ffn;
  return wts / 2 + wts / 32;
}

size_t moe_packed_expert_bytes(int32_t d_latent, int32_t d_ffn) {
  if (d_latent <= 0 || d_ffn <= 0 || d_latent % 128 || d_ffn % 128) return 0;
  return (size_t)packed_expert_bytes(d_latent, d_ffn);
}

moe_status moe_pack_experts(const uint8_t* blob, int32_t num_experts, int32_t d_latent, int32_t d_ffn,
                            uint8_t* packed, moe_stream_t stream) {
  if (num_experts < 0 || d_latent <= 0 || d_ffn <= 0 || d_latent % 128 || d_ffn % 128) return MOE_ERR_INVALID_ARG;
  if (num_experts == 0) return MOE_OK;
  if (!blob || !packed || !aligned16(blob) || !aligned16(packed)) return MOE_ERR_INVALID_ARG;
  const size_t in = (size_t)num_experts * moe_expert_bytes(d_latent, d_ffn);
  const size_t outb = (size_t)num_experts * moe_packed_expert_bytes(d_latent, d_ffn);
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(blob), b0 = reinterpret_cast<uintptr_t>(packed);
  if (a0 < b0 + outb && b0 < a0 + in) return MOE_ERR_INVALID_ARG;  // overlap
  return dev(launch_pack_experts(blob, packed, num_experts, d_latent, d_ffn, reinterpret_cast<hipStream_t>(stream)));
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

// the shared experts on x at the full width: every token's rows t*S + s, grouped by shared
// expert, through the same expert kernels; their fp32 outputs (s_y) join the latent-up
// product before its bf16 rounding
static moe_status run_shared(const moe_config& c, const void* x, const uint8_t* shared_blob, void* ws,
                             const Layout& l, hipStream_t st) {
  const int32_t S = c.num_shared;
  const int64_t rows = c.num_tokens * S;
  const QRows xq{at<uint8_t>(ws, l.xq_hi), at<uint8_t>(ws, l.xq_lo), at<uint8_t>(ws, l.xq_shi),
                 at<uint8_t>(ws, l.xq_slo)};
  MOE_TRY(dev(launch_quantize_rows(static_cast<const uint16_t*>(x), c.num_tokens, c.d_model, xq,
                                   c.act_format == MOE_ACT_FMT_MXFP8, st)));
  PermOut ps{at<int32_t>(ws, l.s_counts), at<int32_t>(ws, l.s_offsets), at<int32_t>(ws, l.s_perm),
             at<int4>(ws, l.s_tiles), at<int32_t>(ws, l.s_nact), S};
  const int64_t gblocks = ceil_div(rows, 256) < 1024 ? ceil_div(rows, 256) : 1024;
  hipLaunchKernelGGL(shared_group_kernel, dim3((unsigned)gblocks), dim3(256), 0, st, ps.counts, ps.offsets, ps.perm,
                     ps.tiles, ps.n_active, c.num_tokens, S);
  MOE_TRY(dev(hipGetLastError()));
  MxArgs ms;
  ms.blob = shared_blob;
  ms.packed = c.expert_layout == MOE_LAYOUT_PACKED;
  ms.L = c.d_model;
  ms.F = c.d_ffn_shared;
  ms.k = S;
  ms.T = c.num_tokens;
  ms.tiles = ps.tiles;
  ms.max_active = S;
  ms.perm = ps.perm;
  ms.hq = xq;
  ms.aq = QRows{at<uint8_t>(ws, l.sq_hi), at<uint8_t>(ws, l.sq_lo), at<uint8_t>(ws, l.sq_shi),
                at<uint8_t>(ws, l.sq_slo)};
  ms.mxfp8 = c.act_format == MOE_ACT_FMT_MXFP8;
  ms.a_bf16 = nullptr;
  ms.y = at<float>(ws, l.s_y);
  ms.clock = nullptr;
  ms.sal = nullptr;
  ms.sal_chunks = 0;
  return run_experts_on(ms, rows, S, ps.counts, ps.offsets, at<int4>(ws, l.s_gtiles), st);
}

// expert_slots non-null: expert_blob is device-readable host memory, and the experts
// the batch routes to are copied into the slots first
static moe_status forward_impl(const void* x, const void* router_w, const void* latent_down, const void* latent_up,
                               const uint8_t* expert_blob, int32_t k, const moe_config* cfg, const float* router_bias,
                               const uint8_t* shared_blob, void* out, moe_routing_out* routing, void* workspace,
                               size_t workspace_bytes, const moe_stage_events* ev, moe_stream_t stream,
                               uint8_t* expert_slots = nullptr, size_t slots_bytes = 0) {
  MOE_TRY(check_config(cfg, k));
  const moe_config& c = *cfg;
  if (c.num_shared > 0 && (!shared_blob || !aligned16(shared_blob))) return MOE_ERR_INVALID_ARG;
  if (c.num_tokens == 0) return MOE_OK;  // nothing to do; pointers may be NULL
  if (!x || !router_w || !latent_down || !latent_up || !expert_blob || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(router_w) || !aligned16(latent_down) || !aligned16(latent_up) ||
      !aligned16(expert_blob) || !aligned16(out))
    return MOE_ERR_INVALID_ARG;
  if (router_bias && (reinterpret_cast<uintptr_t>(router_bias) & 3u)) return MOE_ERR_INVALID_ARG;
  if (routing && routing->saliency && (reinterpret_cast<uintptr_t>(routing->saliency) & 7u)) return MOE_ERR_INVALID_ARG;
  const int64_t ebytes = c.expert_layout == MOE_LAYOUT_PACKED ? packed_expert_bytes(c.d_latent, c.d_ffn)
                                                             : (int64_t)moe_expert_bytes(c.d_latent, c.d_ffn);
  const int32_t nslots = max_tiles(c.num_tokens * k, c.num_experts);
  if (expert_slots) {
    if (!aligned16(expert_slots) || slots_bytes < (size_t)nslots * (size_t)ebytes) return MOE_ERR_INVALID_ARG;
    if (c.num_experts > 1024) return MOE_ERR_UNSUPPORTED;
  }
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
  // events stamped by the dispatch of a stage's main kernel
  auto kclock = [&](int stage) {
    return ev ? reinterpret_cast<unsigned long long*>(ev->kernel_clock[stage]) : nullptr;
  };
  auto kev = [&](int stage) {
    KernelEvents k;
    if (ev) {
      k.begin = reinterpret_cast<hipEvent_t>(ev->kernel_begin[stage]);
      k.end = reinterpret_cast<hipEvent_t>(ev->kernel_end[stage]);
    }
    return k;
  };

  // the shared experts depend on x alone: they run beside the routed path, on a second
  // stream, and join it before the latent-up projection
  SideStream* side = nullptr;
  std::unique_lock<std::mutex> side_lock;
  if (c.num_shared > 0) MOE_TRY(side_for(st, &side));
  if (side) side_lock = std::unique_lock<std::mutex>(side->use);
  moe_status shared_status = MOE_OK;
  if (side) {
    MOE_TRY(dev(hipEventRecord(side->fork, st)));
    MOE_TRY(dev(hipStreamWaitEvent(side->side, side->fork, 0)));
    shared_status = run_shared(c, x, shared_blob, ws, l, side->side);
    MOE_TRY(dev(hipEventRecord(side->join, side->side)));
  }
  auto routed = [&]() -> moe_status {
    int32_t* idx = routing && routing->topk_idx ? routing->topk_idx : at<int32_t>(ws, l.idx);
    float* w = routing && routing->topk_w ? routing->topk_w : at<float>(ws, l.w);
    int32_t* counts = routing && routing->expert_counts ? routing->expert_counts : at<int32_t>(ws, l.counts);
    int32_t* offsets = routing && routing->expert_offsets ? routing->expert_offsets : at<int32_t>(ws, l.offsets);
    int32_t* perm = routing && routing->perm ? routing->perm : at<int32_t>(ws, l.perm);
    float* logits_out = routing ? routing->logits : nullptr;

    MOE_TRY(mark(MOE_STAGE_ROUTER_DOWN, true));
    MOE_TRY(run_router_and_down(c, x, router_w, latent_down, ws, l, st));
    MOE_TRY(mark(MOE_STAGE_ROUTER_DOWN, false));
    RouteArgs ra = route_args(c, k, 0, x, router_w, router_bias, idx, w, logits_out, ws, l);
    ra.h = at<uint16_t>(ws, l.h);
    ra.hq = hq_rows(ws, l);
    PermOut po{counts, offsets, perm, at<int4>(ws, l.tiles), at<int32_t>(ws, l.nact),
               max_tiles(c.num_tokens * k, c.num_experts)};
    MOE_TRY(mark(MOE_STAGE_ROUTE, true));
    if (c.num_tokens <= ROUTE_FUSED_TOKENS) {
      MOE_TRY(dev(launch_route_permute_small(ra, po, st)));
      MOE_TRY(mark(MOE_STAGE_ROUTE, false));
      MOE_TRY(mark(MOE_STAGE_PERMUTE, true));
    } else if (c.num_tokens <= ROUTE_PLACE_TOKENS && c.num_tokens * k <= ROUTE_SMALL_ROWS) {
      MOE_TRY(dev(launch_route(ra, st)));
      MOE_TRY(mark(MOE_STAGE_ROUTE, false));
      MOE_TRY(mark(MOE_STAGE_PERMUTE, true));
      MOE_TRY(dev(launch_place_rows(idx, c.num_tokens, k, c.num_experts, po, st)));
    } else {
      MOE_TRY(dev(launch_route(ra, st)));
      MOE_TRY(mark(MOE_STAGE_ROUTE, false));
      MOE_TRY(mark(MOE_STAGE_PERMUTE, true));
      MOE_TRY(dev(launch_permute(idx, c.num_tokens * k, c.num_experts, po, at<void>(ws, l.permws), st)));
    }
    // the expert stage reads the blob, or the slots holding the routed experts' records
    const uint8_t* eblob = expert_blob;
    const int32_t* eidx = idx;
    const int32_t* ecounts = counts;
    const int32_t* eoffsets = offsets;
    int32_t E_eff = c.num_experts;
    int4* etiles = at<int4>(ws, l.tiles);
    if (expert_slots) {
      MOE_TRY(dev(launch_gather_experts(expert_blob, ebytes, etiles, at<int32_t>(ws, l.nact), nslots, expert_slots, st)));
      MOE_TRY(dev(launch_remap_to_slots(etiles, at<int32_t>(ws, l.nact), nslots, counts, offsets, idx, c.num_tokens * k,
                                        at<int4>(ws, l.tiles_s), at<int32_t>(ws, l.counts_s),
                                        at<int32_t>(ws, l.offsets_s), at<int32_t>(ws, l.idx_s), st)));
      eblob = expert_slots;
      eidx = at<int32_t>(ws, l.idx_s);
      ecounts = at<int32_t>(ws, l.counts_s);
      eoffsets = at<int32_t>(ws, l.offsets_s);
      E_eff = nslots;
      etiles = at<int4>(ws, l.tiles_s);
    }
    MOE_TRY(mark(MOE_STAGE_PERMUTE, false));
    MxArgs mx = mx_args(c, k, eblob, ws, l, perm, at<float>(ws, l.y));
    mx.tiles = etiles;
    double* saliency = routing ? routing->saliency : nullptr;
    if (saliency) {  // the down kernels write their REAP partials
      mx.sal = at<double>(ws, l.salp);
      mx.sal_chunks = sal_chunks(c, k);
    }
    if (down_combine_fits(c.num_tokens, k)) {
      MOE_TRY(mark(MOE_STAGE_GATE_UP, true));
      mx.clock = kclock(MOE_STAGE_GATE_UP);
      MOE_TRY(dev(launch_gateup_mx(mx, st, kev(MOE_STAGE_GATE_UP))));
      MOE_TRY(mark(MOE_STAGE_GATE_UP, false));
      MOE_TRY(mark(MOE_STAGE_DOWN, true));
      mx.clock = kclock(MOE_STAGE_DOWN);
      MOE_TRY(dev(launch_down_combine_mx(mx, eidx, w, at<uint16_t>(ws, l.z), st, kev(MOE_STAGE_DOWN))));
      MOE_TRY(mark(MOE_STAGE_DOWN, false));
      MOE_TRY(mark(MOE_STAGE_COMBINE, true));
      MOE_TRY(mark(MOE_STAGE_COMBINE, false));
    } else {
      const int64_t rows = c.num_tokens * k;
      const int64_t mt = gemm_max_tiles(rows, c.num_experts);
      int4* gt = at<int4>(ws, l.gtiles);
      const bool gemm = use_gemm(rows, c.num_experts);
      MOE_TRY(mark(MOE_STAGE_GATE_UP, true));
      mx.clock = kclock(MOE_STAGE_GATE_UP);
      if (gemm) {
        MOE_TRY(dev(launch_gemm_tiles(ecounts, eoffsets, E_eff, gt, mt, st)));
        MOE_TRY(dev(launch_gateup_gemm(mx, gt, mt, st, kev(MOE_STAGE_GATE_UP))));
      } else {
        MOE_TRY(dev(launch_gateup_mx(mx, st, kev(MOE_STAGE_GATE_UP))));
      }
      MOE_TRY(mark(MOE_STAGE_GATE_UP, false));
      MOE_TRY(mark(MOE_STAGE_DOWN, true));
      mx.clock = kclock(MOE_STAGE_DOWN);
      MOE_TRY(dev(gemm ? launch_down_gemm(mx, gt, mt, st, kev(MOE_STAGE_DOWN))
                       : launch_down_mx(mx, st, kev(MOE_STAGE_DOWN))));
      MOE_TRY(mark(MOE_STAGE_DOWN, false));
      MOE_TRY(mark(MOE_STAGE_COMBINE, true));
      MOE_TRY(dev(launch_combine(at<float>(ws, l.y), w, c.num_tokens, k, c.d_latent, at<uint16_t>(ws, l.z), st)));
      MOE_TRY(mark(MOE_STAGE_COMBINE, false));
    }
    if (saliency)
      MOE_TRY(dev(launch_reap_partials(mx.sal, mx.sal_chunks, w, perm, offsets, c.num_experts, saliency, st)));
    return MOE_OK;
  };
  moe_status routed_status = routed();
  // joined whatever the routed path returned, so a capture never ends with the side
  // stream still forked
  if (side) {
    const moe_status j = dev(hipStreamWaitEvent(st, side->join, 0));
    if (routed_status == MOE_OK) routed_status = j;
  }
  MOE_TRY(shared_status);
  MOE_TRY(routed_status);
  if (c.num_shared > 0 && !side) MOE_TRY(run_shared(c, x, shared_blob, ws, l, st));
  DenseSeg up;
  up.W = static_cast<const uint16_t*>(latent_up);
  up.rows = c.d_model;
  up.router = 0;
  up.out = out;
  up.wnorm = nullptr;
  up.xnorm = nullptr;
  MOE_TRY(mark(MOE_STAGE_UP, true));
  if (c.num_shared > 0) {
    up.add = at<float>(ws, l.s_y);
    up.add_rows = c.num_shared;
  }
  MOE_TRY(dev(launch_dense(at<uint16_t>(ws, l.z), c.num_tokens, c.d_latent, &up, 1, st)));
  return mark(MOE_STAGE_UP, false);
}

moe_status moe_layer_forward(const void* x, const void* router_w, const void* latent_down, const void* latent_up,
                             const uint8_t* expert_blob, int32_t k, const moe_config* cfg,
                             const float* router_bias, void* out, moe_routing_out* routing, void* workspace,
                             size_t workspace_bytes, moe_stream_t stream) {
  return forward_impl(x, router_w, latent_down, latent_up, expert_blob, k, cfg, router_bias, nullptr, out, routing,
                      workspace, workspace_bytes, nullptr, stream);
}

moe_status moe_layer_forward_noalloc(const void* x, const void* router_w, const void* latent_down,
                                     const void* latent_up, const uint8_t* expert_blob, int32_t k,
                                     const moe_config* cfg, const float* router_bias, void* out,
                                     moe_routing_out* routing, moe_stream_t stream) {
  MOE_TRY(check_config(cfg, k));
  if (cfg->num_shared > 0) return MOE_ERR_INVALID_ARG;
  if (cfg->num_tokens == 0) return MOE_OK;
  // refuse a batch whose scratch would not fit before anything touches the device
  if (layout(*cfg, k).total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  MOE_TRY(scratch_for(reinterpret_cast<hipStream_t>(stream), &ws));
  return forward_impl(x, router_w, latent_down, latent_up, expert_blob, k, cfg, router_bias, nullptr, out, routing,
                      ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, nullptr, stream);
}

moe_status moe_layer_forward_shared(const void* x, const void* router_w, const void* latent_down,
                                    const void* latent_up, const uint8_t* expert_blob, int32_t k,
                                    const moe_config* cfg, const float* router_bias, const uint8_t* shared_blob,
                                    void* out, moe_routing_out* routing, void* workspace, size_t workspace_bytes,
                                    moe_stream_t stream) {
  return forward_impl(x, router_w, latent_down, latent_up, expert_blob, k, cfg, router_bias, shared_blob, out,
                      routing, workspace, workspace_bytes, nullptr, stream);
}

moe_status moe_layer_forward_profiled(const void* x, const void* router_w, const void* latent_down,
                                      const void* latent_up, const uint8_t* expert_blob, int32_t k,
                                      const moe_config* cfg, const float* router_bias, void* out,
                                      moe_routing_out* routing, void* workspace, size_t workspace_bytes,
                                      const moe_stage_events* events, moe_stream_t stream) {
  return forward_impl(x, router_w, latent_down, latent_up, expert_blob, k, cfg, router_bias, nullptr, out, routing,
                      workspace, workspace_bytes, events, stream);
}

moe_status moe_expert_slots_bytes(const moe_config* cfg, int32_t k, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_config(cfg, k));
  const moe_config& c = *cfg;
  const int64_t ebytes = c.expert_layout == MOE_LAYOUT_PACKED ? packed_expert_bytes(c.d_latent, c.d_ffn)
                                                             : (int64_t)moe_expert_bytes(c.d_latent, c.d_ffn);
  *bytes = (size_t)max_tiles(c.num_tokens * k, c.num_experts) * (size_t)ebytes;
  return MOE_OK;
}

moe_status moe_layer_forward_streamed(const void* x, const void* router_w, const void* latent_down,
                                      const void* latent_up, const uint8_t* expert_blob_host, int32_t k,
                                      const moe_config* cfg, const float* router_bias, uint8_t* expert_slots,
                                      size_t slots_bytes, void* out, moe_routing_out* routing, void* workspace,
                                      size_t workspace_bytes, moe_stream_t stream) {
  if (!expert_slots) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_config(cfg, k));
  if (cfg->num_shared > 0 || cfg->num_experts > 1024) return MOE_ERR_UNSUPPORTED;
  if (cfg->num_tokens == 0) return MOE_OK;
  size_t need = 0;
  MOE_TRY(moe_expert_slots_bytes(cfg, k, &need));
  if (!aligned16(expert_slots) || slots_bytes < need || !expert_blob_host) return MOE_ERR_INVALID_ARG;
  // the device address of the pinned host records (host memory only: device memory and
  // unregistered host memory are refused)
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, expert_blob_host) != hipSuccess || attr.type != hipMemoryTypeHost)
    return MOE_ERR_INVALID_ARG;
  void* dblob = nullptr;
  if (hipHostGetDevicePointer(&dblob, const_cast<uint8_t*>(expert_blob_host), 0) != hipSuccess || !dblob)
    return MOE_ERR_INVALID_ARG;
  return forward_impl(x, router_w, latent_down, latent_up, static_cast<const uint8_t*>(dblob), k, cfg, router_bias,
                      nullptr, out, routing, workspace, workspace_bytes, nullptr, stream, expert_slots, slots_bytes);
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
  const RouteArgs ra = route_args(c, k, flags, x, router_w, router_bias, routing->topk_idx, routing->topk_w,
                                  routing->logits, workspace, l);
  return dev(launch_route(ra, st));
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

// The standalone grouping's workspace: the permutation's scratch, then the tile list
// and the active-expert count, each 256-byte aligned.
static size_t permute_stage_bytes(int64_t rows, int32_t num_experts, size_t* pws) {
  *pws = align_up(permute_ws_bytes(rows, num_experts), 256);
  return *pws + align_up((size_t)num_experts * 16, 256) + 256;
}

static moe_status check_permute_args(int64_t num_tokens, int32_t k, int32_t num_experts) {
  if (num_tokens < 0 || k < 1 || k > MAX_K || num_experts < 1 || k > num_experts) return MOE_ERR_INVALID_ARG;
  if (num_experts > MAX_E) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status moe_permute_workspace_size(int64_t num_tokens, int32_t k, int32_t num_experts, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_permute_args(num_tokens, k, num_experts));
  size_t pws = 0;
  *bytes = num_tokens == 0 ? 0 : permute_stage_bytes(num_tokens * k, num_experts, &pws);
  return MOE_OK;
}

moe_status moe_permute(const int32_t* topk_idx, int64_t num_tokens, int32_t k, int32_t num_experts,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm, void* workspace,
                       size_t workspace_bytes, moe_stream_t stream) {
  if (!topk_idx || !expert_counts || !expert_offsets || !perm) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_permute_args(num_tokens, k, num_experts));
  const int64_t rows = num_tokens * k;
  if (rows == 0) return MOE_OK;
  size_t pws = 0;
  const size_t need = permute_stage_bytes(rows, num_experts, &pws);
  if (!workspace || workspace_bytes < need) return MOE_ERR_WORKSPACE;
  PermOut po{expert_counts, expert_offsets, perm, at<int4>(workspace, pws),
             at<int32_t>(workspace, pws + align_up((size_t)num_experts * 16, 256)), max_tiles(rows, num_experts)};
  return dev(launch_permute(topk_idx, rows, num_experts, po, workspace, reinterpret_cast<hipStream_t>(stream)));
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
  int32_t* perm = at<int32_t>(ws, l.perm);
  PermOut po{at<int32_t>(ws, l.counts), at<int32_t>(ws, l.offsets), perm, at<int4>(ws, l.tiles),
             at<int32_t>(ws, l.nact), max_tiles(c.num_tokens * k, c.num_experts)};
  MOE_TRY(dev(launch_permute(routing->topk_idx, c.num_tokens * k, c.num_experts, po, at<void>(ws, l.permws), st)));
  MOE_TRY(dev(launch_quantize_rows(static_cast<const uint16_t*>(h), c.num_tokens, c.d_latent, hq_rows(ws, l),
                                   c.act_format == MOE_ACT_FMT_MXFP8, st)));
  MxArgs mx = mx_args(c, k, expert_blob, ws, l, perm, y);
  mx.a_bf16 = static_cast<uint16_t*>(a_out);
  return run_experts(mx, c, k, at<int32_t>(ws, l.counts), at<int32_t>(ws, l.offsets), ws, l, st);
}

moe_status moe_combine(const float* y, const float* topk_w, int64_t num_tokens, int32_t k, int32_t d_latent,
                       void* z, moe_stream_t stream) {
  if (!y || !topk_w || !z || num_tokens < 0 || k < 1 || d_latent <= 0 || d_latent % 32) return MOE_ERR_INVALID_ARG;
  if (!aligned16(y) || (reinterpret_cast<uintptr_t>(z) & 7u)) return MOE_ERR_INVALID_ARG;
  return dev(launch_combine(y, topk_w, num_tokens, k, d_latent, static_cast<uint16_t*>(z),
                            reinterpret_cast<hipStream_t>(stream)));
}

moe_status moe_reap_saliency(const float* y, const float* topk_w, const int32_t* perm, const int32_t* expert_offsets,
                             int64_t num_tokens, int32_t k, int32_t d_latent, int32_t num_experts, double* saliency,
                             moe_stream_t stream) {
  if (!y || !topk_w || !perm || !expert_offsets || !saliency || num_tokens < 0 || k < 1 || k > MAX_K ||
      d_latent <= 0 || num_experts < 1 || k > num_experts)
    return MOE_ERR_INVALID_ARG;
  if (num_tokens * k > (int64_t)INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (num_tokens == 0) return MOE_OK;
  return dev(launch_reap_saliency(y, topk_w, perm, expert_offsets, num_experts, d_latent, saliency,
                                  reinterpret_cast<hipStream_t>(stream)));
}

moe_status moe_reap_keep_bias(const double* saliency, int32_t num_experts, int32_t n_keep, float* bias,
                              moe_stream_t stream) {
  if (!saliency || !bias || num_experts < 1 || n_keep < 0 || n_keep > num_experts) return MOE_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(saliency) & 7u) || (reinterpret_cast<uintptr_t>(bias) & 3u))
    return MOE_ERR_INVALID_ARG;
  if (num_experts > MAX_E) return MOE_ERR_UNSUPPORTED;
  return dev(launch_reap_keep_bias(saliency, num_experts, n_keep, bias, reinterpret_cast<hipStream_t>(stream)));
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
  s.wnorm = nullptr;
  s.xnorm = nullptr;
  return dev(launch_dense(static_cast<const uint16_t*>(in), num_tokens, n_in, &s, 1,
                               reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
