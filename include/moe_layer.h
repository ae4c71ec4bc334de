/*
 * moe_layer.h: C ABI of an MI355X (gfx950) implementation of one
 * Stable-LatentMoE layer whose routed experts stay in MXFP4.
 *
 * The layer (cited by page title and section):
 *  - router: per token, the top-k (k = 16 in Kimi K3) of E = 896 routed
 *    experts by router logit (kimi-k3-mlx digest, architecture table; the
 *    kimi-k3-in-c post's introduction: 16 of 896 experts wake per token);
 *    router weights are probabilities, renormalised over the experts kept
 *    (kimi-k3-mlx digest, REAP pruning section);
 *  - Stable LatentMoE: routed experts work in a 3584-wide latent space under
 *    the 7168-wide residual (kimi-k3-mlx digest, architecture table and the
 *    LatentMoE bullet), so the token is projected down (bf16 7168 -> 3584),
 *    the experts run in the latent space, their weighted sum is projected
 *    back up (bf16 3584 -> 7168);
 *  - each routed expert is a GLU FFN (gate, up, down; 3 x 3584 x 3072 weights)
 *    stored in MXFP4: 4-bit E2M1 codes, low nibble first, one e8m0 exponent
 *    per 32 consecutive weights, 17,547,264 bytes per expert (kimi-k3-in-c
 *    post, "experts that are already 4-bit MXFP4"; kimi-k3-mlx digest,
 *    quantisation tiers); the GLU activation runs in fp32 (kimi-k3-mlx
 *    digest, SiTU-GLU bullet).
 *
 * Readings fixed by this library where the pages are silent:
 *  - logits are fp32; the selection is that of the correctly rounded fp32
 *    value of the exact bf16 dot product, then + bias in one fp32 add; order is
 *    (logit descending, expert index ascending); +0 == -0; NaN ranks last.
 *    Selected ids are written in ascending order.  Weights: softmax over the
 *    k selected logits (renormalize = 1) or over all E (renormalize = 0).
 *  - expert record e sits at byte e * moe_expert_bytes(L, F) of the blob and
 *    holds gate [F][L], up [F][L], down [L][F]; each matrix is its code bytes
 *    (rows x cols/2, element 2j in the low nibble of byte j) followed by its
 *    scale bytes (rows x cols/32; scale s means 2^(s-127), 255 is NaN).
 *  - rounding points: h = bf16(x W_d^T); g, u fp32; a = bf16(act(g) * u);
 *    y fp32; z = bf16(sum_j w_j y_j); out = bf16(z W_u^T); round to nearest
 *    even.  act = SiLU; the SiTU formula is not on the pages, so
 *    MOE_ACT_SITU returns MOE_ERR_UNSUPPORTED.
 *
 * Conventions for every entry point:
 *  - bf16 tensors are passed as raw 16-bit patterns (void* / uint16_t*),
 *    row-major, contiguous.
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates no device memory and keeps no pointer after the enqueued work
 *    completes.  Scratch space comes from the caller's workspace, sized by
 *    moe_workspace_size().
 *  - Work is enqueued on `stream` (a hipStream_t; NULL is the default stream)
 *    and the call returns without waiting.  Argument errors are detected
 *    before anything is enqueued and return synchronously; a failed launch
 *    returns MOE_ERR_DEVICE.
 *  - num_tokens == 0 is a no-op returning MOE_OK.
 *  - Calls on distinct workspaces are independent.  The library's only global
 *    state is the scratch array of moe_layer_forward_noalloc and the side stream
 *    (with its two events) of moe_layer_forward_shared, one of each per device.
 */
#ifndef MOE_LAYER_H
#define MOE_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A hipStream_t (HIP declares hipStream_t as struct ihipStream_t*). */
typedef struct ihipStream_t* moe_stream_t;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,  /* NULL, bad size, misalignment, aliasing */
  MOE_ERR_UNSUPPORTED = -2,  /* a valid but unimplemented option (e.g. MOE_ACT_SITU) */
  MOE_ERR_WORKSPACE = -3,    /* workspace NULL or smaller than moe_workspace_size() */
  MOE_ERR_DEVICE = -4        /* a HIP launch or runtime call failed */
} moe_status;

typedef enum { MOE_ACT_SILU = 0, MOE_ACT_SITU = 1 } moe_act;

/* Activation format at the expert GEMM inputs (moe_config.act_format).
 *  MOE_ACT_FMT_BF16: the bf16 latent rows h and GLU rows a as they are (the products
 *    are those of the bf16 values; the kernels split each value exactly into two e4m3
 *    terms).  The default.
 *  MOE_ACT_FMT_MXFP8: h and a quantised to MXFP8 first, the format the hardware
 *    deep-dive blog's QAT section names for the activations: per 32 consecutive
 *    values an e8m0 scale 2^X, X = floor(log2 max|v|) - 8 (clamped to the e8m0 range;
 *    byte 0 for a block of zeros), and E4M3 elements v / 2^X rounded to nearest even and
 *    saturated to +-448 (the OCP Microscaling v1.0 convention; the pages give no
 *    rounding or saturation rule).  One matrix-core product per K step instead of two;
 *    the output moves by the E4M3 rounding (about 4% relative at the K3 shapes). */
typedef enum { MOE_ACT_FMT_BF16 = 0, MOE_ACT_FMT_MXFP8 = 1 } moe_act_format;

/* Expert weight layouts (moe_config.expert_layout).
 *  MOE_LAYOUT_RECORD: E records of moe_expert_bytes(L, F) in the checkpoint order of
 *    the kimi-k3-in-c post, MXFP4 section: gate [F][L], up [F][L], down [L][F], each
 *    matrix its E2M1 codes row-major (two per byte, low nibble first) followed by its
 *    e8m0 scales row-major (one per 32 consecutive weights of a row).
 *  MOE_LAYOUT_PACKED: the same codes and scales, reordered by moe_pack_experts so that
 *    the kernels stream every load as one contiguous run: E records of
 *    moe_packed_expert_bytes(L, F); in a record gate, up, down; a matrix of R rows and
 *    K columns is R/16 groups of 16 rows, a group K/128 code tiles of 1024 bytes (tile
 *    s, bytes 16l..16l+15: row l%16 of the group, its weights 128s+32(l/16) ..
 *    128s+32(l/16)+31) then ceil(K/512) scale tiles of 256 bytes (tile c, byte 4l+j:
 *    the scale of those 32 weights for s = 4c+j, 127 where s >= K/128).  Same size as
 *    the record when L and F are multiples of 512. */
typedef enum { MOE_LAYOUT_RECORD = 0, MOE_LAYOUT_PACKED = 1 } moe_expert_layout;

/* Route flags (moe_route only). */
enum {
  /* recompute every logit exactly instead of only the ones near the top-k
   * boundary (for tests of the exact path) */
  MOE_ROUTE_EXACT_ALL = 1
};

typedef struct {
  int64_t num_tokens;   /* T >= 0 */
  int32_t d_model;      /* d, multiple of 32, at most 8192 */
  int32_t d_latent;     /* L, multiple of 32; the layer call needs a multiple of 128, at most 7168 */
  int32_t d_ffn;        /* F, likewise */
  int32_t num_experts;  /* E >= 1, at most 1024 */
  int32_t act;          /* moe_act */
  int32_t renormalize;  /* 1: softmax over the k selected logits; 0: over all E */
  int64_t bias_row_stride; /* router bias: 0 -> one fp32 [E] row for all tokens; E -> fp32 [T][E] */
  int32_t expert_layout;   /* moe_expert_layout of expert_blob */
  int32_t act_format;      /* moe_act_format of the expert GEMM inputs */
  int32_t num_shared;      /* always-on shared experts (0..8; needs moe_layer_forward_shared) */
  int32_t d_ffn_shared;    /* their FFN width F_s (multiple of 128, at most 7168; 0 if none) */
} moe_config;

/* Optional routing outputs of moe_layer_forward / inputs+outputs of the stage
 * calls.  Every member may be NULL in moe_layer_forward. */
typedef struct {
  int32_t* topk_idx;       /* [T][k] expert ids, ascending within a row */
  float* topk_w;           /* [T][k] routing weights */
  float* logits;           /* [T][E] fp32 logits incl. bias; entries recomputed
                              exactly near the top-k boundary are exact, the rest
                              are within the certified error bound */
  int32_t* expert_counts;  /* [E] rows routed to each expert */
  int32_t* expert_offsets; /* [E+1] exclusive prefix of expert_counts */
  int32_t* perm;           /* [T*k] row t*k+j of each routed (token, slot), grouped by
                              expert, tokens ascending inside a group */
  double* saliency;        /* [E] fp64, 8-byte aligned: the layer adds the REAP sums of
                              this batch, saliency[e] += sum over e's routed rows r of
                              topk_w[r] * ||y[r]||_2 (as moe_reap_saliency), from partial
                              sums the down kernels write; accumulated across calls */
} moe_routing_out;

/* Bytes of one expert record: 3 * L * F weights at 0.53125 B (kimi-k3-in-c
 * post, MXFP4 section).  0 if L or F is not a positive multiple of 32. */
size_t moe_expert_bytes(int32_t d_latent, int32_t d_ffn);

/* Bytes of one expert in MOE_LAYOUT_PACKED; 0 if L or F is not a positive
 * multiple of 128. */
size_t moe_packed_expert_bytes(int32_t d_latent, int32_t d_ffn);

/* Reorders num_experts checkpoint records (MOE_LAYOUT_RECORD, 16-byte aligned) into
 * MOE_LAYOUT_PACKED at packed (num_experts * moe_packed_expert_bytes, 16-byte
 * aligned, not overlapping blob).  A pure byte permutation, run once when the
 * weights are loaded.  L and F multiples of 128. */
moe_status moe_pack_experts(const uint8_t* blob, int32_t num_experts, int32_t d_latent, int32_t d_ffn,
                            uint8_t* packed, moe_stream_t stream);

/* Human-readable name of a status. */
const char* moe_status_string(moe_status s);

/* Workspace bytes needed by moe_layer_forward and by every stage call for this
 * config and k.  Writes *bytes; MOE_ERR_INVALID_ARG for a bad config. */
moe_status moe_workspace_size(const moe_config* cfg, int32_t k, size_t* bytes);

/*
 * The whole layer: out[T][d] (bf16) for x[T][d] (bf16).
 *   router_w     bf16 [E][d]
 *   latent_down  bf16 [L][d]     (h = x W_d^T)
 *   latent_up    bf16 [d][L]     (out = z W_u^T)
 *   expert_blob  E experts in cfg->expert_layout, 16-byte aligned
 *   k            experts per token, 1 <= k <= min(E, 64)
 *   router_bias  nullable fp32, shape per cfg->bias_row_stride
 *   routing      nullable; non-NULL members receive the routing
 * x, out and workspace must not overlap; every pointer 16-byte aligned.
 */
moe_status moe_layer_forward(const void* x, const void* router_w, const void* latent_down,
                             const void* latent_up, const uint8_t* expert_blob, int32_t k,
                             const moe_config* cfg, const float* router_bias, void* out,
                             moe_routing_out* routing, void* workspace, size_t workspace_bytes,
                             moe_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): moe_layer_forward without the
 * workspace argument.  Its scratch is one device array of MOE_NOALLOC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends; the call allocates
 * nothing (no hipMalloc, no allocating library routine).
 *  - A batch whose moe_workspace_size(cfg, k) exceeds MOE_NOALLOC_SCRATCH_BYTES returns
 *    MOE_ERR_WORKSPACE before anything is enqueued (at the Kimi K3 shapes, d 7168,
 *    L 3584, F 3072, E 896, k 16: up to 184 tokens).
 *  - Every call on one GPU uses that GPU's one array, which keeps the last call's
 *    contents (the layer needs no part of it cleared): calls that overlap on one GPU
 *    (other streams, other host threads) race, and the caller must serialise them.
 *  - stream must belong to the current device (else MOE_ERR_INVALID_ARG).
 *  - cfg->num_shared must be 0.  Other arguments and the result as moe_layer_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_layer_forward_noalloc(const void* x, const void* router_w, const void* latent_down,
                                     const void* latent_up, const uint8_t* expert_blob, int32_t k,
                                     const moe_config* cfg, const float* router_bias, void* out,
                                     moe_routing_out* routing, moe_stream_t stream);

/* Stages of moe_layer_forward, in launch order. */
typedef enum {
  MOE_STAGE_ROUTER_DOWN = 0, /* router logits and latent down projection (one launch) */
  MOE_STAGE_ROUTE = 1,       /* certified top-k, weights */
  MOE_STAGE_PERMUTE = 2,     /* grouping of routed rows by expert */
  MOE_STAGE_GATE_UP = 3,     /* MXFP4 gate/up GEMMs with the fp32 GLU */
  MOE_STAGE_DOWN = 4,        /* MXFP4 down GEMMs */
  MOE_STAGE_COMBINE = 5,     /* weighted combine */
  MOE_STAGE_UP = 6,          /* latent up projection */
  MOE_NUM_STAGES = 7
} moe_stage;

/* A hipEvent_t (HIP declares it as struct ihipEvent_t*). */
typedef struct ihipEvent_t* moe_event_t;

/* Timing of the stages (every entry may be NULL; NULL entries are skipped):
 *  begin/end: caller-created events recorded on the stream right before and right after
 *    the kernels of each stage (hipEventRecord), so a stage's span includes its launch
 *    gaps;
 *  kernel_begin/kernel_end: caller-created events stamped by the dispatch of the stage's
 *    main kernel itself (hipExtLaunchKernelGGL) at that kernel's start and end, so they
 *    time the kernel alone (eager calls; not recorded into a graph);
 *  kernel_clock: device pointers to 2 * MOE_CLOCK_SLOTS uint64 each, which the caller
 *    sets to pairs {UINT64_MAX, 0} before the stage runs; block b of the stage's main
 *    kernel lowers pair b % MOE_CLOCK_SLOTS's first word to the block's start and raises
 *    its second word to the block's end, in ticks of the device's constant-rate wall
 *    clock (hipDeviceAttributeWallClockRate kHz).  The kernel's span is the least first
 *    word to the greatest second word.  The pointers are kernel arguments, so they also
 *    work in a captured graph, on every replay.
 *  The kernel_* entries are honoured for MOE_STAGE_GATE_UP (the gate/up kernel) and
 *  MOE_STAGE_DOWN (the down kernel, fused with the combine for up to 64 routed rows) and
 *  ignored for the other stages. */
#define MOE_CLOCK_SLOTS 1024
typedef struct {
  moe_event_t begin[MOE_NUM_STAGES];
  moe_event_t end[MOE_NUM_STAGES];
  moe_event_t kernel_begin[MOE_NUM_STAGES];
  moe_event_t kernel_end[MOE_NUM_STAGES];
  uint64_t* kernel_clock[MOE_NUM_STAGES];
} moe_stage_events;

/* moe_layer_forward with hipEventRecord calls around its stages, for timing
 * individual kernels on the stream they run on.  Same arguments, same result. */
moe_status moe_layer_forward_profiled(const void* x, const void* router_w, const void* latent_down,
                                      const void* latent_up, const uint8_t* expert_blob, int32_t k,
                                      const moe_config* cfg, const float* router_bias, void* out,
                                      moe_routing_out* routing, void* workspace, size_t workspace_bytes,
                                      const moe_stage_events* events, moe_stream_t stream);

/* The layer with cfg->num_shared always-on shared experts (kimi-k3-mlx digest,
 * architecture table: two per token; LatentMoE bullet: they work at the full width,
 * not in the latent).  The pages give neither their width nor their format; this
 * build's reading: each is a SiLU-GLU expert on the token x, stored like a routed
 * expert (the same record layout, cfg->expert_layout) with (L, F) = (d_model,
 * d_ffn_shared), so shared_blob holds num_shared records of
 * moe_expert_bytes(d_model, d_ffn_shared) (or the packed size); each has weight 1, and
 * its fp32 output is added to the latent-up product before the one bf16 rounding:
 *   out[t] = bf16(z[t] . W_u^T + sum_s y_s(x[t])).
 * x is split for the matrix cores in cfg->act_format like h.  The workspace grows by
 * the shared rows (moe_workspace_size accounts for them).  moe_layer_forward is this
 * call with num_shared = 0; with num_shared > 0 it returns MOE_ERR_INVALID_ARG.
 * shared_blob: device, 16-byte aligned.
 * The shared experts depend on x alone, so they run beside the routed path on a second
 * stream that the library creates once per device (default priority, non-blocking) at
 * the first call whose stream is not being captured, and keeps until the process ends:
 * `stream` records an event, the side stream waits on it, runs the shared experts and
 * records a second event that `stream` waits on before the latent-up projection.  Stream
 * capture records this fork and join as graph edges.  A first call made while `stream`
 * is being captured runs the shared experts on `stream` itself (same result).  Calls on
 * one device from several host threads take the side stream one at a time. */
moe_status moe_layer_forward_shared(const void* x, const void* router_w, const void* latent_down,
                                    const void* latent_up, const uint8_t* expert_blob, int32_t k,
                                    const moe_config* cfg, const float* router_bias, const uint8_t* shared_blob,
                                    void* out, moe_routing_out* routing, void* workspace, size_t workspace_bytes,
                                    moe_stream_t stream);

/* Bytes of the HBM slot buffer moe_layer_forward_streamed needs: one expert record
 * (moe_expert_bytes, or moe_packed_expert_bytes for the packed layout) per expert a
 * batch can activate, min(E, T*k) of them.  Host function. */
moe_status moe_expert_slots_bytes(const moe_config* cfg, int32_t k, size_t* bytes);

/* The layer with its expert records held in host memory (in-c post, sections on how the
 * memory requirement shrinks and on streaming the trunk: only the experts a token routes
 * to need to be near the compute; a Kimi K3 has 92 routed layers of 15.7 GB of experts,
 * 1.45 TB, more than the 288 GB of HBM).  After the routing and the grouping, a kernel
 * copies the record of every active expert (at most min(E, T*k)) from the host blob
 * into expert_slots over the host link, and the expert kernels read the slots.  No host
 * synchronisation: the active-expert list never leaves the device.  Same result as
 * moe_layer_forward on the same records, bit for bit.
 *  expert_blob_host: host memory allocated pinned (hipHostMalloc; torch pin_memory),
 *    E records in cfg->expert_layout; the library maps it with hipHostGetDevicePointer
 *    and returns MOE_ERR_INVALID_ARG for memory that is not pinned host memory.
 *  expert_slots: device, 16-byte aligned, slots_bytes >= moe_expert_slots_bytes.
 *  cfg->num_experts at most 1024; cfg->num_shared must be 0 (MOE_ERR_UNSUPPORTED).
 *  Other arguments as moe_layer_forward; the routing outputs keep the global expert ids. */
moe_status moe_layer_forward_streamed(const void* x, const void* router_w, const void* latent_down,
                                      const void* latent_up, const uint8_t* expert_blob_host, int32_t k,
                                      const moe_config* cfg, const float* router_bias, uint8_t* expert_slots,
                                      size_t slots_bytes, void* out, moe_routing_out* routing, void* workspace,
                                      size_t workspace_bytes, moe_stream_t stream);

/* ---- stage entry points (the same kernels moe_layer_forward runs) ---- */

/* Dequantise one [rows][cols] MXFP4 matrix (codes then scales as above) to
 * fp32, bit-exact: E2M1(code) * 2^(s-127), inf past the fp32 range, NaN for
 * s = 255.  cols multiple of 32.  No workspace. */
moe_status moe_dequant_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t rows, int32_t cols,
                             float* out, moe_stream_t stream);

/* Router logits and exact top-k selection: fills routing->logits, topk_idx,
 * topk_w (all three required).  flags: MOE_ROUTE_*.  Uses the workspace. */
moe_status moe_route(const void* x, const void* router_w, const float* router_bias,
                     const moe_config* cfg, int32_t k, int32_t flags, moe_routing_out* routing,
                     void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* Selection alone on caller-given fp32 logits [T][E] (no certification: the
 * given logits are taken as exact).  Writes idx [T][k] and w [T][k]. */
moe_status moe_topk(const float* logits, int64_t num_tokens, int32_t num_experts, int32_t k,
                    int32_t renormalize, int32_t* topk_idx, float* topk_w, moe_stream_t stream);

/* Grouping of routed rows by expert: from idx [T][k] fill counts [E],
 * offsets [E+1], perm [T*k] (bit-exact, deterministic).  Uses a device
 * workspace of at least moe_permute_workspace_size(T, k, E) bytes, 16-byte
 * aligned (moe_workspace_size of a cfg with the same T and E is also enough);
 * MOE_ERR_WORKSPACE if it is smaller. */
moe_status moe_permute(const int32_t* topk_idx, int64_t num_tokens, int32_t k, int32_t num_experts,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm,
                       void* workspace, size_t workspace_bytes, moe_stream_t stream);

/* Bytes of device workspace moe_permute needs for T tokens of k rows over E
 * experts, written to *bytes (host pointer; 0 for T = 0).  Host-only, no device
 * call.  MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED as moe_permute would return. */
moe_status moe_permute_workspace_size(int64_t num_tokens, int32_t k, int32_t num_experts, size_t* bytes);

/* Routed experts on latent rows: h bf16 [T][L] -> y fp32 [T*k][L] with row
 * t*k+j the output of expert topk_idx[t][j] on h[t]; a_out (nullable) bf16
 * [T*k][F] receives the GLU output in the same row order.  routing must hold
 * topk_idx, expert_counts, expert_offsets and perm (from moe_permute).  An id may
 * repeat within a token (each slot is its own row); ids outside [0, E) are skipped:
 * their rows of y and a_out are left as they were. */
moe_status moe_expert_ffn(const void* h, const uint8_t* expert_blob, int32_t k, const moe_config* cfg,
                          const moe_routing_out* routing, float* y, void* a_out, void* workspace,
                          size_t workspace_bytes, moe_stream_t stream);

/* Weighted combine: z[t][l] = bf16(sum_j w[t][j] y[t*k+j][l]). */
moe_status moe_combine(const float* y, const float* topk_w, int64_t num_tokens, int32_t k,
                       int32_t d_latent, void* z, moe_stream_t stream);

/* REAP saliency (kimi-k3-mlx digest, REAP section: the score of expert j is the mean
 * over calibration tokens of the router weight g_j times the 2-norm of the expert's
 * output).  For every routed row r (slot t*k + j) of expert e:
 *   saliency[e] += topk_w[r] * ||y[r]||_2,
 * the rows of an expert taken in the order of perm (tokens ascending), norms and sums
 * in fp64.  y: fp32 [T*k][d_latent], the expert outputs by slot (moe_expert_ffn);
 * topk_w: fp32 [T*k] (moe_route); perm, expert_offsets: [T*k], [E+1] (moe_permute);
 * saliency: fp64 [num_experts] on the device, accumulated across calls (the caller
 * zeroes it, and divides by the number of calibration tokens at the end).  All device
 * pointers.  An expert pruned after scoring is a router bias of -inf on it in
 * moe_layer_forward / moe_route: it is never selected while k or more experts remain and
 * the weights are renormalised over the experts left.  With fewer than k left, every
 * survivor is selected and the other slots take the lowest-numbered pruned experts at
 * weight 0 (ties at -inf go to the lower index); that routing takes the general path,
 * where a pruned expert's logit is known to be exactly -inf and is not recomputed. */
moe_status moe_reap_saliency(const float* y, const float* topk_w, const int32_t* perm,
                             const int32_t* expert_offsets, int64_t num_tokens, int32_t k,
                             int32_t d_latent, int32_t num_experts, double* saliency,
                             moe_stream_t stream);

/* The router bias of a REAP-pruned layer (kimi-k3-mlx digest, REAP section: keep the
 * experts of highest saliency, e.g. 242 or 179 of 896): bias[e] = 0 for the n_keep
 * experts ranked first by saliency (higher first, ties to the lower index, NaN after
 * every number), -inf for the others.  saliency: fp64 [num_experts]; bias: fp32
 * [num_experts]; both device.  1 <= num_experts <= 1024 (else MOE_ERR_UNSUPPORTED),
 * 0 <= n_keep <= num_experts. */
moe_status moe_reap_keep_bias(const double* saliency, int32_t num_experts, int32_t n_keep, float* bias,
                              moe_stream_t stream);

/* Dense bf16 projection: out[t][o] = bf16(sum_i in[t][i] W[o][i]), fp32
 * accumulation (the latent down/up projections).  n_in multiple of 32. */
moe_status moe_linear_bf16(const void* in, const void* W, int64_t num_tokens, int32_t n_in,
                           int32_t n_out, void* out, moe_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_LAYER_H */
