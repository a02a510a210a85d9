/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE-layer forward library (libmoe.so).
 *
 * The layer, as the vLLM fused-MoE config page describes it (page "MoE 的隐藏加速开关：
 * 那些按显卡命名的 config 到底是什么", section 02, the Tokens -> Router -> Grouped GEMM ->
 * weighted-sum diagram):
 *   1. route:   logits = hidden . W_r^T (+ bias); each token keeps its top-k experts
 *               (descending logit, exact ties to the lower expert id) with gate weights
 *               softmax(kept logits);
 *   2. permute: the T*k (token, slot) assignments are grouped by expert in the stable
 *               order of (expert, token, slot);
 *   3. experts: every assignment runs its expert's SwiGLU FFN,
 *               y = (silu(x Wg^T) * (x Wu^T)) Wd^T, as one grouped GEMM whose tiles each
 *               fetch their own expert's weights;
 *   4. combine: out[t] = sum_j w[t,j] * y[t,j]  (+ shared-expert output, weight 1).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked (host).  Every tensor is row-major,
 *     contiguous and 16-byte aligned; the workspace is 256-byte aligned.
 *   - Calls are asynchronous and ordered on the given stream.  None allocates, frees or
 *     synchronizes, except moe_last_device_error, which synchronizes its stream.
 *   - Arguments are validated on the host before anything is enqueued; on any error a
 *     status code is returned and nothing is enqueued.  Nothing throws across the ABI.
 *   - A call with T == 0 validates the problem, enqueues nothing and returns MOE_OK; its
 *     tensor pointers may then be NULL.
 *   - The caller owns every buffer, including the workspace.  The library keeps no
 *     per-call state outside the workspace (only a cache of device properties).
 *   - Calls that share one workspace must not run concurrently (on different streams);
 *     each call leaves the workspace's control block ready for the next call, so
 *     back-to-back calls and hipGraph replays need no reset.
 *   - Results are bitwise reproducible for a fixed build, device and input, whatever the
 *     launch grid or the order in which work items are taken.
 *
 * Layouts (E routed experts, d hidden, n expert intermediate, k top-k, T tokens):
 *   hidden   [T, d]     act dtype          out [T, d] act dtype (must not alias hidden)
 *   w_router [E, d]     act dtype          one row per expert
 *   bias     [E]        float32 or NULL    added to the logits
 *   w_gate   [E, n, d]  weight dtype       one row per intermediate channel
 *   w_up     [E, n, d]  weight dtype
 *   w_down   [E, d, n]  weight dtype       one row per output channel
 *   fp8 block scales (weight dtype MOE_FP8_E4M3, scale_block = 128), one float32 per
 *   128x128 block of each [rows, cols] matrix:  s_gate, s_up [E, n/128, d/128],
 *   s_down [E, d/128, n/128]; W[i,j] = e4m3(q[i,j]) * s[i/128, j/128]
 *   (the fp8_w8a8 + block_shape [128,128] weights named in section 03 of the same page).
 *   shared expert (n_shared = 1): sh_gate, sh_up [n, d], sh_down [d, n] and, for fp8,
 *   sh_s_gate, sh_s_up [n/128, d/128], sh_s_down [d/128, n/128]; it has weight 1 and
 *   runs on every token (GC-MoE article, "two MMA implementations": fused shared experts).
 *
 * Expert weight layout (moe_problem.w_layout).  MOE_W_ROWMAJOR: the [rows, K] matrices above
 * as they are; the compute calls do not take them (MOE_ERR_UNSUPPORTED), moe_pack_weights
 * converts them.  MOE_W_PACKED, the layout moe_forward and moe_forward_ex read: each matrix
 * is cut into fragments of 16 consecutive rows, and a
 * fragment is stored K step by K step, a step being 64 bytes of each of its 16 rows (32 bf16,
 * 64 fp8 or 16 fp32 values) laid out as one contiguous 1 KB block in which row r's bytes
 * [16 g, 16 g + 16) of the step sit at offset 16 * (16 g + r).  This is the register layout of
 * the 16-row operand of the MFMA instructions, so every weight load of the kernel reads 1 KB
 * of contiguous memory; moe_pack_weights converts row-major weights once, at load time.  The
 * packed matrices have the same size and the same per-expert offsets; scales and the router
 * are never packed.
 *
 * This layout departs from a plain [E, d, n] / [E, n, d] (K-major, input-dimension rows)
 * boundary: expert matrices are output-channel-major ([rows = output channels, K]) and the
 * compute calls take them packed.  moe_pack_weights is the one conversion, done once at load
 * time; a caller with [E, d, n] gate/up weights transposes them to [E, n, d] first.
 *
 * Supported (act dtype, weight dtype): (F32, F32), (BF16, BF16), (BF16, FP8_E4M3); act_quant
 * MOE_AQ_FP8 with FP8_E4M3 weights only (else MOE_ERR_UNSUPPORTED).
 * Shape limits: 1 <= k <= E <= 1024, d and n multiples of 256, T*k < 2^31, hidden
 * (T*d) and the expert intermediate (T*k + n_shared*T rows of n) each below 4 GB in the
 * activation dtype; with fp8 weights also d <= 32768 and n <= 16384 (else
 * MOE_ERR_UNSUPPORTED).
 *
 * Execution and co-residency.  The forward is one persistent launch of at most as many
 * workgroups as the GPU holds at once (compute units x the kernel's occupancy).  Some work
 * items are bound to workgroups and others wait, on device counters, for items taken before
 * them, so the launch assumes that all of its workgroups become resident: it should not share
 * the GPU with kernels that hold compute units for long (other streams, other processes).
 * Every device-side wait is bounded (about 2 s of the device's 100 MHz clock); a wait that
 * runs out sets the workspace's fault flag, the launch drains and exits, and
 * moe_last_device_error reports MOE_ERR_DEVICE_FAULT (the outputs are then unspecified).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

#define MOE_ABI_VERSION 4

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* null/misaligned pointer, bad shape, k > E, ...        */
  MOE_ERR_UNSUPPORTED = 2,        /* legal but not implemented: dtype combo, shape limits  */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,/* ws_bytes < moe_workspace_size()                        */
  MOE_ERR_HIP = 4,                /* a HIP runtime call (launch, device query) failed       */
  MOE_ERR_DEVICE_FAULT = 5,       /* a device-side wait timed out, or the workspace was not
                                     initialised with moe_workspace_init                   */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 /* OCP e4m3fn */ } moe_dtype;

typedef enum { MOE_W_ROWMAJOR = 0, MOE_W_PACKED = 1 } moe_weight_layout;

/* Activations of the expert GEMMs (moe_problem.act_quant).
 * MOE_AQ_NONE: the GEMMs read the activations as they are (hidden rows; H rounded to the
 *   activation dtype), and fp8 weights are decoded exactly to bf16 on the way (w8a16).
 * MOE_AQ_FP8 (fp8 weights only): the expert GEMMs of m-tiles above 16 rows (moe_plan_info
 *   m_tile_rows; decode-sized batches use 16-row m-tiles and are unaffected) run on the fp8
 *   matrix cores with fp8 activations, as the fp8_w8a8 kernel with block_shape [128,128] of
 *   the vLLM fused-MoE config page (section 03): the gate/up GEMMs read the hidden rows, and
 *   the down GEMM reads H = silu(g) * u (requantised right after SwiGLU, GC-MoE article, "two
 *   MMA implementations"), as OCP E4M3 codes with one power-of-two scale per token per 128
 *   consecutive K elements: 2^s with s the smallest integer (>= -127) such that the block's
 *   largest magnitude is at most 448 * 2^s, codes rounded to nearest, ties to even.  The
 *   weights keep their float32 128x128 block scales.  Outputs then carry the E4M3 rounding
 *   of the activations (about 4% relative error for normally distributed data). */
typedef enum { MOE_AQ_NONE = 0, MOE_AQ_FP8 = 1 } moe_act_quant;

/* (host) problem descriptor; dtype fields hold moe_dtype values. */
typedef struct {
  int64_t T;          /* tokens in this call (the M of the grouped GEMM), T >= 0         */
  int32_t d;          /* hidden size                                                      */
  int32_t n;          /* expert intermediate size                                         */
  int32_t E;          /* routed experts                                                   */
  int32_t k;          /* experts kept per token, 1 <= k <= E                              */
  int32_t n_shared;   /* 0 or 1 always-on shared expert                                   */
  int32_t act_dtype;  /* MOE_F32 or MOE_BF16: hidden, w_router, out                       */
  int32_t w_dtype;    /* MOE_F32, MOE_BF16 or MOE_FP8_E4M3: expert weights               */
  int32_t scale_block;/* 128 when w_dtype == MOE_FP8_E4M3, else 0                         */
  int32_t w_layout;   /* moe_weight_layout of w_gate, w_up, w_down and the shared expert     */
  int32_t act_quant;  /* moe_act_quant: MOE_AQ_NONE, or MOE_AQ_FP8 with fp8 weights           */
} moe_problem;

/* (host) struct of device pointers to the expert weights (layouts above). */
typedef struct {
  const void *w_gate, *w_up, *w_down;
  const float *s_gate, *s_up, *s_down;          /* fp8 only, else NULL */
  const void *sh_gate, *sh_up, *sh_down;        /* n_shared == 1 only, else NULL */
  const float *sh_s_gate, *sh_s_up, *sh_s_down; /* fp8 and n_shared == 1 only */
} moe_weights;

/* (host) struct of optional device outputs of the routing and permutation; any field may
 * be NULL.  topk_ids/topk_weights [T,k] int32/float32 (slot j = j-th largest logit),
 * logits [T,E] float32 (bias included), counts [E], offsets [E+1] (exclusive prefix sum
 * of counts, offsets[E] = T*k), perm [T*k] (perm[p] = t*k+j in (expert, token, slot)
 * order) and inv_perm [T*k] (inv_perm[t*k+j] = p), all int32. */
typedef struct {
  int32_t *topk_ids;
  float *topk_weights;
  float *logits;
  int32_t *counts, *offsets, *perm, *inv_perm;
} moe_route_out;

/* (host) optional launch controls, for tests and ablations; pass NULL for the defaults.
 * grid_wgs: workgroups of the persistent launch (0 = CUs x occupancy; larger values are
 *           reduced to CUs x occupancy, since some work items are bound to workgroups).
 * m_tile_rows, group_m: overrides of the tile table (for the tuner and ablations).
 * trace/trace_bytes: optional device buffer of 32-byte records, one per work item, indexed
 *           by item (clearing, router, then ticketed items in phase order): {start, end}
 *           of the 100 MHz device clock (uint64 each), then the item in bits 0-31 with the
 *           start and end of the item's MFMA tile loop in bits 32-47 and 48-63 (clock ticks
 *           after start; 0 = none), then (workgroup << 32 |
 *           item kind); kinds: 0 clear, 1 router,
 *           2 top-k (+ plan), 3 shared gate/up, 4 scatter, 5 gate/up, 6 down, 7 combine,
 *           8 activation quantisation (MOE_AQ_FP8; numbered after the top-k items, before the scatter items).
 *           Items beyond the buffer are not recorded.  NULL (default) records nothing.
 * schedule: 0 = dynamic (work items taken from an atomic queue in the workspace),
 *           1 = static (item i is bound to workgroup i mod grid, like static expert-to-SM
 *               binding in the Weave review, section 4.2); other values are reserved and
 *               refused (2: MOE_ERR_UNSUPPORTED, else MOE_ERR_INVALID_ARGUMENT).
 * Both schedules give bitwise identical results. */
typedef struct {
  int32_t grid_wgs;
  int32_t schedule;
  void *trace;
  int64_t trace_bytes;
  int32_t m_tile_rows;  /* 0 = the tuned M-bucket table's; else 16, 32, 64, 128 or 160.
                           The workspace must be sized for the chosen tile:
                           moe_workspace_size reports the table's (a smaller tile needs a few
                           KB more for its m-tile descriptors), else MOE_ERR_WORKSPACE_TOO_SMALL */
  int32_t group_m;      /* 0 = the table's; else 1..64 m-tiles per group of the grouped order */
  int32_t reserved[2];  /* zero */
} moe_launch_options;

/* (host) the work decomposition moe_forward chooses for a problem (moe_plan_describe). */
typedef struct {
  int32_t m_tile_rows;     /* token rows per m-tile of the grouped GEMM: 16, 32, 64, 128 or 160 */
  int32_t gateup_cols;     /* H columns per gate/up work item                                 */
  int32_t down_cols;       /* output columns per down work item                              */
  int32_t router_k_split;  /* parts the router's K is split into (partial logits added in order) */
  int32_t max_m_tiles;     /* bound on routed m-tiles for any routing (sizes the workspace)   */
  int32_t group_m;         /* m-tiles per group of the grouped item order (m-tiles > 16 rows) */
  int32_t fp8_activations; /* 1: the expert GEMMs read fp8 activations (MOE_AQ_FP8 and m-tiles
                              above 16 rows), else 0                                         */
  int32_t reserved;
} moe_plan_info;

/* The tiling moe_forward uses for p (host only, no HIP call), chosen from the per-M bucket
 * table (vLLM fused-MoE config page, section 03: one tile setting per range of the step's
 * token count; keyed here by the mean rows per routed expert, T*k/E).  Validation as for
 * moe_workspace_size. */
moe_status moe_plan_describe(const moe_problem *p, moe_plan_info *info /* (host) out */);

/* Bytes of workspace a problem needs (host only, no HIP call).  The bound depends on T*k
 * and the shapes, never on the routing.  Returns INVALID_ARGUMENT/UNSUPPORTED like the
 * compute calls. */
moe_status moe_workspace_size(const moe_problem *p, size_t *bytes /* (host) out */);

/* Clears the workspace's control block (a fill kernel on `stream`).  Call once after
 * allocating a workspace, and again after a MOE_ERR_DEVICE_FAULT.  Needs at least 196608
 * bytes. */
moe_status moe_workspace_init(void *ws, size_t ws_bytes, hipStream_t stream);

/* Step 1 alone: router logits, top-k and gate weights.  topk_ids and topk_weights are
 * required; logits and bias may be NULL.  Needs a workspace sized for p: the call runs the
 * forward's persistent kernel with only its routing phase enabled, and that kernel's queue and
 * counters live in the workspace. */
moe_status moe_route(const moe_problem *p, const void *hidden, const void *w_router,
                     const float *bias, int32_t *topk_ids, float *topk_weights, float *logits,
                     void *ws, size_t ws_bytes, hipStream_t stream);

/* Step 2 alone: histogram, exclusive scan and stable scatter of given top-k ids
 * (each row of topk_ids must hold k distinct ids in [0, E)).  All outputs required.  An id
 * out of range or repeated within a row is ignored or counted once, the outputs are then
 * unspecified, and moe_last_device_error reports MOE_ERR_DEVICE_FAULT. */
moe_status moe_permute(const moe_problem *p, const int32_t *topk_ids, int32_t *counts,
                       int32_t *offsets, int32_t *perm, int32_t *inv_perm, void *ws,
                       size_t ws_bytes, hipStream_t stream);

/* The whole layer (steps 1-4) in one persistent launch.  route_out may be NULL. */
moe_status moe_forward(const moe_problem *p, const void *hidden, const void *w_router,
                       const float *bias, const moe_weights *w, void *out,
                       const moe_route_out *route_out, void *ws, size_t ws_bytes,
                       hipStream_t stream);

/* moe_forward with launch controls (opts may be NULL). */
moe_status moe_forward_ex(const moe_problem *p, const void *hidden, const void *w_router,
                          const float *bias, const moe_weights *w, void *out,
                          const moe_route_out *route_out, void *ws, size_t ws_bytes,
                          hipStream_t stream, const moe_launch_options *opts);

/* Bytes of the fixed device scratch that moe_forward_noalloc uses as its workspace. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

/* moe_forward for callers that cannot allocate device memory: code under hipGraph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Instead of a caller's workspace it
 * uses a fixed array of MOE_NOALLOC_SCRATCH_BYTES (64 MiB) in device memory inside the
 * library; every GPU the library runs on holds its own copy until the process ends.  It calls
 * no hipMalloc or hipFree and allocates nothing else.
 *   - Arguments, layouts and results are those of moe_forward (packed weights only); results
 *     are bitwise identical to moe_forward's.
 *   - A problem whose workspace (moe_workspace_size) exceeds MOE_NOALLOC_SCRATCH_BYTES is
 *     refused with MOE_ERR_WORKSPACE_TOO_SMALL before anything is enqueued (decode-sized
 *     batches fit: e.g. T = 16 at d = 2048, n = 512, E = 256, k = 8 needs about 1 MiB).
 *   - The first call on a device looks up the array's address and enqueues, on `stream`, a
 *     fill kernel that initialises the whole array; later calls enqueue only the layer.
 *   - All calls on one GPU share its array, which keeps the last call's contents: calls that
 *     overlap on one GPU (different streams, not ordered) race and give undefined results.
 *     Calls on other streams must be ordered after the first call on the device.
 *   - A device-side wait timeout (possible only when other kernels hold the compute units
 *     this launch needs) leaves that call's outputs unspecified and is not reported here;
 *     the array's control block resets itself at the end of every call. */
moe_status moe_forward_noalloc(const moe_problem *p, const void *hidden, const void *w_router,
                               const float *bias, const moe_weights *w, void *out,
                               const moe_route_out *route_out, hipStream_t stream);

/* Converts row-major expert weights to the packed layout (see above), on `stream`: every
 * matrix of src (w_gate, w_up, w_down and, when p->n_shared, sh_gate, sh_up, sh_down) is
 * written, permuted, to the matching pointer of dst, which must not overlap it.  Scale
 * pointers are not used (scales keep their layout).  p->w_layout is ignored.  No workspace,
 * no allocation; validation as for the compute calls. */
moe_status moe_pack_weights(const moe_problem *p, const moe_weights *src, const moe_weights *dst,
                            hipStream_t stream);

/* Synchronizes `stream`, then reports MOE_ERR_DEVICE_FAULT if a device-side wait of an
 * earlier call on this workspace timed out (or the workspace was never initialised),
 * else MOE_OK.  The fault flag stays set until moe_workspace_init. */
moe_status moe_last_device_error(const void *ws, hipStream_t stream);

/* Static, never NULL. */
const char *moe_status_string(moe_status s);

/* MOE_ABI_VERSION of the built library. */
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
