/*
 * gqe.h -- C ABI of the MI355X (gfx950) forward (prefill) pass of the Grouped Query Experts
 * (GQE) attention layer.
 *
 * The layer (GQE README, "Algorithm Overview"; gist.science explainer, "Technical Summary"
 * -> "Architecture and Routing"): N query-head experts are split into G GQA groups of
 * n = N/G experts.  Inside each group a router takes a softmax over the group's experts and
 * keeps the top-k per token.  The k routed query heads of every group, plus one always-on
 * shared query head, attend causally to the G dense, unchanged KV heads.  The output is built
 * by the "gqe" variant (hard concatenation + renormalised weighted-sum slot + shared head) or
 * by the "weighted_concat" / "hard_concat" ablations (README "Parameters", "Ablations").
 *
 * Conventions for every entry point:
 *  - Return value: GQE_OK (0) or a negative GQE_ERR_* code.  A thread-local message is then
 *    available from gqe_last_error().  No C++ exception crosses this boundary and nothing
 *    aborts.  Every argument check is done on the host before any device call.
 *  - Device pointers are plain addresses in the memory of the current HIP device.  All
 *    tensors are dense and row-major in the "x @ W" convention; shapes are given per argument.
 *  - Ownership: the caller owns every device buffer (x, y, weights, packed weights, workspace,
 *    routing outputs) and the stream.  The library owns only the opaque host handle; it
 *    allocates no device memory and copies nothing between host and device in gqe_forward
 *    (the attention work schedule is rebuilt in the workspace by a kernel of every forward).
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = the default stream).  Work is
 *    enqueued asynchronously; only gqe_aux_stats synchronises.
 *  - A handle is not re-entrant: calls that use one handle (or one workspace) must not overlap
 *    on different streams.
 */
#ifndef GQE_H_
#define GQE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status codes */
#define GQE_OK 0
#define GQE_ERR_INVALID_CONFIG (-1) /* config violates the method's constraints          */
#define GQE_ERR_NULL_POINTER (-2)   /* a required pointer is NULL                        */
#define GQE_ERR_MISALIGNED (-3)     /* a device pointer is not 16-byte aligned           */
#define GQE_ERR_UNSUPPORTED (-4)    /* valid for the method, not implemented for gfx950 */
#define GQE_ERR_WORKSPACE (-5)      /* workspace / packed-weight buffer too small        */
#define GQE_ERR_SHAPE (-6)          /* batch or seq out of range                         */
#define GQE_ERR_HIP (-7)            /* a HIP runtime call or kernel launch failed        */
#define GQE_ERR_STATE (-8)          /* call order violated (e.g. forward before packing)  */

/* ------------------------------------------------------------------ enums */
#define GQE_VARIANT_GQE 0             /* README "Ablations": "gqe", the full method       */
#define GQE_VARIANT_WEIGHTED_CONCAT 1 /* "weighted_concat": no renormalised slot          */
#define GQE_VARIANT_HARD_CONCAT 2     /* "hard_concat": hard concat only                  */

#define GQE_DTYPE_F32 0  /* x, weights (except the router), y in float32                */
#define GQE_DTYPE_BF16 1 /* x, weights (except the router), y in bfloat16 (RNE-rounded) */

/* ------------------------------------------------------------------ configuration
 * Mirrors GQEAttention(dim, num_query_experts=16, num_kv_heads=8, top_k=1, head_dim=None,
 * variant="gqe") (README "Usage" and "Parameters").
 *  dim               d, the hidden size; required, > 0.
 *  num_query_experts N, routed query-head experts; must be divisible by num_kv_heads
 *                    (README "Parameters").  N <= 64.
 *  num_kv_heads      G, GQA groups = dense KV heads.
 *  top_k             k, experts activated per group, 1 <= k <= N/G.
 *  head_dim          d_h; 0 means dim / N (README "Parameters": defaults to dim // N).
 *  variant           GQE_VARIANT_*.
 *  shared_head       1 = one always-on shared query head (README "Algorithm Overview"),
 *                    0 = none.
 *  shared_kv_group   the KV group the shared head attends to (0 <= . < G).
 *  dtype             GQE_DTYPE_*.
 *  causal            must be 1 (prefill of a decoder: key s' attends only if s' <= s).
 *  dense_gqa         0 = GQE.  1 = the all-active GQA baseline on the same kernels: every
 *                    expert is a head (requires top_k == N/G, hard_concat, shared_head == 0);
 *                    no router runs.
 *  rope_base         0 = no positional encoding (the pages describe none).  > 0: the rotary
 *                    position embedding of RoFormer (Su et al.) on every query and key head,
 *                    interleaved pairs: (v[2i], v[2i+1]) at position m is rotated by the angle
 *                    m * rope_base^(-2i/head_dim) (10000 is the usual base); head_dim must be even.
 *                    Positions count from 0 at the first token of every sequence (gqe_forward) or
 *                    are given per sequence (gqe_decode); the cache holds rotated keys.
 */
typedef struct {
    int32_t dim;
    int32_t num_query_experts;
    int32_t num_kv_heads;
    int32_t top_k;
    int32_t head_dim;
    int32_t variant;
    int32_t shared_head;
    int32_t shared_kv_group;
    int32_t dtype;
    int32_t causal;
    int32_t dense_gqa;
    float rope_base;
} gqe_config_t;

/* ------------------------------------------------------------------ weights
 * Device pointers, row-major, "x @ W" orientation (tutorial moe_layer: x @ router_w).
 * The router is always float32; all other weights are in cfg.dtype.
 *  w_router   [d, N]       router projection (README "Algorithm Overview": per-group router)
 *  b_router   [N] or NULL  router bias
 *  w_q        [N, d, d_h]  routed query-head experts
 *  w_q_shared [d, d_h]     shared query head (required iff shared_head)
 *  w_k, w_v   [d, G*d_h]   dense KV projections; head g uses columns g*d_h .. g*d_h+d_h-1
 *  w_o        [N, d_h, d]  output projection slice of every expert slot ("hard concat")
 *  w_o_rslot  [G, d_h, d]  renormalised weighted-sum slot of every group (variant gqe only)
 *  w_o_shared [d_h, d]     output projection of the shared head (required iff shared_head)
 * The pointers are stored by gqe_init and read by gqe_pack_weights (and, for float32, by
 * gqe_forward); they must stay valid for as long as the handle uses them.
 */
typedef struct {
    const float* w_router;
    const float* b_router;
    const void* w_q;
    const void* w_q_shared;
    const void* w_k;
    const void* w_v;
    const void* w_o;
    const void* w_o_rslot;
    const void* w_o_shared;
} gqe_weights_t;

typedef struct gqe_handle gqe_handle_t;

/* Validates cfg and the weight pointers on the host (no device call) and creates a handle.
 * Errors: GQE_ERR_NULL_POINTER, GQE_ERR_INVALID_CONFIG (e.g. "num_query_experts must be
 * divisible by num_kv_heads"), GQE_ERR_UNSUPPORTED, GQE_ERR_MISALIGNED. */
int gqe_init(const gqe_config_t* cfg, const gqe_weights_t* weights, gqe_handle_t** out);

/* Bytes of the caller-owned device buffer that holds the weights in the kernels' layouts
 * (transposed head blocks, the router widened to float64, the stacked output projection). */
int gqe_packed_weights_bytes(const gqe_handle_t* h, size_t* bytes);

/* Enqueues the repacking of the weights given to gqe_init into `packed` (device, >= the size
 * above, 256-byte aligned) and records `packed` in the handle.  Call once after gqe_init and
 * again whenever the weights change.  Layout change only: no arithmetic of the layer. */
int gqe_pack_weights(gqe_handle_t* h, void* packed, size_t bytes, void* stream);

/* Bytes of scratch that gqe_forward needs for a [batch, seq] input (routing decisions,
 * per-expert statistics, Q/K/V, head outputs, the attention work schedule and the float32
 * partial results of attention items that the schedule splits along the key range).
 * batch >= 1, seq >= 1, batch * seq <= 2^28.  Host only.  Errors: GQE_ERR_NULL_POINTER,
 * GQE_ERR_SHAPE. */
int gqe_workspace_bytes(const gqe_handle_t* h, int64_t batch, int64_t seq, size_t* bytes);

/* The forward pass y = GQE(x) (README "Usage": y = attn(x)).
 *  x          [batch, seq, d] device, cfg.dtype; not aliased with y.
 *  y          [batch, seq, d] device, cfg.dtype (written).
 *  workspace  device, >= gqe_workspace_bytes(batch, seq), 256-byte aligned; also holds the
 *             routing statistics read later by gqe_aux_stats and what gqe_backward reads (routing,
 *             Q, K, V^T, O and, on the matrix-core attention path, every query row's log-sum-exp).
 *  route_idx  optional [batch, seq, G, k] int32: global expert id of the r-th choice of each
 *             group (descending router logit; ties -> lower id).  NULL to skip.
 *  route_w    optional [batch, seq, G, k] float32: renormalised weight p / sum(p_selected)
 *             of each choice.  NULL to skip.
 * Enqueues all kernels on `stream` and returns; no device allocation, no host-device copy, no
 * synchronisation (it may be captured in a HIP graph).  Requires gqe_pack_weights first (else
 * GQE_ERR_STATE).  Errors: NULL/misaligned pointers, GQE_ERR_SHAPE, GQE_ERR_WORKSPACE,
 * GQE_ERR_HIP (launch failure). */
int gqe_forward(gqe_handle_t* h, const void* x, void* y, int64_t batch, int64_t seq,
                void* workspace, size_t ws_bytes, void* stream, int32_t* route_idx,
                float* route_w);

/* The same forward pass for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The workspace is not passed in:
 * the library holds one static device array of GQE_STATIC_SCRATCH_BYTES (64 MiB) per GPU it runs
 * on, until the process ends (enough for the main setting, 8 x 2048 tokens at d = 768, N = 16,
 * G = 8, d_h = 48).  The caller still owns x, y and the routing outputs.  Allocates nothing, copies
 * nothing, enqueues on `stream` and returns.  Every call on one GPU (any handle) shares that GPU's
 * array, which keeps the last call's contents: gqe_aux_stats, gqe_bucket and gqe_kv_export of this
 * handle read it until the next call on that GPU (gqe_backward needs the workspace of a
 * gqe_forward); calls that overlap on one GPU race.
 * Errors: as gqe_forward, and GQE_ERR_WORKSPACE when the shape needs more than
 * GQE_STATIC_SCRATCH_BYTES (gqe_workspace_bytes tells), GQE_ERR_HIP when the array's device address
 * cannot be looked up. */
#define GQE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int gqe_forward_static(gqe_handle_t* h, const void* x, void* y, int64_t batch, int64_t seq, void* stream,
                       int32_t* route_idx, float* route_w);

/* Load-balancing statistics of the last gqe_forward on this handle (README "Algorithm
 * Overview": Switch-style auxiliary loss; "Usage": loss = lm_loss + 0.01 *
 * collect_aux_loss(attn)).  Synchronises `stream`, then copies to host memory:
 *  counts[N]     number of tokens that selected each expert (exact)
 *  mean_prob[N]  mean over tokens of the in-group router probability of each expert
 *  aux_loss      (1/G) sum_g n sum_{e in g} (count_e / (T k)) mean_prob_e -- unscaled; the
 *                caller applies the 0.01 coefficient
 *  active_heads  G*k + shared_head (README: 9 of 16 heads at N=16, G=8, k=1)
 * Any output pointer may be NULL.  In dense_gqa mode counts are T per expert, mean_prob 1/n.
 * Errors: GQE_ERR_STATE if no forward ran. */
int gqe_aux_stats(gqe_handle_t* h, void* stream, int64_t* counts, double* mean_prob,
                  double* aux_loss, int32_t* active_heads);

/* Byte offsets of the intermediates inside the workspace of a [batch, seq] forward, for
 * stage-by-stage checks:  offs[0] Q_act [B, H_act, S, d_h] (stored multiplied by
 * log2(e)/sqrt(d_h), the attention scale in log2 units), offs[1] K [B, G, S_pad, d_h],
 * offs[2] V^T [B, G, d_h, S_pad] (inside every 16-key chunk, bits 2 and 3 of the key offset are
 * swapped), offs[3] O_act [B, S, H_act, d_h], offs[4] route_idx [T, G, k] int32, offs[5]
 * route_w [T, G, k] f32, offs[6] p_sel [T, G, k] f32, offs[7] statistics (counts [N] int64,
 * mean probability [N] f64, aux f64), offs[8] key norms [B, G, S_pad] f32, offs[9] largest key
 * norm of every 64-key tile [B, G, S_pad / 64] f32, offs[10] the attention jobs [dims[3]][8]
 * int32 and offs[11] the merge records [.][8] int32 (the tables gqe_attention_schedule returns,
 * as the forward built them); dims[0] = H_act, dims[1] = S_pad, dims[2] = matrix-core stages
 * (1 projection, 2 attention, 4 combine), dims[3] = attention jobs.  Errors:
 * GQE_ERR_NULL_POINTER, GQE_ERR_SHAPE. */
int gqe_workspace_layout(const gqe_handle_t* h, int64_t batch, int64_t seq, size_t offs[12],
                         int64_t dims[4]);

/* Token-to-expert bucketing of the last forward's routing: the global form of the gather the
 * routed query projections do tile by tile (GQE README "Algorithm Overview": a router selects k
 * query-head experts per token in every GQA group and only those heads are computed).  The
 * T*G*k assignments (token t, group g, rank r) are sorted stably by global expert id, tokens
 * ascending inside each expert:
 *   offs [N + 1] int32: offs[e] = position of expert e's first assignment, offs[N] = T*G*k
 *   perm [T*G*k] int32: token id at each position
 *   inv  [T][G][k] int32: position of assignment (t, g, r) in perm
 * Device pointers, caller-owned, 4-byte aligned.  Enqueued on `stream` (asynchronous); reads
 * the routing and the per-block expert counts in the last forward's workspace, which must be
 * unchanged, and writes a small scratch area inside it.
 * Errors: GQE_ERR_NULL_POINTER, GQE_ERR_STATE (no forward yet, or the all-active GQA
 * configuration, which has no routing), GQE_ERR_MISALIGNED, GQE_ERR_SHAPE (T*G*k >= 2^31),
 * GQE_ERR_HIP. */
int gqe_bucket(gqe_handle_t* h, void* stream, int32_t* offs, int32_t* perm, int32_t* inv);

/* The work schedule of the matrix-core attention for a [batch, seq] forward (host only, no device
 * call; the same tables gqe_forward builds in its workspace).  The causal attention of item (batch b, group g,
 * positions p0 .. p0+np-1, the nh active heads of the group at each position: 256 / nh positions
 * per item) reads the key tiles 0 .. (last position)/64; long items are split into chunks of
 * consecutive key tiles whose float32 partial results a merge kernel combines (online-softmax
 * merge over disjoint key ranges).  Order: jobs by key-tile count, longest first; equal counts in
 * the order group, item, chunk; the batch's B sequences of one (group, item, chunk) in a row.
 *  jobs    NULL or [max_jobs][8] int32, dispatch order: b, g, nh, p0, np, kt0, kt1 (key tiles
 *          [kt0, kt1)), partial slot (-1: the job covers the whole item and writes O itself)
 *  merges  NULL or [max_merges][8] int32: b, g, nh, p0, np, first slot, chunks, 0
 *  counts  [4]: jobs, merges, partial slots, chunk cap in key tiles (0: nothing split)
 * Errors: GQE_ERR_NULL_POINTER, GQE_ERR_SHAPE, GQE_ERR_STATE (scalar attention path),
 * GQE_ERR_WORKSPACE (a buffer smaller than the count). */
int gqe_attention_schedule(const gqe_handle_t* h, int64_t batch, int64_t seq, int32_t* jobs,
                           int64_t max_jobs, int32_t* merges, int64_t max_merges, int64_t counts[4]);

/* ------------------------------------------------------------------ decode with a dense KV cache
 * GQE README "Algorithm Overview" and the gist.science explainer ("Architecture and Routing",
 * "Dense KV Path"): the KV projections and the KV cache stay dense and unchanged; only the
 * query-head computation is routed.  A decode step takes one new token per sequence; its output
 * is row p of the causal forward pass over positions 0..p of that sequence, where p is the
 * token's position and positions 0..p-1 are read from the cache.
 *
 * Cache: kcache and vcache, each [cache_batch, G, s_max, d_h] in cfg.dtype, row-major, device,
 * caller-owned, 16-byte aligned, not overlapping; head g of sequence b at position s is the d_h
 * vector at [b, g, s, :] (the keys and values the forward pass computes: x @ W_k / x @ W_v,
 * columns g*d_h ..).  Sequence b of a decode batch uses cache row b.
 *
 * Supported: d_h * element size a multiple of 16 bytes and d_h <= 128; at most 8 active query
 * heads per KV group (top_k + shared head, or N/G for dense_gqa); at most 192 output slots and
 * 8192 slot x head-dim values per token.  Otherwise GQE_ERR_UNSUPPORTED. */

/* Copies the keys and values of every token of the last gqe_forward on this handle (batch B, seq S)
 * into cache rows b0 .. b0+B-1, positions 0 .. S-1 (the prefill of the cache).  Reads the last
 * forward's workspace, which must be unchanged.  Requires S <= s_max and b0 + B <= cache_batch.
 * Enqueued on `stream`.  Errors: GQE_ERR_NULL_POINTER, GQE_ERR_STATE (no forward yet),
 * GQE_ERR_MISALIGNED, GQE_ERR_SHAPE, GQE_ERR_INVALID_CONFIG (caches overlap), GQE_ERR_HIP. */
int gqe_kv_export(gqe_handle_t* h, void* stream, void* kcache, void* vcache, int64_t cache_batch,
                  int64_t s_max, int64_t b0);

/* Bytes of scratch that gqe_decode needs for `batch` sequences with caches of s_max positions
 * (routing of the new tokens, float32 queries, per-chunk partial attention results, merged head
 * outputs).  1 <= batch <= 2^20, 1 <= s_max <= 2^28.  Host only.  Errors: GQE_ERR_NULL_POINTER,
 * GQE_ERR_SHAPE, GQE_ERR_UNSUPPORTED. */
int gqe_decode_workspace_bytes(const gqe_handle_t* h, int64_t batch, int64_t s_max, size_t* bytes);

/* One decode step.
 *  x          [batch, d] device, cfg.dtype: the new token of every sequence; not aliased with y.
 *  y          [batch, d] device, cfg.dtype (written): the layer output of those tokens.
 *  pos        [batch] device int32: position of sequence b's new token = number of its tokens
 *             already in the cache.  The token's key and value are written to the cache at
 *             [b, g, pos[b], :], then it attends to cache positions 0 .. pos[b].  A position
 *             outside [0, s_max) is not processed: no cache write, and y[b, :] is NaN.
 *  kcache, vcache  the cache, [batch, G, s_max, d_h] (see above).
 *  workspace  device, >= gqe_decode_workspace_bytes(batch, s_max), 256-byte aligned.
 *  route_idx, route_w  optional [batch, G, k] routing outputs as in gqe_forward (NULL to skip).
 * Enqueues its kernels on `stream` and returns.  Requires gqe_pack_weights first (the router
 * reads the packed weights); the other weights are read in their gqe_init layouts, so the pointers
 * given to gqe_init must stay valid.  Does not change the statistics read by gqe_aux_stats.
 * Errors: NULL/misaligned pointers, GQE_ERR_SHAPE, GQE_ERR_UNSUPPORTED, GQE_ERR_WORKSPACE,
 * GQE_ERR_STATE, GQE_ERR_INVALID_CONFIG (aliasing), GQE_ERR_HIP. */
int gqe_decode(gqe_handle_t* h, const void* x, void* y, int64_t batch, const int32_t* pos,
               void* kcache, void* vcache, int64_t s_max, void* workspace, size_t ws_bytes,
               void* stream, int32_t* route_idx, float* route_w);

/* ------------------------------------------------------------------ backward pass
 * The training half of the method (README "Usage": loss = lm_loss + 0.01 * collect_aux_loss(attn);
 * explainer "Output Construction": the renormalised weighted-sum slot gives the language-modelling
 * loss a differentiable path to the router; "Training and Loss": the load-balancing loss).
 * gqe_backward computes the gradients of  L = sum(dy * y) + aux_coef * aux  (dy = dL/dy of the
 * caller's loss, aux the balance loss of gqe_aux_stats) with respect to x and every weight, the
 * routing decisions of the forward pass held fixed (top-k is piecewise constant).
 * All gradients are float32, row-major in the layouts of gqe_weights_t; every pointer is a device
 * address, 4-byte aligned, and is overwritten (not accumulated into).  d_router and
 * d_router_bias may be NULL only for dense_gqa; d_q_shared / d_o_shared may be NULL without the
 * shared head, d_o_rslot unless variant gqe. */
typedef struct {
    float* dx;            /* [batch, seq, d] */
    float* d_router;      /* [d, N] */
    float* d_router_bias; /* [N] */
    float* d_q;           /* [N, d, d_h] */
    float* d_q_shared;    /* [d, d_h] */
    float* d_k;           /* [d, G*d_h] */
    float* d_v;           /* [d, G*d_h] */
    float* d_o;           /* [N, d_h, d] */
    float* d_o_rslot;     /* [G, d_h, d] */
    float* d_o_shared;    /* [d_h, d] */
} gqe_grads_t;

/* Bytes of scratch gqe_backward needs for a [batch, seq] forward (per-slot projections of dy,
 * head-output gradients, row statistics, router-logit gradients, dQ, dK, dV).  Host only.
 * Errors: GQE_ERR_NULL_POINTER, GQE_ERR_SHAPE, GQE_ERR_UNSUPPORTED. */
int gqe_backward_workspace_bytes(const gqe_handle_t* h, int64_t batch, int64_t seq, size_t* bytes);

/* The backward pass of the last gqe_forward on this handle.
 *  x, dy          [batch, seq, d] device, cfg.dtype; x the forward's input, dy the loss gradient.
 *  aux_coef       weight of the balance loss in L (the README's 0.01; 0 for none).
 *  fwd_workspace  the workspace of that forward (routing, statistics, Q, K, V^T, O, the row
 *                 log-sum-exp of its matrix-core attention), unchanged.
 *  workspace      device, >= gqe_backward_workspace_bytes(batch, seq), 256-byte aligned.
 * Enqueued on `stream`.  Supported: n = N/G <= 16, head_dim a multiple of 16, head_dim <= 128.
 * Errors: GQE_ERR_NULL_POINTER, GQE_ERR_STATE (no forward of this shape on this workspace),
 * GQE_ERR_MISALIGNED, GQE_ERR_WORKSPACE, GQE_ERR_UNSUPPORTED, GQE_ERR_HIP. */
int gqe_backward(gqe_handle_t* h, const void* x, const void* dy, int64_t batch, int64_t seq, double aux_coef,
                 void* fwd_workspace, void* workspace, size_t ws_bytes, const gqe_grads_t* grads, void* stream);

/* Kernel timing for measurement.  While enabled, gqe_forward and gqe_decode record a HIP event on
 * their stream right before and right after each kernel they launch; a kernel's duration is the
 * time between the two.  Kernel slots, in launch order:
 *   0 router (logits, softmax, top-k, weights, per-block statistics)   1 router statistics
 *   2 projections (routed + shared Q, K, V)                              3 key norms (only when the
 *   projections run on the scalar path and attention on matrix cores)   4 attention preparation
 *   5 attention                                                          6 attention merge
 *   7 combine + output projection
 * and of gqe_decode (slot 0 is its router):
 *   8 decode projections    9 decode attention    10 decode merge    11 decode combine
 * and of gqe_backward:
 *   12 output-side gradients (dy W_slot^T, head outputs, router logits)   13 attention
 *   14 weight gradients     15 input gradient dx
 * and 16 the attention schedule builder of gqe_forward when it runs as a kernel of its own (the
 * all-active GQA configuration; otherwise it runs inside the router launch, slot 0).
 * gqe_profile_read_kernels waits for the recorded events, returns the summed milliseconds per
 * kernel slot (0 for slots not launched) and the number of forwards they cover, and starts a new
 * accumulation.  gqe_profile_read does the same summed per stage (0 router = slots 0+1,
 * 1 projections = 2+3+8, 2 attention = 16+4+5+6+9+10, 3 combine = 7+11).  Not re-entrant; errors as
 * GQE_ERR_NULL_POINTER / GQE_ERR_HIP. */
#define GQE_PROF_KERNELS 17
int gqe_profile_enable(gqe_handle_t* h, int enable);
int gqe_profile_read(gqe_handle_t* h, double stage_ms[4], int64_t* forwards);
int gqe_profile_read_kernels(gqe_handle_t* h, double kernel_ms[GQE_PROF_KERNELS], int64_t* forwards);

/* Destroys the handle.  NULL is ignored. */
void gqe_destroy(gqe_handle_t* h);

/* Message of the last failing call on this thread ("" if none). */
const char* gqe_last_error(void);

/* ------------------------------------------------------------------ top-k MoE-MLP
 * The mixture-of-experts MLP of the cseroadmap tutorial "Grouped-query attention and mixture of
 * experts", section "Mixture of experts (MoE)" (its moe_layer sketch): a router scores all E experts
 * with softmax(x W_r + b_r), keeps the top_k of largest probability (ties -> lower expert id) and
 * mixes the chosen experts' outputs with the renormalised weights p / sum(p_selected):
 *     y[t] = sum_r w[t, r] act(x[t] W1[e_r]) W2[e_r]
 * Each expert is a two-layer MLP without biases (the page does not fix its form); act is GELU
 * (0.5 h (1 + erf(h / sqrt 2))) or ReLU.  The hidden activation is stored in bf16, the expert
 * outputs are mixed in float32 and y is rounded once to bf16.  Same conventions as above (caller-
 * owned device buffers, asynchronous on `stream`, negative GQE_ERR_* codes, gqe_last_error). */
typedef struct gqe_moe_handle gqe_moe_handle_t;

#define GQE_ACT_GELU 0
#define GQE_ACT_RELU 1

typedef struct {
    int32_t dim;         /* d: a multiple of 32 */
    int32_t num_experts; /* E: 1..16 */
    int32_t top_k;       /* 1..E */
    int32_t d_ff;        /* hidden width of every expert: a multiple of 32 */
    int32_t activation;  /* GQE_ACT_GELU or GQE_ACT_RELU */
    int32_t dtype;       /* GQE_DTYPE_BF16 (the only supported type) */
} gqe_moe_config_t;

typedef struct {
    const float* w_router; /* [d, E] float32 */
    const float* b_router; /* [E] float32, or NULL (no bias, as in the tutorial's sketch) */
    const void* w1;        /* [E, d, d_ff] bf16 */
    const void* w2;        /* [E, d_ff, d] bf16 */
} gqe_moe_weights_t;

/* Validates the config (GQE_ERR_INVALID_CONFIG: E < 1, top_k outside 1..E, d or d_ff < 1, unknown
 * activation; GQE_ERR_UNSUPPORTED: dtype other than bf16, E > 16, d or d_ff not a multiple of 32)
 * and the weight pointers (16-byte aligned, w_router 4-byte), then allocates a host handle. */
int gqe_moe_init(const gqe_moe_config_t* cfg, const gqe_moe_weights_t* w, gqe_moe_handle_t** out);

/* Bytes of the device buffer gqe_moe_pack_weights fills (router weights in float64, expert weights
 * transposed so that the reduction dimension is contiguous). */
int gqe_moe_packed_weights_bytes(const gqe_moe_handle_t* h, size_t* bytes);

/* Fills `packed` (device, 256-byte aligned, >= gqe_moe_packed_weights_bytes) from the weights
 * given to gqe_moe_init; enqueued on `stream`.  Call again after changing the weights. */
int gqe_moe_pack_weights(gqe_moe_handle_t* h, void* packed, size_t bytes, void* stream);

/* Bytes of scratch a forward of `tokens` tokens needs (routing, bucketing, the hidden activations
 * [tokens * top_k, d_ff] bf16 and the expert outputs [tokens * top_k, d] float32). */
int gqe_moe_workspace_bytes(const gqe_moe_handle_t* h, int64_t tokens, size_t* bytes);

/* y[tokens, d] (bf16, written) from x[tokens, d] (bf16); x and y device, 16-byte aligned, not
 * overlapping; workspace 256-byte aligned.  route_idx / route_w: optional [tokens, top_k] int32 /
 * float32 device outputs (expert ids best first, renormalised weights).  tokens = 0 is a no-op
 * (x and y may then be NULL);
 * tokens * top_k must stay below 2^31.  Errors: GQE_ERR_NULL_POINTER, GQE_ERR_MISALIGNED,
 * GQE_ERR_SHAPE, GQE_ERR_WORKSPACE, GQE_ERR_STATE (weights not packed), GQE_ERR_HIP. */
int gqe_moe_forward(gqe_moe_handle_t* h, const void* x, void* y, int64_t tokens, void* workspace,
                    size_t ws_bytes, void* stream, int32_t* route_idx, float* route_w);

/* Load statistics of the last forward (synchronises `stream`): tokens routed to each expert
 * (counts[E], their shares are counts / (tokens * top_k)), the mean router probability of each
 * expert (mean_prob[E]) and the balance loss E * sum_e share_e * mean_prob_e.  Any output may be
 * NULL.  Errors: GQE_ERR_NULL_POINTER, GQE_ERR_STATE (no forward), GQE_ERR_HIP. */
int gqe_moe_stats(gqe_moe_handle_t* h, void* stream, int64_t* counts, double* mean_prob, double* aux_loss);

/* Byte offsets inside the workspace of a forward of `tokens` tokens, for stage-by-stage checks:
 * offs[0] bucket offsets [E + 1] int32, offs[1] token of every bucket position [tokens * top_k]
 * int32, offs[2] position of every (token, rank) [tokens, top_k] int32, offs[3] hidden
 * activations [tokens * top_k, d_ff] bf16 in bucket order, offs[4] expert outputs
 * [tokens * top_k, d] float32 in bucket order, offs[5] routing [tokens, top_k] int32,
 * offs[6] renormalised weights [tokens, top_k] float32. */
int gqe_moe_workspace_layout(const gqe_moe_handle_t* h, int64_t tokens, size_t offs[7]);

/* Per-kernel timing as for the attention layer: slots 0 router, 1 router statistics, 2 bucketing,
 * 3 up projection (W1 and the activation), 4 down projection (W2), 5 combine. */
#define GQE_MOE_PROF_KERNELS 6
int gqe_moe_profile_enable(gqe_moe_handle_t* h, int enable);
int gqe_moe_profile_read_kernels(gqe_moe_handle_t* h, double kernel_ms[GQE_MOE_PROF_KERNELS], int64_t* forwards);

/* Destroys the handle.  NULL is ignored. */
void gqe_moe_destroy(gqe_moe_handle_t* h);

#ifdef __cplusplus
}
#endif

#endif /* GQE_H_ */
