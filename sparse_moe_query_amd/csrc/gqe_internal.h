// Internal declarations of libgqe: the handle, the workspace plan and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "../../include/gqe.h"
#include "gqe_common.h"

#define GQE_ATTN_COLS 256        // query columns (position, head) of one attention work item
#define GQE_ATTN_MAX_CHUNKS 32   // key-range chunks an attention item may be split into
// token chunks of the backward's router weight gradient (its partial sums share the split-K buffer)
constexpr int kRouterChunks = 128;
// split-K pieces of the backward's weight gradients (sums over the tokens)
constexpr int kWgradSplits = 16;
constexpr int kWgSplits = 8;      // token pieces of the bf16 weight-gradient products
#define GQE_DEC_MAX_HEADS 8      // decode: active query heads of one KV group
#define GQE_DEC_MAX_SLOTS 192    // decode: output-projection slots of one token
#define GQE_DEC_MAX_SLOT_DIMS 8192  // decode: slots x d_h of one token

struct GqeDims {
    int d, N, G, k, n, dh, H, s;  // s = shared head on; H = active heads per token
    int variant, dtype, skv, dense;
    float rope;                   // rotary embedding base (0: none)
};

// Byte offsets into the caller's packed-weights buffer.
struct PackedLayout {
    size_t wr64, br64;   // router weights in float64 (d x N rounded up to 16) and biases
    size_t wproj;        // bf16 path: head blocks [HB][dh][d] (K_g, V_g, shared Q, W_q[e])
    size_t wo;           // bf16 path: stacked output projection as per-(column tile, slot) stages
    size_t rope;         // rotary embedding frequencies [64] f64, cycles per position (0 when off)
    size_t total;
    int hb_total;        // number of projection head blocks
    int slots;           // output-projection slots (expert slots, renormalised slots, shared)
    int wo_pitch;        // 16-byte chunks per output column of one W_stack stage (0: not packed)
    int rslot_fused;     // variant gqe with one choice per group: each expert slot carries
                         // W_o[e] + W_oR[g] (the renormalised weight is exactly 1), no own slot
};

// One attention work group: item (batch b, group g, nh heads per position, positions
// [p0, p0 + np)) restricted to key tiles [kt0, kt1); part = partial-result slot, or -1 when the
// job covers the whole item and writes O itself.  Eight int32 per job on the device.
struct AttnJob {
    int32_t b, g, nh, p0, np, kt0, kt1, part;
};
// One merge work group: the item's nc chunks sit in slots slot0 .. slot0 + nc - 1.
struct AttnMerge {
    int32_t b, g, nh, p0, np, slot0, nc, pad;
};

// ---------------------------------------------------------------- attention work schedule
// Items of one sequence: group g carries nh = k heads per position (k + 1 in the shared head's
// group); an item is 256 / nh consecutive positions, items i = 0 .. ceil(S / (256 / nh)) - 1 in
// group order.  Item (g, i) reads key tiles [0, kt), kt = (last position) / 64 + 1; with a chunk
// cap C > 0 an item longer than C tiles is cut into nc = min(ceil(kt / C), 32) chunks, chunk c
// covering tiles [c kt / nc, (c + 1) kt / nc).  A template is one (g, i, c); templates are
// numbered group-major, then item, then chunk.  Dispatch order: templates sorted by length
// (kt1 - kt0) descending, ties by template number, and each template's B sequences in a row
// (job = B rank + b).  Split item (g, i) of sequence b owns partial slots B ss + b nc + c, where ss
// is the number of chunks of the split items before it, and merge record B mi + b, where mi is the
// number of split items before it.  The host planner (attn_sched.cpp) and the device builder
// (k_sched.hip) both follow this definition, so the table gqe_forward builds in the workspace
// equals the one gqe_attention_schedule returns.
__host__ __device__ inline int attn_item_nh(int g, int k, int s, int skv) { return k + ((s && g == skv) ? 1 : 0); }
__host__ __device__ inline int attn_items_of_group(int64_t S, int nh) {
    const int P = GQE_ATTN_COLS / nh;
    return ((int)S + P - 1) / P;  // S < 2^28: 32-bit arithmetic (no 64-bit division on the device)
}
// positions are below 2^28, so the item geometry fits int
__host__ __device__ inline int attn_item_tiles(int64_t S, int nh, int i, int* p0, int* np) {
    const int P = GQE_ATTN_COLS / nh;
    const int a = i * P;
    const int n = (int)S - a < P ? (int)S - a : P;
    *p0 = a;
    *np = n;
    return (a + n - 1) / GQE_KV_TILE + 1;
}
__host__ __device__ inline int attn_chunks_of(int kt, int C) {
    if (C <= 0 || kt <= C) return 1;
    const int nc = (kt + C - 1) / C;
    return nc < GQE_ATTN_MAX_CHUNKS ? nc : GQE_ATTN_MAX_CHUNKS;
}
// (c + 1) kt < 2^31: c < 32 chunks and kt <= 2^22 key tiles (at most 2^28 positions)
__host__ __device__ inline void attn_chunk_range(int kt, int nc, int c, int* kt0, int* kt1) {
    *kt0 = c * kt / nc;
    *kt1 = (c + 1) * kt / nc;
}

// Sizes of the schedule of a [B, S] forward (a pure function of the config, B and S).
struct AttnCounts {
    int chunk = 0;          // chunk cap C in key tiles (0: no item split)
    int items = 0;          // items of one sequence (all groups)
    int tpl = 0;            // templates of one sequence
    int maxlen = 0;         // longest template in key tiles
    int64_t njobs = 0;      // B tpl
    int64_t nmerges = 0;    // B x split items of one sequence
    int64_t nslots = 0;     // B x chunks of the split items of one sequence
};
AttnCounts attn_counts(const GqeDims& D, int64_t B, int64_t S);

struct AttnSchedule {
    std::vector<AttnJob> jobs;      // dispatch order
    std::vector<AttnMerge> merges;
    AttnCounts n;
};
AttnSchedule plan_attention(const GqeDims& D, int64_t B, int64_t S);

// Byte offsets into the caller's workspace for one [B, S] forward.
struct WorkPlan {
    int64_t B, S, T, S_pad;
    int64_t nblk_router;
    size_t idx, wsel, psel;           // [T, G, k] int32 / f32 / f32
    size_t probs;                     // [T, N] f32 in-group router probabilities (for the backward)
    size_t part_cnt, part_psum;       // [nblk_router, N] int32 / f64
    size_t bucket_boff;               // [nblk_router, N] int32 (gqe_bucket)
    size_t stats;                     // counts [N] i64, mean [N] f64, aux f64
    size_t q, kk, vt, o;              // Q_act, K, V^T, O_act
    size_t kn;                        // per-key norms [B][G][S_pad] f32
    size_t knt;                       // per-64-key-tile maximum norm [B][G][S_pad/64] f32
    size_t part_o, part_ml;           // attention partials [nslots][256][d_h] / [nslots][256][2] f32
    size_t lse;                       // [T][H] f32 row log-sum-exp (log2 units) of the attention
    bool lse_ok;                      // the last forward wrote lse (matrix-core attention)
    int64_t nslots;
    // the attention schedule, built on the device by every forward (matrix-core attention only):
    // jobs [njobs][8], merges [nmerges][8] int32, and the builder's scratch
    AttnCounts ac;
    size_t sched_jobs, sched_merges, sched_scratch;
    size_t total;
};

// Byte offsets into the caller's workspace for one decode step of B sequences with caches of
// s_max positions.
struct DecodePlan {
    WorkPlan r;                       // routing buffers of the B new tokens (idx, wsel, psel, partials)
    int64_t B, s_max, NC;             // NC = key chunks per cache row
    int C, MH;                        // keys per chunk, largest active head count of a group
    int NS;                           // output-projection slots of one token
    int NSX;                          // every output slot (N experts + group slots + shared)
    size_t qd, part, od, yp;          // queries [B][H][dh], chunk partials [B][G][NC][MH][dh+2], O [B][H][dh],
                                      // per-slot output rows [B][NS][d] (all f32)
    size_t total;
};

// Byte offsets into the caller's backward workspace for a [B, S] forward (all float32).
struct BwdPlan {
    int NS;                           // output-projection slots of one token
    int NSX;                          // every output slot (N experts + group slots + shared)
    size_t U, dO, Dd, lse, dl, cf, wn, dQ, dK, dV;
    size_t kvp;                       // bf16 attention: float32 dK / dV partials of the shared head's group
    size_t offs, perm, inv, rank;     // token lists of the routed experts (bucketing) and choice ranks
    size_t part;                      // split-K partial sums of the weight gradients
    size_t vr, dob;                   // bf16 attention: row-major V and bf16 dO
    size_t wg_gcat, wg_wcat, wg_ocat; // bf16 weight / input gradients: concatenated gradients (routed experts
                                      // zero-expanded), matching weights, slot vectors
    size_t wg_wslot;                  // bf16: the output-slot weights in one matrix
    size_t total;
};


struct gqe_handle {
    gqe_config_t cfg;
    gqe_weights_t w;
    GqeDims D;
    bool mfma;             // bf16 matrix-core path available for this config
    bool mfma_proj, mfma_attn, mfma_combine;  // per stage
    PackedLayout pl;
    void* packed;          // set by gqe_pack_weights
    // last forward (for gqe_aux_stats)
    bool ran;
    void* last_ws;
    WorkPlan last_plan;
    // kernel timing (gqe_profile_enable)
    bool prof = false;
    std::vector<hipEvent_t> prof_ev;     // 2 * KT_COUNT events per recorded forward
    std::vector<uint32_t> prof_mask;     // kernel slots recorded by each forward
    size_t prof_used = 0;                // forwards recorded
    // schedule sizes of the last shapes seen (host memory only; the tables live in the workspace)
    static constexpr int kCountCache = 8;
    struct CountEntry {
        int64_t B = 0, S = 0;
        AttnCounts c;
    };
    mutable CountEntry count_cache[kCountCache];
    mutable int count_next = 0;
};

// Kernel timing slots, in launch order (GQE_PROF_KERNELS in gqe.h).
enum {
    KT_ROUTER = 0, KT_ROUTER_STATS, KT_PROJ, KT_KEYNORM, KT_ATTN_PREP, KT_ATTN, KT_ATTN_MERGE, KT_COMBINE,
    KT_DEC_PROJ, KT_DEC_ATTN, KT_DEC_MERGE, KT_DEC_COMBINE,
    KT_BWD_OUT, KT_BWD_ATTN, KT_BWD_WGRAD, KT_BWD_DX, KT_ATTN_SCHED, KT_COUNT
};

// Records events on the stream right before and right after each kernel a launcher enqueues
// (when timing is on).
struct KernelMarks {
    hipEvent_t* ev = nullptr;  // 2 * KT_COUNT events: [2 slot] before, [2 slot + 1] after
    uint32_t* mask = nullptr;
    hipStream_t st = nullptr;
    hipError_t err = hipSuccess;
    void begin(int slot) {
        if (ev && err == hipSuccess) err = hipEventRecord(ev[2 * slot], st);
    }
    void mark(int slot) {
        if (!ev || err != hipSuccess) return;
        err = hipEventRecord(ev[2 * slot + 1], st);
        if (err == hipSuccess) *mask |= 1u << slot;
    }
};

// ---------------------------------------------------------------- top-k MoE-MLP
struct MoeDims {
    int d, E, k, dff, act, dtype;
};
struct MoePacked {
    size_t wr64, br64;  // router (as the attention router's packed form, one group)
    size_t w1t, w2t;    // expert weights transposed: [E][d_ff][d], [E][d][d_ff] bf16
    size_t total;
};
struct MoePlan {
    WorkPlan r;         // router and bucketing buffers (one group of E experts)
    size_t offs, perm, inv;  // bucketing: [E + 1], [T k], [T k] int32
    size_t H, Y;        // hidden [T k][d_ff] bf16, expert outputs [T k][d] f32, bucket order
    size_t total;
};
// MoE timing slots (the router's own launcher records slots 0 and 1)
enum { KM_MOE_ROUTER = 0, KM_MOE_STATS = 1, KM_MOE_BUCKET, KM_MOE_UP, KM_MOE_DOWN, KM_MOE_COMBINE, KM_MOE_COUNT };
hipError_t launch_moe_pack(const MoeDims& M, const void* w1, const void* w2, void* packed, const MoePacked& pl,
                           hipStream_t st);
hipError_t launch_moe_experts(const MoeDims& M, const MoePlan& P, const void* x, void* y, const void* packed,
                              const MoePacked& pl, char* ws, hipStream_t st, KernelMarks* km);
// router weights packed in float64 as the router kernels read them
hipError_t launch_pack_router(const GqeDims& D, const float* w_router, const float* b_router, size_t wr64_off,
                              size_t br64_off, void* packed, hipStream_t st);

// sets the message gqe_last_error returns on this thread; returns code (GQE_OK clears it)
int gqe_set_error(int code, const char* msg);
// gqe_forward with an optional workspace provider (called after the argument checks with the
// bytes the shape needs; returns the workspace and its size, or NULL after setting the error
// message and its code)
int gqe_forward_impl(gqe_handle_t* h, const void* x, void* y, int64_t batch, int64_t seq, void* workspace,
                     size_t ws_bytes, void* stream, int32_t* route_idx, float* route_w,
                     void* (*ws_for)(size_t need, size_t* have, int* code));

WorkPlan make_plan(const GqeDims& D, int64_t B, int64_t S, const AttnCounts& ac);
// Builds the attention schedule of P (jobs, merges) in the workspace on the stream.
hipError_t launch_attn_sched(const GqeDims& D, const WorkPlan& P, char* ws, hipStream_t st);
// Scratch bytes the device schedule builder needs.
size_t attn_sched_scratch_bytes(const AttnCounts& ac);
hipError_t launch_kn_simple(const GqeDims& D, const WorkPlan& P, char* ws, hipStream_t st, KernelMarks* km);
bool router_uses_mfma(const GqeDims& D);
PackedLayout make_packed_layout(const GqeDims& D, bool mfma);

// ---------------------------------------------------------------- launchers (return hipError_t)
hipError_t launch_pack(const GqeDims& D, const gqe_weights_t& w, const PackedLayout& pl,
                       void* packed, bool mfma, hipStream_t st);
hipError_t launch_router(const GqeDims& D, const WorkPlan& P, const void* x, const void* packed,
                         const PackedLayout& pl, char* ws, int32_t* route_idx, float* route_w,
                         hipStream_t st, KernelMarks* km, bool finalize);
// Router for a handful of tokens (one block per token; no balance statistics).
hipError_t launch_router_tokens(const GqeDims& D, int64_t T, const void* x, const void* packed,
                                const PackedLayout& pl, int32_t* idx, float* wsel, float* psel, int32_t* route_idx,
                                float* route_w, hipStream_t st, KernelMarks* km);
hipError_t launch_proj_simple(const GqeDims& D, const WorkPlan& P, const gqe_weights_t& w,
                              const void* x, const double* rope, char* ws, hipStream_t st, KernelMarks* km);
hipError_t launch_attn_simple(const GqeDims& D, const WorkPlan& P, char* ws, hipStream_t st, KernelMarks* km);
hipError_t launch_combine_simple(const GqeDims& D, const WorkPlan& P, const gqe_weights_t& w,
                                 void* y, char* ws, hipStream_t st, KernelMarks* km);
// build_sched: the launch's first work group also builds the attention schedule
hipError_t launch_proj_mfma(const GqeDims& D, const WorkPlan& P, const void* x,
                            const void* packed, const PackedLayout& pl, char* ws,
                            hipStream_t st, KernelMarks* km, bool build_sched);
hipError_t launch_attn_mfma(const GqeDims& D, const WorkPlan& P, char* ws, hipStream_t st, KernelMarks* km, bool prep);
int decode_units(const GqeDims& D);
int decode_chunk(const GqeDims& D);
hipError_t launch_kv_export(const GqeDims& D, const WorkPlan& P, const char* ws, void* kc, void* vc, int64_t s_max,
                            int64_t b0, hipStream_t st);
hipError_t launch_decode(const GqeDims& D, const DecodePlan& P, const gqe_weights_t& w, const double* rope,
                         const void* x, void* y, const int32_t* pos, void* kc, void* vc, char* ws, hipStream_t st,
                         KernelMarks* km);
hipError_t launch_backward(const GqeDims& D, const WorkPlan& P, const BwdPlan& BP, const gqe_weights_t& w,
                           const void* packed, const PackedLayout& pl, const void* x, const void* dy, double aux_coef,
                           const char* fws, char* ws, const gqe_grads_t& gr, hipStream_t st, KernelMarks* km);
hipError_t launch_bucket(const GqeDims& D, const WorkPlan& P, char* ws, int32_t* offs, int32_t* perm, int32_t* inv,
                         hipStream_t st);
bool combine_mfma_supported(const GqeDims& D);
int combine_stage_pitch(int dh);
hipError_t launch_combine_mfma(const GqeDims& D, const WorkPlan& P, const void* packed,
                               const PackedLayout& pl, void* y, char* ws, hipStream_t st, KernelMarks* km);
