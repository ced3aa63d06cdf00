// C ABI of libgqe: argument validation, workspace planning and launch order.
// Every check runs on the host before any device call; no exception leaves this file.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>

#include "gqe_common.h"
#include "gqe_internal.h"

#ifndef MFMA_PATH_ENABLED
#define MFMA_PATH_ENABLED 0
#endif


static thread_local char g_err[512] = "";

static int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}
static int ok() {
    g_err[0] = 0;
    return GQE_OK;
}
// the same thread-local message for the other entry points of the library
int gqe_set_error(int code, const char* msg) {
    snprintf(g_err, sizeof(g_err), "%s", msg);
    return code;
}
static bool misaligned(const void* p, size_t a) { return ((uintptr_t)p) % a != 0; }

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

WorkPlan make_plan(const GqeDims& D, int64_t B, int64_t S, const AttnCounts& ac) {
    WorkPlan P;
    P.B = B;
    P.S = S;
    P.T = B * S;
    P.S_pad = round_up(S, GQE_KV_TILE);
    P.nblk_router = ceil_div(P.T, 64);
    const size_t es = D.dtype == GQE_DTYPE_BF16 ? 2 : 4;
    const size_t gk = (size_t)P.T * D.G * D.k;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    P.idx = take(gk * 4);
    P.wsel = take(gk * 4);
    P.psel = take(gk * 4);
    P.probs = take((size_t)P.T * D.N * 4);
    P.part_cnt = take((size_t)P.nblk_router * D.N * 4);
    P.part_psum = take((size_t)P.nblk_router * D.N * 8);
    P.bucket_boff = take((size_t)P.nblk_router * D.N * 4);
    P.stats = take((size_t)D.N * 16 + 64);
    P.q = take((size_t)B * D.H * S * D.dh * es);
    P.kk = take((size_t)B * D.G * P.S_pad * D.dh * es);
    P.vt = take((size_t)B * D.G * D.dh * P.S_pad * es);
    P.o = take((size_t)B * S * D.H * D.dh * es);
    P.kn = take((size_t)B * D.G * P.S_pad * 4);
    P.knt = take((size_t)B * D.G * (P.S_pad / GQE_KV_TILE) * 4);
    P.ac = ac;
    P.nslots = ac.nslots;
    P.part_o = take((size_t)ac.nslots * GQE_ATTN_COLS * D.dh * 4);
    P.part_ml = take((size_t)ac.nslots * GQE_ATTN_COLS * 2 * 4);
    P.lse = take((size_t)P.T * D.H * 4);
    P.lse_ok = false;
    P.sched_jobs = take((size_t)ac.njobs * sizeof(AttnJob));
    P.sched_merges = take((size_t)ac.nmerges * sizeof(AttnMerge));
    P.sched_scratch = take(ac.njobs > 0 ? attn_sched_scratch_bytes(ac) : 0);
    P.total = off;
    return P;
}

// Decode workspace: the router's buffers for the B new tokens, then the float32 queries, chunk
// partials and merged head outputs.
static DecodePlan make_decode_plan(const GqeDims& D, int64_t B, int64_t s_max) {
    DecodePlan P{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    WorkPlan& r = P.r;
    r.B = B;
    r.S = 1;
    r.T = B;
    r.S_pad = GQE_KV_TILE;
    r.nblk_router = ceil_div(B, 64);
    const size_t gk = (size_t)B * D.G * D.k;
    r.idx = take(gk * 4);
    r.wsel = take(gk * 4);
    r.psel = take(gk * 4);
    r.part_cnt = take((size_t)r.nblk_router * D.N * 4);
    r.part_psum = take((size_t)r.nblk_router * D.N * 8);
    r.stats = take((size_t)D.N * 16 + 64);
    P.B = B;
    P.s_max = s_max;
    P.C = decode_chunk(D);
    P.NC = ceil_div(s_max, P.C);
    P.MH = (D.dense ? D.n : D.k) + D.s;
    P.qd = take((size_t)B * D.H * D.dh * 4);
    P.part = take((size_t)B * D.G * P.NC * P.MH * (D.dh + 2) * 4);
    P.od = take((size_t)B * D.H * D.dh * 4);
    P.NS = D.G * (D.dense ? D.n : D.k) + ((!D.dense && D.variant == GQE_VARIANT_GQE) ? D.G : 0) + D.s;
    P.yp = take((size_t)B * P.NS * D.d * 4);
    P.total = off;
    r.total = off;
    return P;
}

// Shapes the decode kernels handle: 16-byte cache rows, d_h <= 128, a bounded number of active
// heads per group and of output slots per token.
static int decode_supported(const GqeDims& D) {
    const int es = D.dtype == GQE_DTYPE_BF16 ? 2 : 4;
    if ((D.dh * es) % 16 != 0 || D.dh > 128)
        return fail(GQE_ERR_UNSUPPORTED, "decode needs head_dim * element size to be a multiple of 16 bytes and head_dim <= 128");
    if ((D.d * es) % 16 != 0) return fail(GQE_ERR_UNSUPPORTED, "decode needs dim * element size to be a multiple of 16 bytes");
    const int mh = (D.dense ? D.n : D.k) + D.s;
    if (mh > GQE_DEC_MAX_HEADS) return fail(GQE_ERR_UNSUPPORTED, "decode handles at most %d active heads per group", GQE_DEC_MAX_HEADS);
    const int slots = D.G * (D.dense ? D.n : D.k) + ((!D.dense && D.variant == GQE_VARIANT_GQE) ? D.G : 0) + D.s;
    if (slots > GQE_DEC_MAX_SLOTS || slots * D.dh > GQE_DEC_MAX_SLOT_DIMS)
        return fail(GQE_ERR_UNSUPPORTED, "decode handles at most %d output slots x head dims per token", GQE_DEC_MAX_SLOT_DIMS);
    return GQE_OK;
}

static bool decode_shape_ok(int64_t batch, int64_t s_max) {
    return batch >= 1 && batch <= ((int64_t)1 << 20) && s_max >= 1 && s_max <= ((int64_t)1 << 28);
}

PackedLayout make_packed_layout(const GqeDims& D, bool mfma) {
    PackedLayout L;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    L.wr64 = take((size_t)D.d * round_up(D.N, 16) * 8);
    L.br64 = take((size_t)D.N * 8);
    L.rope = take(64 * 8);
    L.hb_total = 2 * D.G + D.s + D.N;
    const bool rslot = !D.dense && D.variant == GQE_VARIANT_GQE;
    L.slots = D.dense ? D.N : D.N + (rslot ? D.G : 0) + D.s;
    L.wo_pitch = 0;
    L.rslot_fused = 0;
    L.wproj = L.wo = 0;
    if (mfma) {
        L.wproj = take((size_t)L.hb_total * D.dh * D.d * 2);
        if (combine_mfma_supported(D)) {
            if (rslot && D.k == 1) {
                L.rslot_fused = 1;
                L.slots = D.N + D.s;
            }
            L.wo_pitch = combine_stage_pitch(D.dh);
            L.wo = take((size_t)D.d * L.slots * L.wo_pitch * 16);
        }
    }
    L.total = off;
    return L;
}

// The matrix-core path covers bf16 with head dims that tile by 16 and hidden sizes that tile
// by 64; everything else the method allows runs on the scalar path.
static bool mfma_supported(const GqeDims& D) {
    if (MFMA_PATH_ENABLED == 0) return false;
    if (D.dtype != GQE_DTYPE_BF16) return false;
    if (!(D.dh == 32 || D.dh == 48 || D.dh == 64)) return false;
    if (D.d % 64 != 0) return false;
    if (D.N > 64 || D.n > 16) return false;
    if (!D.dense && 8 * D.k + D.n > 24) return false;
    if (D.H > 64) return false;
    return true;
}

// Sizes of the attention schedule for [B, S] (all zero on the scalar attention path).  The chunk
// cap comes from a host simulation of the dispatch; the last few shapes are cached in the handle
// (host memory only).
static AttnCounts attn_counts_for(const gqe_handle* h, int64_t B, int64_t S) {
    if (!h->mfma_attn) return AttnCounts{};
    for (const gqe_handle::CountEntry& c : h->count_cache)
        if (c.B == B && c.S == S) return c.c;
    const AttnCounts ac = attn_counts(h->D, B, S);
    gqe_handle::CountEntry& slot = h->count_cache[h->count_next];
    slot.B = B;
    slot.S = S;
    slot.c = ac;
    h->count_next = (h->count_next + 1) % gqe_handle::kCountCache;
    return ac;
}

// Job and slot numbers are 32-bit.
static int attn_counts_supported(const AttnCounts& ac) {
    if (ac.njobs > 0x7fffffff || ac.nslots > 0x7fffffff)
        return fail(GQE_ERR_SHAPE, "attention schedule of %lld jobs exceeds 2^31", (long long)ac.njobs);
    return GQE_OK;
}

// Events of the next recorded call while kernel timing is on (gqe_profile_enable).
static int prof_marks(gqe_handle* h, hipStream_t st, KernelMarks* marks) {
    hipError_t e = hipSuccess;
    const size_t need = (h->prof_used + 1) * (2 * KT_COUNT);
    while (h->prof_ev.size() < need && e == hipSuccess) {
        hipEvent_t x0;
        e = hipEventCreate(&x0);
        if (e == hipSuccess) h->prof_ev.push_back(x0);
    }
    if (e != hipSuccess) return fail(GQE_ERR_HIP, "event creation failed: %s", hipGetErrorString(e));
    if (h->prof_mask.size() < h->prof_used + 1) h->prof_mask.resize(h->prof_used + 1);
    marks->ev = &h->prof_ev[h->prof_used * (2 * KT_COUNT)];
    marks->mask = &h->prof_mask[h->prof_used];
    *marks->mask = 0;
    marks->st = st;
    h->prof_used += 1;
    return GQE_OK;
}

extern "C" {

const char* gqe_last_error(void) { return g_err; }

int gqe_init(const gqe_config_t* cfg, const gqe_weights_t* w, gqe_handle_t** out) {
    if (!cfg || !w || !out) return fail(GQE_ERR_NULL_POINTER, "gqe_init: cfg, weights and out must be non-NULL");
    *out = nullptr;
    const gqe_config_t& c = *cfg;
    if (c.dim <= 0) return fail(GQE_ERR_INVALID_CONFIG, "dim must be positive (got %d)", c.dim);
    if (!(c.rope_base >= 0.f) || c.rope_base > 3.0e38f)
        return fail(GQE_ERR_INVALID_CONFIG, "rope_base must be finite and >= 0 (0 = no rotary embedding)");
    if (c.num_query_experts <= 0 || c.num_kv_heads <= 0)
        return fail(GQE_ERR_INVALID_CONFIG, "num_query_experts and num_kv_heads must be positive");
    if (c.num_query_experts % c.num_kv_heads != 0)
        return fail(GQE_ERR_INVALID_CONFIG, "num_query_experts must be divisible by num_kv_heads (%d %% %d != 0)",
                    c.num_query_experts, c.num_kv_heads);
    const int n = c.num_query_experts / c.num_kv_heads;
    if (c.top_k < 1 || c.top_k > n)
        return fail(GQE_ERR_INVALID_CONFIG, "top_k must be in [1, num_query_experts/num_kv_heads = %d] (got %d)", n, c.top_k);
    if (c.head_dim < 0) return fail(GQE_ERR_INVALID_CONFIG, "head_dim must be >= 0 (0 = dim // num_query_experts)");
    const int dh = c.head_dim ? c.head_dim : c.dim / c.num_query_experts;
    if (dh <= 0) return fail(GQE_ERR_INVALID_CONFIG, "dim // num_query_experts is 0; give head_dim explicitly");
    if (c.variant < 0 || c.variant > 2) return fail(GQE_ERR_INVALID_CONFIG, "unknown variant %d", c.variant);
    if (c.dtype != GQE_DTYPE_F32 && c.dtype != GQE_DTYPE_BF16) return fail(GQE_ERR_INVALID_CONFIG, "unknown dtype %d", c.dtype);
    if (c.shared_head != 0 && c.shared_head != 1) return fail(GQE_ERR_INVALID_CONFIG, "shared_head must be 0 or 1");
    if (c.shared_head && (c.shared_kv_group < 0 || c.shared_kv_group >= c.num_kv_heads))
        return fail(GQE_ERR_INVALID_CONFIG, "shared_kv_group must be in [0, num_kv_heads)");
    if (c.dense_gqa != 0 && c.dense_gqa != 1) return fail(GQE_ERR_INVALID_CONFIG, "dense_gqa must be 0 or 1");
    if (c.dense_gqa && (c.top_k != n || c.variant != GQE_VARIANT_HARD_CONCAT || c.shared_head))
        return fail(GQE_ERR_INVALID_CONFIG, "dense_gqa requires top_k == num_query_experts/num_kv_heads, variant hard_concat and no shared head");
    if (c.causal != 1) return fail(GQE_ERR_UNSUPPORTED, "only causal prefill (causal = 1) is implemented");
    if (c.num_query_experts > 64) return fail(GQE_ERR_UNSUPPORTED, "num_query_experts > 64 is not supported");
    if (dh > 128) return fail(GQE_ERR_UNSUPPORTED, "head_dim > 128 is not supported");
    if (c.rope_base > 0.f && dh % 2 != 0) return fail(GQE_ERR_INVALID_CONFIG, "rope_base > 0 needs an even head_dim");

    if (!c.dense_gqa && !w->w_router) return fail(GQE_ERR_NULL_POINTER, "w_router is required");
    if (!w->w_q || !w->w_k || !w->w_v || !w->w_o) return fail(GQE_ERR_NULL_POINTER, "w_q, w_k, w_v and w_o are required");
    if (c.shared_head && (!w->w_q_shared || !w->w_o_shared))
        return fail(GQE_ERR_NULL_POINTER, "w_q_shared and w_o_shared are required when shared_head = 1");
    if (c.variant == GQE_VARIANT_GQE && !c.dense_gqa && !w->w_o_rslot)
        return fail(GQE_ERR_NULL_POINTER, "w_o_rslot is required for variant gqe");
    const void* ptrs[] = {w->w_router, w->b_router, w->w_q, w->w_q_shared, w->w_k, w->w_v, w->w_o, w->w_o_rslot, w->w_o_shared};
    for (const void* p : ptrs)
        if (p && misaligned(p, 16)) return fail(GQE_ERR_MISALIGNED, "weight pointers must be 16-byte aligned");

    gqe_handle* h = new (std::nothrow) gqe_handle();
    if (!h) return fail(GQE_ERR_INVALID_CONFIG, "out of host memory");
    h->cfg = c;
    h->w = *w;
    GqeDims& D = h->D;
    D.d = c.dim;
    D.N = c.num_query_experts;
    D.G = c.num_kv_heads;
    D.k = c.top_k;
    D.n = n;
    D.dh = dh;
    D.s = c.shared_head;
    D.H = D.G * D.k + D.s;
    D.variant = c.variant;
    D.dtype = c.dtype;
    D.skv = c.shared_head ? c.shared_kv_group : 0;
    D.dense = c.dense_gqa;
    D.rope = c.rope_base;
    h->mfma = mfma_supported(D);
    h->mfma_attn = D.dtype == GQE_DTYPE_BF16 && (dh == 32 || dh == 48 || dh == 64) && D.H <= 64;
    h->mfma_proj = h->mfma;
    h->mfma_combine = h->mfma && combine_mfma_supported(D);
    h->pl = make_packed_layout(D, h->mfma);
    h->packed = nullptr;
    h->ran = false;
    h->last_ws = nullptr;
    *out = h;
    return ok();
}

int gqe_packed_weights_bytes(const gqe_handle_t* h, size_t* bytes) {
    if (!h || !bytes) return fail(GQE_ERR_NULL_POINTER, "handle and bytes must be non-NULL");
    *bytes = h->pl.total;
    return ok();
}

int gqe_pack_weights(gqe_handle_t* h, void* packed, size_t bytes, void* stream) {
    if (!h || !packed) return fail(GQE_ERR_NULL_POINTER, "handle and packed must be non-NULL");
    if (misaligned(packed, 256)) return fail(GQE_ERR_MISALIGNED, "packed buffer must be 256-byte aligned");
    if (bytes < h->pl.total) return fail(GQE_ERR_WORKSPACE, "packed buffer too small: %zu < %zu", bytes, h->pl.total);
    hipError_t e = launch_pack(h->D, h->w, h->pl, packed, h->mfma, (hipStream_t)stream);
    if (e != hipSuccess) return fail(GQE_ERR_HIP, "weight packing failed: %s", hipGetErrorString(e));
    h->packed = packed;
    return ok();
}

int gqe_workspace_bytes(const gqe_handle_t* h, int64_t batch, int64_t seq, size_t* bytes) {
    if (!h || !bytes) return fail(GQE_ERR_NULL_POINTER, "handle and bytes must be non-NULL");
    if (batch < 1 || seq < 1 || batch * seq > ((int64_t)1 << 28))
        return fail(GQE_ERR_SHAPE, "batch and seq must be >= 1 with batch*seq <= 2^28");
    const AttnCounts ac = attn_counts_for(h, batch, seq);
    const int rc = attn_counts_supported(ac);
    if (rc != GQE_OK) return rc;
    *bytes = make_plan(h->D, batch, seq, ac).total;
    return ok();
}

int gqe_workspace_layout(const gqe_handle_t* h, int64_t batch, int64_t seq, size_t offs[12], int64_t dims[4]) {
    if (!h || !offs || !dims) return fail(GQE_ERR_NULL_POINTER, "handle, offs and dims must be non-NULL");
    if (batch < 1 || seq < 1 || batch * seq > ((int64_t)1 << 28)) return fail(GQE_ERR_SHAPE, "bad batch/seq");
    WorkPlan P = make_plan(h->D, batch, seq, attn_counts_for(h, batch, seq));
    offs[0] = P.q;
    offs[1] = P.kk;
    offs[2] = P.vt;
    offs[3] = P.o;
    offs[4] = P.idx;
    offs[5] = P.wsel;
    offs[6] = P.psel;
    offs[7] = P.stats;
    offs[8] = P.kn;
    offs[9] = P.knt;
    offs[10] = P.sched_jobs;
    offs[11] = P.sched_merges;
    dims[0] = h->D.H;
    dims[1] = P.S_pad;
    dims[2] = (h->mfma_proj ? 1 : 0) | (h->mfma_attn ? 2 : 0) | (h->mfma_combine ? 4 : 0);
    dims[3] = P.ac.njobs;
    return ok();
}

int gqe_forward(gqe_handle_t* h, const void* x, void* y, int64_t batch, int64_t seq, void* workspace,
                size_t ws_bytes, void* stream, int32_t* route_idx, float* route_w) {
    return gqe_forward_impl(h, x, y, batch, seq, workspace, ws_bytes, stream, route_idx, route_w, nullptr);
}

}  // extern "C"

// The forward pass on a given workspace.  When ws_for is given, it is called after every
// argument check with the workspace size the shape needs and returns the workspace to use (or
// NULL, having set the error message and code).
int gqe_forward_impl(gqe_handle_t* h, const void* x, void* y, int64_t batch, int64_t seq, void* workspace,
                     size_t ws_bytes, void* stream, int32_t* route_idx, float* route_w,
                     void* (*ws_for)(size_t need, size_t* have, int* code)) {
    if (!h || !x || !y || (!workspace && !ws_for))
        return fail(GQE_ERR_NULL_POINTER, "handle, x, y and workspace must be non-NULL");
    if (!h->packed) return fail(GQE_ERR_STATE, "gqe_pack_weights must run before gqe_forward");
    if (batch < 1 || seq < 1 || batch * seq > ((int64_t)1 << 28))
        return fail(GQE_ERR_SHAPE, "batch and seq must be >= 1 with batch*seq <= 2^28 (got %lld x %lld)",
                    (long long)batch, (long long)seq);
    if (misaligned(x, 16) || misaligned(y, 16)) return fail(GQE_ERR_MISALIGNED, "x and y must be 16-byte aligned");
    if (workspace && misaligned(workspace, 256)) return fail(GQE_ERR_MISALIGNED, "workspace must be 256-byte aligned");
    if ((route_idx && misaligned(route_idx, 4)) || (route_w && misaligned(route_w, 4)))
        return fail(GQE_ERR_MISALIGNED, "routing outputs must be 4-byte aligned");
    const GqeDims& D = h->D;
    const size_t es = D.dtype == GQE_DTYPE_BF16 ? 2 : 4;
    const size_t xbytes = (size_t)batch * seq * D.d * es;
    const char* xb = (const char*)x;
    const char* yb = (const char*)y;
    if (xb < yb + xbytes && yb < xb + xbytes) return fail(GQE_ERR_INVALID_CONFIG, "x and y must not alias");
    const AttnCounts ac = attn_counts_for(h, batch, seq);
    {
        const int rc = attn_counts_supported(ac);
        if (rc != GQE_OK) return rc;
    }
    WorkPlan P = make_plan(D, batch, seq, ac);
    if (ws_for) {
        int code = GQE_ERR_WORKSPACE;
        workspace = ws_for(P.total, &ws_bytes, &code);
        if (!workspace) return code;   // ws_for set the message
    }
    if (ws_bytes < P.total) return fail(GQE_ERR_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes, P.total);
    hipStream_t st = (hipStream_t)stream;
    char* ws = (char*)workspace;
    hipError_t e = hipSuccess;
    KernelMarks marks;
    KernelMarks* km = nullptr;
    if (h->prof) {
        const int rc = prof_marks(h, st, &marks);
        if (rc != GQE_OK) return rc;
        km = &marks;
    }
    // the attention schedule depends only on the shape and is built in the workspace: by the first
    // work group of the matrix-core projection launch, overlapping the projections, or else by a
    // kernel of its own
    if (h->mfma_attn && !h->mfma_proj) {
        if (km) km->begin(KT_ATTN_SCHED);
        e = launch_attn_sched(D, P, ws, st);
        if (km) km->mark(KT_ATTN_SCHED);
    }
    // with the matrix-core projection, its last work group finalizes the router statistics and
    // (S % 64 == 0) its key blocks write the per-tile key-norm maxima the attention reads
    if (e == hipSuccess && !D.dense)
        e = launch_router(D, P, x, h->packed, h->pl, ws, route_idx, route_w, st, km, !h->mfma_proj);
    if (e == hipSuccess)
        e = h->mfma_proj ? launch_proj_mfma(D, P, x, h->packed, h->pl, ws, st, km, h->mfma_attn)
                         : launch_proj_simple(D, P, h->w, x, (const double*)((const char*)h->packed + h->pl.rope), ws, st,
                                              km);
    if (e == hipSuccess && !h->mfma_proj && h->mfma_attn) e = launch_kn_simple(D, P, ws, st, km);
    if (e == hipSuccess)
        e = h->mfma_attn ? launch_attn_mfma(D, P, ws, st, km, !(h->mfma_proj && P.S % 64 == 0))
                         : launch_attn_simple(D, P, ws, st, km);
    if (e == hipSuccess)
        e = h->mfma_combine ? launch_combine_mfma(D, P, h->packed, h->pl, y, ws, st, km)
                            : launch_combine_simple(D, P, h->w, y, ws, st, km);
    if (e == hipSuccess && km && marks.err != hipSuccess) e = marks.err;
    if (e != hipSuccess) return fail(GQE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    h->ran = true;
    h->last_ws = workspace;
    h->last_plan = P;
    h->last_plan.lse_ok = h->mfma_attn;
    return ok();
}

extern "C" {

int gqe_aux_stats(gqe_handle_t* h, void* stream, int64_t* counts, double* mean_prob, double* aux_loss,
                  int32_t* active_heads) {
    if (!h) return fail(GQE_ERR_NULL_POINTER, "handle must be non-NULL");
    if (!h->ran) return fail(GQE_ERR_STATE, "no forward has run on this handle");
    const GqeDims& D = h->D;
    if (active_heads) *active_heads = D.H;
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return fail(GQE_ERR_HIP, "stream synchronisation failed: %s", hipGetErrorString(e));
    const WorkPlan& P = h->last_plan;
    if (D.dense) {
        // all-active GQA: every expert sees every token with in-group probability 1/n
        for (int i = 0; i < D.N; ++i) {
            if (counts) counts[i] = P.T;
            if (mean_prob) mean_prob[i] = 1.0 / D.n;
        }
        if (aux_loss) *aux_loss = 1.0;
        return ok();
    }
    const char* st = (const char*)h->last_ws + P.stats;
    if (counts) {
        e = hipMemcpy(counts, st, sizeof(int64_t) * D.N, hipMemcpyDeviceToHost);
        if (e != hipSuccess) return fail(GQE_ERR_HIP, "copy of counts failed: %s", hipGetErrorString(e));
    }
    if (mean_prob) {
        e = hipMemcpy(mean_prob, st + 8 * D.N, sizeof(double) * D.N, hipMemcpyDeviceToHost);
        if (e != hipSuccess) return fail(GQE_ERR_HIP, "copy of mean_prob failed: %s", hipGetErrorString(e));
    }
    if (aux_loss) {
        e = hipMemcpy(aux_loss, st + 16 * D.N, sizeof(double), hipMemcpyDeviceToHost);
        if (e != hipSuccess) return fail(GQE_ERR_HIP, "copy of aux_loss failed: %s", hipGetErrorString(e));
    }
    return ok();
}

int gqe_bucket(gqe_handle_t* h, void* stream, int32_t* offs, int32_t* perm, int32_t* inv) {
    if (!h || !offs || !perm || !inv) return fail(GQE_ERR_NULL_POINTER, "handle, offs, perm and inv must be non-NULL");
    if (!h->ran) return fail(GQE_ERR_STATE, "no forward has run on this handle");
    const GqeDims& D = h->D;
    if (D.dense) return fail(GQE_ERR_STATE, "the all-active GQA configuration has no routing to bucket");
    if (misaligned(offs, 4) || misaligned(perm, 4) || misaligned(inv, 4))
        return fail(GQE_ERR_MISALIGNED, "offs, perm and inv must be 4-byte aligned");
    const WorkPlan& P = h->last_plan;
    if (P.T * D.G * D.k >= ((int64_t)1 << 31)) return fail(GQE_ERR_SHAPE, "T*G*k must be below 2^31");
    const hipError_t e = launch_bucket(D, P, (char*)h->last_ws, offs, perm, inv, (hipStream_t)stream);
    if (e != hipSuccess) return fail(GQE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int gqe_attention_schedule(const gqe_handle_t* h, int64_t batch, int64_t seq, int32_t* jobs, int64_t max_jobs,
                           int32_t* merges, int64_t max_merges, int64_t counts[4]) {
    if (!h || !counts) return fail(GQE_ERR_NULL_POINTER, "handle and counts must be non-NULL");
    if (batch < 1 || seq < 1 || batch * seq > ((int64_t)1 << 28)) return fail(GQE_ERR_SHAPE, "bad batch/seq");
    if (!h->mfma_attn) return fail(GQE_ERR_STATE, "this configuration runs the scalar attention path (no schedule)");
    const AttnSchedule sc = plan_attention(h->D, batch, seq);
    counts[0] = (int64_t)sc.jobs.size();
    counts[1] = (int64_t)sc.merges.size();
    counts[2] = sc.n.nslots;
    counts[3] = sc.n.chunk;
    if (jobs) {
        if (max_jobs < counts[0]) return fail(GQE_ERR_WORKSPACE, "jobs buffer holds %lld < %lld records",
                                              (long long)max_jobs, (long long)counts[0]);
        std::memcpy(jobs, sc.jobs.data(), sc.jobs.size() * sizeof(AttnJob));
    }
    if (merges) {
        if (max_merges < counts[1]) return fail(GQE_ERR_WORKSPACE, "merges buffer holds %lld < %lld records",
                                                (long long)max_merges, (long long)counts[1]);
        std::memcpy(merges, sc.merges.data(), sc.merges.size() * sizeof(AttnMerge));
    }
    return ok();
}

int gqe_kv_export(gqe_handle_t* h, void* stream, void* kcache, void* vcache, int64_t cache_batch, int64_t s_max,
                  int64_t b0) {
    if (!h || !kcache || !vcache) return fail(GQE_ERR_NULL_POINTER, "handle, kcache and vcache must be non-NULL");
    if (!h->ran) return fail(GQE_ERR_STATE, "no forward has run on this handle");
    if (misaligned(kcache, 16) || misaligned(vcache, 16)) return fail(GQE_ERR_MISALIGNED, "caches must be 16-byte aligned");
    const WorkPlan& P = h->last_plan;
    if (!decode_shape_ok(cache_batch, s_max) || b0 < 0 || b0 + P.B > cache_batch || P.S > s_max)
        return fail(GQE_ERR_SHAPE, "the last forward [%lld x %lld] does not fit cache rows %lld.. of [%lld x %lld]",
                    (long long)P.B, (long long)P.S, (long long)b0, (long long)cache_batch, (long long)s_max);
    if (h->D.dh > 128) return fail(GQE_ERR_UNSUPPORTED, "head_dim > 128");
    const size_t cbytes = (size_t)cache_batch * h->D.G * s_max * h->D.dh * (h->D.dtype == GQE_DTYPE_BF16 ? 2 : 4);
    const char* kb = (const char*)kcache;
    const char* vb = (const char*)vcache;
    if (kb < vb + cbytes && vb < kb + cbytes) return fail(GQE_ERR_INVALID_CONFIG, "kcache and vcache must not overlap");
    const hipError_t e = launch_kv_export(h->D, P, (const char*)h->last_ws, kcache, vcache, s_max, b0, (hipStream_t)stream);
    if (e != hipSuccess) return fail(GQE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int gqe_decode_workspace_bytes(const gqe_handle_t* h, int64_t batch, int64_t s_max, size_t* bytes) {
    if (!h || !bytes) return fail(GQE_ERR_NULL_POINTER, "handle and bytes must be non-NULL");
    if (!decode_shape_ok(batch, s_max)) return fail(GQE_ERR_SHAPE, "batch must be in [1, 2^20] and s_max in [1, 2^28]");
    const int rc = decode_supported(h->D);
    if (rc != GQE_OK) return rc;
    *bytes = make_decode_plan(h->D, batch, s_max).total;
    return ok();
}

int gqe_decode(gqe_handle_t* h, const void* x, void* y, int64_t batch, const int32_t* pos, void* kcache,
               void* vcache, int64_t s_max, void* workspace, size_t ws_bytes, void* stream, int32_t* route_idx,
               float* route_w) {
    if (!h || !x || !y || !pos || !kcache || !vcache || !workspace)
        return fail(GQE_ERR_NULL_POINTER, "handle, x, y, pos, kcache, vcache and workspace must be non-NULL");
    if (!h->packed) return fail(GQE_ERR_STATE, "gqe_pack_weights must run before gqe_decode");
    if (!decode_shape_ok(batch, s_max)) return fail(GQE_ERR_SHAPE, "batch must be in [1, 2^20] and s_max in [1, 2^28]");
    const int rc = decode_supported(h->D);
    if (rc != GQE_OK) return rc;
    if (misaligned(x, 16) || misaligned(y, 16) || misaligned(kcache, 16) || misaligned(vcache, 16))
        return fail(GQE_ERR_MISALIGNED, "x, y, kcache and vcache must be 16-byte aligned");
    if (misaligned(pos, 4)) return fail(GQE_ERR_MISALIGNED, "pos must be 4-byte aligned");
    if (misaligned(workspace, 256)) return fail(GQE_ERR_MISALIGNED, "workspace must be 256-byte aligned");
    if ((route_idx && misaligned(route_idx, 4)) || (route_w && misaligned(route_w, 4)))
        return fail(GQE_ERR_MISALIGNED, "routing outputs must be 4-byte aligned");
    const GqeDims& D = h->D;
    const size_t es = D.dtype == GQE_DTYPE_BF16 ? 2 : 4;
    const size_t xbytes = (size_t)batch * D.d * es;
    const char* xb = (const char*)x;
    const char* yb = (const char*)y;
    if (xb < yb + xbytes && yb < xb + xbytes) return fail(GQE_ERR_INVALID_CONFIG, "x and y must not alias");
    const size_t cbytes = (size_t)batch * D.G * s_max * D.dh * es;
    const char* kb = (const char*)kcache;
    const char* vb = (const char*)vcache;
    if (kb < vb + cbytes && vb < kb + cbytes) return fail(GQE_ERR_INVALID_CONFIG, "kcache and vcache must not overlap");
    const DecodePlan P = make_decode_plan(D, batch, s_max);
    if (ws_bytes < P.total) return fail(GQE_ERR_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes, P.total);
    hipStream_t st = (hipStream_t)stream;
    char* ws = (char*)workspace;
    KernelMarks marks;
    KernelMarks* km = nullptr;
    hipError_t e = hipSuccess;
    if (h->prof) {
        const int rc = prof_marks(h, st, &marks);
        if (rc != GQE_OK) return rc;
        km = &marks;
    }
    if (!D.dense)
        e = launch_router_tokens(D, batch, x, h->packed, h->pl, (int32_t*)(ws + P.r.idx), (float*)(ws + P.r.wsel),
                                 (float*)(ws + P.r.psel), route_idx, route_w, st, km);
    if (e == hipSuccess)
        e = launch_decode(D, P, h->w, (const double*)((const char*)h->packed + h->pl.rope), x, y, pos, kcache, vcache,
                          ws, st, km);
    if (e == hipSuccess && km && marks.err != hipSuccess) e = marks.err;
    if (e != hipSuccess) return fail(GQE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

static int backward_supported(const GqeDims& D) {
    if (D.n > 16) return fail(GQE_ERR_UNSUPPORTED, "backward handles at most 16 experts per group");
    if (D.dh % 16 != 0 || D.dh > 128) return fail(GQE_ERR_UNSUPPORTED, "backward needs head_dim a multiple of 16, <= 128");
    return GQE_OK;
}

static BwdPlan make_bwd_plan(const GqeDims& D, int64_t B, int64_t S) {
    BwdPlan P{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    const size_t T = (size_t)(B * S);
    P.NS = D.G * D.k + ((!D.dense && D.variant == GQE_VARIANT_GQE) ? D.G : 0) + D.s;
    P.NSX = D.N + ((!D.dense && D.variant == GQE_VARIANT_GQE) ? D.G : 0) + D.s;
    P.U = take(T * std::max(P.NS, P.NSX) * D.dh * 4);
    P.dO = take(T * D.H * D.dh * 4);
    P.Dd = take(T * D.H * 4);
    P.lse = take(T * D.H * 4);
    P.dl = take(T * D.N * 4);
    P.cf = take(T * D.H * 4);
    P.wn = take(T * D.H * 4);
    P.dQ = take(T * D.H * D.dh * 4);
    P.dK = take(T * D.G * D.dh * 4);
    P.dV = take(T * D.G * D.dh * 4);
    P.kvp = take(4 * T * D.dh * 4);
    P.offs = take((size_t)(D.N + 1) * 4);
    P.perm = take(T * D.G * D.k * 4);
    P.inv = take(T * D.G * D.k * 4);
    P.rank = take(T * D.G * D.k * 4);
    {
        // split-K partials: kWgradSplits pieces of every weight-gradient sub-problem, each at most (d + 1) x max(d_h, N)
        // (input side, 2G + s + N + 1 sub-problems) or d_h x d (output side, N + G + 1)
        const size_t in_side = (size_t)(2 * D.G + D.s + D.N) * D.d * D.dh;
        const size_t out_side = (size_t)(D.N + D.G + D.s) * D.dh * D.d;
        const size_t router_side = (size_t)kRouterChunks * (D.d + 1) * D.N;
        P.part = take(std::max((size_t)kWgradSplits * std::max(in_side, out_side), router_side) * 4);
    }
    const size_t S_pad = (size_t)round_up(S, GQE_KV_TILE);
    P.vr = take((size_t)B * D.G * S_pad * D.dh * 2);
    P.dob = take((size_t)B * D.H * S_pad * D.dh * 2);
    if (D.dtype == GQE_DTYPE_BF16) {
        const size_t kp = (size_t)round_up((int64_t)(2 * D.G + D.s + D.N) * D.dh, 64);
        P.wg_gcat = take(T * kp * 2);
        P.wg_wcat = take((size_t)D.d * kp * 2);
        P.wg_wslot = take((size_t)P.NSX * D.dh * D.d * 2);
        P.wg_ocat = take(T * (D.N + D.G + D.s) * D.dh * 2);
    }
    P.total = off;
    return P;
}

int gqe_backward_workspace_bytes(const gqe_handle_t* h, int64_t batch, int64_t seq, size_t* bytes) {
    if (!h || !bytes) return fail(GQE_ERR_NULL_POINTER, "handle and bytes must be non-NULL");
    if (batch < 1 || seq < 1 || batch * seq > ((int64_t)1 << 28)) return fail(GQE_ERR_SHAPE, "bad batch/seq");
    const int rc = backward_supported(h->D);
    if (rc != GQE_OK) return rc;
    *bytes = make_bwd_plan(h->D, batch, seq).total;
    return ok();
}

int gqe_backward(gqe_handle_t* h, const void* x, const void* dy, int64_t batch, int64_t seq, double aux_coef,
                 void* fwd_workspace, void* workspace, size_t ws_bytes, const gqe_grads_t* grads, void* stream) {
    if (!h || !x || !dy || !fwd_workspace || !workspace || !grads)
        return fail(GQE_ERR_NULL_POINTER, "handle, x, dy, workspaces and grads must be non-NULL");
    const GqeDims& D = h->D;
    const gqe_grads_t& g = *grads;
    if (!g.dx || !g.d_q || !g.d_k || !g.d_v || !g.d_o || (!D.dense && (!g.d_router || !g.d_router_bias)) ||
        (D.s && (!g.d_q_shared || !g.d_o_shared)) || (!D.dense && D.variant == GQE_VARIANT_GQE && !g.d_o_rslot))
        return fail(GQE_ERR_NULL_POINTER, "a required gradient pointer is NULL");
    const float* gp[] = {g.dx, g.d_router, g.d_router_bias, g.d_q, g.d_q_shared, g.d_k, g.d_v, g.d_o, g.d_o_rslot, g.d_o_shared};
    for (const float* p : gp)
        if (p && misaligned(p, 4)) return fail(GQE_ERR_MISALIGNED, "gradient pointers must be 4-byte aligned");
    if (misaligned(x, 16) || misaligned(dy, 16)) return fail(GQE_ERR_MISALIGNED, "x and dy must be 16-byte aligned");
    if (misaligned(workspace, 256)) return fail(GQE_ERR_MISALIGNED, "workspace must be 256-byte aligned");
    const int rc = backward_supported(D);
    if (rc != GQE_OK) return rc;
    if (!h->ran || h->last_ws != fwd_workspace || h->last_plan.B != batch || h->last_plan.S != seq)
        return fail(GQE_ERR_STATE, "gqe_backward needs the last gqe_forward of this [batch, seq] and its workspace");
    if (!(aux_coef == aux_coef)) return fail(GQE_ERR_INVALID_CONFIG, "aux_coef is NaN");
    const BwdPlan BP = make_bwd_plan(D, batch, seq);
    if (ws_bytes < BP.total) return fail(GQE_ERR_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes, BP.total);
    hipStream_t st = (hipStream_t)stream;
    KernelMarks marks;
    KernelMarks* km = nullptr;
    if (h->prof) {
        const int prc = prof_marks(h, st, &marks);
        if (prc != GQE_OK) return prc;
        km = &marks;
    }
    hipError_t e = launch_backward(D, h->last_plan, BP, h->w, h->packed, h->pl, x, dy, aux_coef,
                                   (const char*)fwd_workspace, (char*)workspace, g, st, km);
    if (e == hipSuccess && km && marks.err != hipSuccess) e = marks.err;
    if (e != hipSuccess) return fail(GQE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int gqe_profile_enable(gqe_handle_t* h, int enable) {
    if (!h) return fail(GQE_ERR_NULL_POINTER, "handle must be non-NULL");
    h->prof = enable != 0;
    h->prof_used = 0;
    return ok();
}

int gqe_profile_read_kernels(gqe_handle_t* h, double kernel_ms[GQE_PROF_KERNELS], int64_t* forwards) {
    if (!h || !kernel_ms) return fail(GQE_ERR_NULL_POINTER, "handle and kernel_ms must be non-NULL");
    for (int i = 0; i < KT_COUNT; ++i) kernel_ms[i] = 0.0;
    for (size_t f = 0; f < h->prof_used; ++f) {
        hipEvent_t* ev = &h->prof_ev[f * (2 * KT_COUNT)];
        const uint32_t mask = h->prof_mask[f];
        for (int k = 0; k < KT_COUNT; ++k) {
            if (!((mask >> k) & 1)) continue;
            hipError_t e = hipEventSynchronize(ev[2 * k + 1]);
            if (e != hipSuccess) return fail(GQE_ERR_HIP, "event wait failed: %s", hipGetErrorString(e));
            float ms = 0.f;
            e = hipEventElapsedTime(&ms, ev[2 * k], ev[2 * k + 1]);
            if (e != hipSuccess) return fail(GQE_ERR_HIP, "event timing failed: %s", hipGetErrorString(e));
            kernel_ms[k] += ms;
        }
    }
    if (forwards) *forwards = (int64_t)h->prof_used;
    h->prof_used = 0;
    return ok();
}

int gqe_profile_read(gqe_handle_t* h, double stage_ms[4], int64_t* forwards) {
    if (!h || !stage_ms) return fail(GQE_ERR_NULL_POINTER, "handle and stage_ms must be non-NULL");
    double k[KT_COUNT];
    const int rc = gqe_profile_read_kernels(h, k, forwards);
    if (rc != GQE_OK) return rc;
    stage_ms[0] = k[KT_ROUTER] + k[KT_ROUTER_STATS];
    stage_ms[1] = k[KT_PROJ] + k[KT_KEYNORM] + k[KT_DEC_PROJ];
    stage_ms[2] = k[KT_ATTN_SCHED] + k[KT_ATTN_PREP] + k[KT_ATTN] + k[KT_ATTN_MERGE] + k[KT_DEC_ATTN] + k[KT_DEC_MERGE];
    stage_ms[3] = k[KT_COMBINE] + k[KT_DEC_COMBINE];
    return ok();
}

void gqe_destroy(gqe_handle_t* h) {
    if (!h) return;
    for (hipEvent_t e : h->prof_ev) (void)hipEventDestroy(e);
    delete h;
}

}  // extern "C"
