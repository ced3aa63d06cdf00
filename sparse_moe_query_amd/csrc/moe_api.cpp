// C ABI of the top-k MoE-MLP (include/gqe.h, "top-k MoE-MLP"): validation, workspace planning,
// launch order.  The router and the bucketing are the attention layer's (one group of E experts);
// the expert products and the combine are k_moe.hip.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <new>
#include <vector>

#include "gqe_common.h"
#include "gqe_internal.h"

struct gqe_moe_handle {
    gqe_moe_config_t cfg;
    gqe_moe_weights_t w;
    MoeDims M;
    GqeDims D;  // the router's view: one group of E experts
    MoePacked pl;
    void* packed = nullptr;
    bool ran = false;
    void* last_ws = nullptr;
    MoePlan last_plan{};
    bool prof = false;
    std::vector<hipEvent_t> ev;   // 2 * KM_MOE_COUNT events per recorded forward
    std::vector<uint32_t> mask;
    size_t used = 0;
};

namespace {

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    return gqe_set_error(code, buf);
}
int ok() { return gqe_set_error(GQE_OK, ""); }
bool misaligned(const void* p, size_t a) { return ((uintptr_t)p) % a != 0; }
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

MoePacked make_packed(const MoeDims& M) {
    MoePacked pl{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    pl.wr64 = take((size_t)M.d * round_up(M.E, 16) * 8);
    pl.br64 = take((size_t)M.E * 8);
    pl.w1t = take((size_t)M.E * M.dff * M.d * 2);
    pl.w2t = take((size_t)M.E * M.d * M.dff * 2);
    pl.total = off;
    return pl;
}

MoePlan make_moe_plan(const MoeDims& M, int64_t T) {
    MoePlan P{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    const size_t tk = (size_t)T * M.k;
    P.r.B = 1;
    P.r.S = T;
    P.r.T = T;
    P.r.nblk_router = ceil_div(T, 64);
    P.r.idx = take(tk * 4);
    P.r.wsel = take(tk * 4);
    P.r.psel = take(tk * 4);
    P.r.probs = take((size_t)T * M.E * 4);
    P.r.part_cnt = take((size_t)P.r.nblk_router * M.E * 4);
    P.r.part_psum = take((size_t)P.r.nblk_router * M.E * 8);
    P.r.bucket_boff = take((size_t)P.r.nblk_router * M.E * 4);
    P.r.stats = take((size_t)M.E * 16 + 64);
    P.offs = take((size_t)(M.E + 1) * 4);
    P.perm = take(tk * 4);
    P.inv = take(tk * 4);
    P.H = take(tk * M.dff * 2);
    P.Y = take(tk * M.d * 4);
    P.total = off;
    return P;
}

bool shape_ok(const gqe_moe_handle* h, int64_t T) { return T >= 0 && T * h->M.k < ((int64_t)1 << 31); }

int marks_for(gqe_moe_handle* h, hipStream_t st, KernelMarks* km) {
    hipError_t e = hipSuccess;
    const size_t need = (h->used + 1) * (2 * KM_MOE_COUNT);
    while (h->ev.size() < need && e == hipSuccess) {
        hipEvent_t x0;
        e = hipEventCreate(&x0);
        if (e == hipSuccess) h->ev.push_back(x0);
    }
    if (e != hipSuccess) return fail(GQE_ERR_HIP, "event creation failed: %s", hipGetErrorString(e));
    if (h->mask.size() < h->used + 1) h->mask.resize(h->used + 1);
    km->ev = &h->ev[h->used * (2 * KM_MOE_COUNT)];
    km->mask = &h->mask[h->used];
    *km->mask = 0;
    km->st = st;
    ++h->used;
    return GQE_OK;
}

}  // namespace

extern "C" {

int gqe_moe_init(const gqe_moe_config_t* cfg, const gqe_moe_weights_t* w, gqe_moe_handle_t** out) {
    if (!cfg || !w || !out) return fail(GQE_ERR_NULL_POINTER, "cfg, weights and out must be non-NULL");
    *out = nullptr;
    const gqe_moe_config_t& c = *cfg;
    if (c.dim < 1 || c.d_ff < 1) return fail(GQE_ERR_INVALID_CONFIG, "dim and d_ff must be positive");
    if (c.num_experts < 1) return fail(GQE_ERR_INVALID_CONFIG, "num_experts must be positive");
    if (c.top_k < 1 || c.top_k > c.num_experts)
        return fail(GQE_ERR_INVALID_CONFIG, "top_k must be in 1..num_experts (%d)", c.num_experts);
    if (c.activation != GQE_ACT_GELU && c.activation != GQE_ACT_RELU)
        return fail(GQE_ERR_INVALID_CONFIG, "unknown activation %d", c.activation);
    if (c.dtype != GQE_DTYPE_BF16) return fail(GQE_ERR_UNSUPPORTED, "the MoE-MLP supports bf16 only");
    if (c.num_experts > 16) return fail(GQE_ERR_UNSUPPORTED, "at most 16 experts");
    if (c.dim % 32 || c.d_ff % 32) return fail(GQE_ERR_UNSUPPORTED, "dim and d_ff must be multiples of 32");
    if (!w->w_router || !w->w1 || !w->w2) return fail(GQE_ERR_NULL_POINTER, "w_router, w1 and w2 are required");
    if (misaligned(w->w_router, 4) || (w->b_router && misaligned(w->b_router, 4)) || misaligned(w->w1, 16) ||
        misaligned(w->w2, 16))
        return fail(GQE_ERR_MISALIGNED, "w1, w2 must be 16-byte aligned, the router 4-byte");
    gqe_moe_handle* h = new (std::nothrow) gqe_moe_handle();
    if (!h) return fail(GQE_ERR_HIP, "host allocation failed");
    h->cfg = c;
    h->w = *w;
    h->M = MoeDims{c.dim, c.num_experts, c.top_k, c.d_ff, c.activation, c.dtype};
    h->D = GqeDims{};
    h->D.d = c.dim;
    h->D.N = c.num_experts;
    h->D.G = 1;
    h->D.k = c.top_k;
    h->D.n = c.num_experts;
    h->D.dtype = c.dtype;
    h->pl = make_packed(h->M);
    *out = h;
    return ok();
}

int gqe_moe_packed_weights_bytes(const gqe_moe_handle_t* h, size_t* bytes) {
    if (!h || !bytes) return fail(GQE_ERR_NULL_POINTER, "handle and bytes must be non-NULL");
    *bytes = h->pl.total;
    return ok();
}

int gqe_moe_pack_weights(gqe_moe_handle_t* h, void* packed, size_t bytes, void* stream) {
    if (!h || !packed) return fail(GQE_ERR_NULL_POINTER, "handle and packed must be non-NULL");
    if (misaligned(packed, 256)) return fail(GQE_ERR_MISALIGNED, "packed must be 256-byte aligned");
    if (bytes < h->pl.total) return fail(GQE_ERR_WORKSPACE, "packed buffer too small (%zu < %zu)", bytes, h->pl.total);
    const hipStream_t st = (hipStream_t)stream;
    hipError_t e = launch_pack_router(h->D, h->w.w_router, h->w.b_router, h->pl.wr64, h->pl.br64, packed, st);
    if (e == hipSuccess) e = launch_moe_pack(h->M, h->w.w1, h->w.w2, packed, h->pl, st);
    if (e != hipSuccess) return fail(GQE_ERR_HIP, "packing failed: %s", hipGetErrorString(e));
    h->packed = packed;
    return ok();
}

int gqe_moe_workspace_bytes(const gqe_moe_handle_t* h, int64_t tokens, size_t* bytes) {
    if (!h || !bytes) return fail(GQE_ERR_NULL_POINTER, "handle and bytes must be non-NULL");
    if (!shape_ok(h, tokens)) return fail(GQE_ERR_SHAPE, "tokens out of range");
    *bytes = make_moe_plan(h->M, tokens).total;
    return ok();
}

int gqe_moe_workspace_layout(const gqe_moe_handle_t* h, int64_t tokens, size_t offs[7]) {
    if (!h || !offs) return fail(GQE_ERR_NULL_POINTER, "handle and offs must be non-NULL");
    if (!shape_ok(h, tokens)) return fail(GQE_ERR_SHAPE, "tokens out of range");
    const MoePlan P = make_moe_plan(h->M, tokens);
    offs[0] = P.offs;
    offs[1] = P.perm;
    offs[2] = P.inv;
    offs[3] = P.H;
    offs[4] = P.Y;
    offs[5] = P.r.idx;
    offs[6] = P.r.wsel;
    return ok();
}

int gqe_moe_forward(gqe_moe_handle_t* h, const void* x, void* y, int64_t tokens, void* workspace, size_t ws_bytes,
                    void* stream, int32_t* route_idx, float* route_w) {
    if (!h || !workspace) return fail(GQE_ERR_NULL_POINTER, "handle and workspace must be non-NULL");
    if (tokens > 0 && (!x || !y)) return fail(GQE_ERR_NULL_POINTER, "x and y must be non-NULL");
    if (!h->packed) return fail(GQE_ERR_STATE, "gqe_moe_pack_weights has not run");
    if (!shape_ok(h, tokens)) return fail(GQE_ERR_SHAPE, "tokens must be >= 0 with tokens * top_k < 2^31");
    if (misaligned(x, 16) || misaligned(y, 16)) return fail(GQE_ERR_MISALIGNED, "x and y must be 16-byte aligned");
    if (misaligned(workspace, 256)) return fail(GQE_ERR_MISALIGNED, "workspace must be 256-byte aligned");
    if ((route_idx && misaligned(route_idx, 4)) || (route_w && misaligned(route_w, 4)))
        return fail(GQE_ERR_MISALIGNED, "routing outputs must be 4-byte aligned");
    const MoePlan P = make_moe_plan(h->M, tokens);
    if (ws_bytes < P.total) return fail(GQE_ERR_WORKSPACE, "workspace too small (%zu < %zu)", ws_bytes, P.total);
    h->ran = true;
    h->last_ws = workspace;
    h->last_plan = P;
    if (tokens == 0) return ok();
    const hipStream_t st = (hipStream_t)stream;
    KernelMarks marks, *km = nullptr;
    if (h->prof) {
        const int rc = marks_for(h, st, &marks);
        if (rc != GQE_OK) return rc;
        km = &marks;
    }
    char* ws = (char*)workspace;
    hipError_t e = launch_router(h->D, P.r, x, h->packed, PackedLayout{h->pl.wr64, h->pl.br64}, ws, route_idx,
                                 route_w, st, km, true);
    if (e == hipSuccess) {
        if (km) km->begin(KM_MOE_BUCKET);
        e = launch_bucket(h->D, P.r, ws, (int32_t*)(ws + P.offs), (int32_t*)(ws + P.perm), (int32_t*)(ws + P.inv), st);
        if (km) km->mark(KM_MOE_BUCKET);
    }
    if (e == hipSuccess) e = launch_moe_experts(h->M, P, x, y, h->packed, h->pl, ws, st, km);
    if (e == hipSuccess && km && marks.err != hipSuccess) e = marks.err;
    if (e != hipSuccess) return fail(GQE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int gqe_moe_stats(gqe_moe_handle_t* h, void* stream, int64_t* counts, double* mean_prob, double* aux_loss) {
    if (!h) return fail(GQE_ERR_NULL_POINTER, "handle must be non-NULL");
    if (!h->ran) return fail(GQE_ERR_STATE, "no forward has run on this handle");
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return fail(GQE_ERR_HIP, "stream synchronisation failed: %s", hipGetErrorString(e));
    const int E = h->M.E;
    if (h->last_plan.r.T == 0) {
        for (int i = 0; i < E; ++i) {
            if (counts) counts[i] = 0;
            if (mean_prob) mean_prob[i] = 0.0;
        }
        if (aux_loss) *aux_loss = 0.0;
        return ok();
    }
    const char* st = (const char*)h->last_ws + h->last_plan.r.stats;
    if (counts) e = hipMemcpy(counts, st, sizeof(int64_t) * E, hipMemcpyDeviceToHost);
    if (e == hipSuccess && mean_prob) e = hipMemcpy(mean_prob, st + 8 * E, sizeof(double) * E, hipMemcpyDeviceToHost);
    if (e == hipSuccess && aux_loss) e = hipMemcpy(aux_loss, st + 16 * E, sizeof(double), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(GQE_ERR_HIP, "copy of the statistics failed: %s", hipGetErrorString(e));
    return ok();
}

int gqe_moe_profile_enable(gqe_moe_handle_t* h, int enable) {
    if (!h) return fail(GQE_ERR_NULL_POINTER, "handle must be non-NULL");
    h->prof = enable != 0;
    h->used = 0;
    return ok();
}

int gqe_moe_profile_read_kernels(gqe_moe_handle_t* h, double kernel_ms[GQE_MOE_PROF_KERNELS], int64_t* forwards) {
    if (!h || !kernel_ms) return fail(GQE_ERR_NULL_POINTER, "handle and kernel_ms must be non-NULL");
    for (int i = 0; i < KM_MOE_COUNT; ++i) kernel_ms[i] = 0.0;
    for (size_t f = 0; f < h->used; ++f) {
        hipEvent_t* ev = &h->ev[f * (2 * KM_MOE_COUNT)];
        const uint32_t mask = h->mask[f];
        for (int k = 0; k < KM_MOE_COUNT; ++k) {
            if (!((mask >> k) & 1)) continue;
            hipError_t e = hipEventSynchronize(ev[2 * k + 1]);
            float ms = 0.f;
            if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev[2 * k], ev[2 * k + 1]);
            if (e != hipSuccess) return fail(GQE_ERR_HIP, "event timing failed: %s", hipGetErrorString(e));
            kernel_ms[k] += ms;
        }
    }
    if (forwards) *forwards = (int64_t)h->used;
    h->used = 0;
    return ok();
}

void gqe_moe_destroy(gqe_moe_handle_t* h) {
    if (!h) return;
    for (hipEvent_t e : h->ev) (void)hipEventDestroy(e);
    delete h;
}

}  // extern "C"
