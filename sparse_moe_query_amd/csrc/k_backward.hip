// Backward pass of the GQE layer (gfx950): gradients of L = sum(dy * y) + aux_coef * aux with
// respect to x and every weight, the routing decisions of the forward pass held fixed.
//
// GQE README "Usage" trains with lm_loss + 0.01 * collect_aux_loss(attn); the explainer's "Output
// Construction" notes that the renormalised weighted-sum slot is the language-modelling loss's
// differentiable path to the router (top-k itself is piecewise constant), and its "Training and
// Loss" adds the load-balancing loss.  The steps are the chain rule through the forward definition,
// in reverse order:
//
//   ProbU             U[t][slot] = dy_t W_slot^T for every output slot of the token (routed expert
//                     e: W_o[e], over its tokens; group g: W_oR[g]; shared head: W_os)
//   bwd_route_kernel  per (token, group): head-output gradients do = c U_e + w U_g, D = do . o for
//                     the attention; from the forward's stored router probabilities the
//                     probability gradients (weighted_concat coefficient, renormalisation
//                     w = p / sum_sel p, aux loss) and the logit gradients through the in-group
//                     softmax
//   bwd_dq_kernel     per 64 queries of a head: the row log-sum-exp (log2 units, from the stored
//                     queries and keys), then dq = sum_j p_j (do . v_j - D) k_j / sqrt(d_h),
//                     rotated back (rotary embedding)
//   bwd_dkv_kernel    per 64 keys of a group: dk_j, dv_j over every later query of every head
//   ProbWo, ProbWx    weight gradients as sums over the tokens that use each weight block
//   bwd_router_wgrad  router weight and bias gradients (float32)
//   ProbDx*           dx = dense part (dk W_k^T, dv W_v^T, shared dq W_qs^T, router logits W_r^T),
//                     then the routed dq W_q[e]^T per (group, rank)
//
// The GEMM-shaped steps run through one tiled kernel over gathered token lists (the global
// bucketing of the forward's routing): on matrix cores for bf16 layers (tgemm_mfma_kernel), in
// float32 FMAs otherwise (tgemm_kernel).  The attention steps of bf16 layers run on matrix cores
// (bwd_*_mfma_kernel), those of float32 layers stage 64-row tiles in LDS, four lanes per row.
// Everything reads the forward pass's workspace (routing, router probabilities, statistics, Q, K,
// V^T, O), which must be unchanged.
#include <math.h>

#include <algorithm>
#include <cmath>

#include "gqe_common.h"
#include "gqe_internal.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;

struct BwdArgs {
    const void* x;          // [T][d]
    const void* dy;         // [T][d]
    // forward workspace
    const int32_t* idx;     // [T][G][k]
    const int64_t* counts;  // [N]
    const void* Q;          // [B][H][S][dh], times log2(e)/sqrt(dh), rotated
    const void* K;          // [B][G][S_pad][dh], rotated
    const void* Vt;         // [B][G][dh][S_pad], keys slotted
    const void* O;          // [B][S][H][dh]
    // weights (gqe_init layouts) and the packed rotary table
    const void *wq, *wqs, *wk, *wv, *wo, *wor, *wos;
    const float* wr;        // [d][N]
    const float* probs;     // [T][N] the forward's in-group router probabilities
    const double* rope;     // rotary frequencies (cycles per position) or null
    // backward workspace
    float* U;               // [T][NS][dh] (slot order: see wgp)
    float* dO;              // [T][H][dh]
    float* Dd;              // [T][H]
    float* lse;             // [T][H]: row log-sum-exp (log2 units); the forward's when lse_fwd
    int lse_fwd;            // bf16 matrix-core attention: lse was written by the forward
    float* dl;              // [T][N]
    float* cf;              // [T][H]: output coefficient of each routed head (p for weighted_concat, else 1)
    float* wn;              // [T][H]: renormalised weight of each routed head (variant gqe)
    // query / key / value gradients, float32 for float32 layers and bf16 for bf16 layers (the
    // matrix-core products that read them round to bf16 anyway)
    void* dQ;               // [T][H][dh] (before the rotation)
    void* dK;               // [T][G][dh] (before the rotation)
    void* dV;               // [T][G][dh]
    float* part;            // split-K partial sums of the weight gradients
    uint16_t* vr;           // bf16 path: V row-major [B][G][S_pad][dh]
    uint16_t* dob;          // bf16 path: dO in bf16 [B][H][S_pad][dh]
    float* kvp;             // bf16 path: [4][T][dh] float32 dK / dV of the shared head's group, split
                            // into its routed heads' part and the shared head's part
    uint16_t* wg_gcat;      // bf16 path: concatenated gradients, routed experts zero-expanded [T][kp]
    uint16_t* wg_wcat;      // bf16 path: the matching input-side weights [d][kp]
    uint16_t* wg_wslot;     // bf16 path: the output-slot weights [NS dh][d]
    uint16_t* wg_ocat;      // bf16 path: zero-expanded output-slot vectors [T][N + G + s][dh]
    // outputs (float32)
    float *dx, *dwr, *dbr, *dwq, *dwqs, *dwk, *dwv, *dwo, *dwor, *dwos;
    double aux_coef;
    int64_t B, S, T, S_pad;
    int d, N, G, k, n, dh, H, s, skv, variant, dense, NS, Np;
    // bf16 whole-product path (see run): U holds every expert's slot ([N experts | G group slots |
    // shared], NS = N + G + s) instead of the token's chosen ones ([G k ranks | G | s])
    int wgp;
};

template <typename T>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
    return to_f32(reinterpret_cast<const T*>(p)[i]);
}

// four consecutive elements (16-byte aligned for float32, 8-byte for bf16) as float32
template <typename T>
__device__ __forceinline__ f32x4_t ld4(const void* p, int64_t i);
template <>
__device__ __forceinline__ f32x4_t ld4<float>(const void* p, int64_t i) {
    return *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(p) + i);
}
template <>
__device__ __forceinline__ f32x4_t ld4<bf16_t>(const void* p, int64_t i) {
    const u32x2_t q = *reinterpret_cast<const u32x2_t*>(reinterpret_cast<const bf16_t*>(p) + i);
    return f32x4_t{__uint_as_float(q[0] << 16), __uint_as_float(q[0] & 0xffff0000u), __uint_as_float(q[1] << 16),
                   __uint_as_float(q[1] & 0xffff0000u)};
}
// eight consecutive elements (16-byte aligned for bf16, 32-byte for float32) as float32
template <typename T>
__device__ __forceinline__ void ld8(const void* p, int64_t i, float (&v)[8]) {
    const f32x4_t a = ld4<T>(p, i), b = ld4<T>(p, i + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[e] = a[e];
        v[4 + e] = b[e];
    }
}
__device__ __forceinline__ void ld8f(const float* p, float (&v)[8]) { ld8<float>(p, 0, v); }
__device__ __forceinline__ u32x4_t pack8(const float (&v)[8]) {
    return u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
}
// the storage type of dQ, dK, dV for layers of type T
template <typename T>
struct GradT {
    typedef float type;
};
template <>
struct GradT<bf16_t> {
    typedef bf16_t type;
};
template <typename T>
__device__ __forceinline__ float gread(const void* p, int64_t i) {
    return ld<typename GradT<T>::type>(p, i);
}
template <typename T>
__device__ __forceinline__ void gread8(const void* p, int64_t i, float (&v)[8]) {
    ld8<typename GradT<T>::type>(p, i, v);
}
template <typename T>
__device__ __forceinline__ void gwrite(void* p, int64_t i, float v) {
    typedef typename GradT<T>::type G;
    reinterpret_cast<G*>(p)[i] = from_f32<G>(v);
}
__device__ __forceinline__ float dot4(const f32x4_t& u, const f32x4_t& v) {
    return u[0] * v[0] + u[1] * v[1] + u[2] * v[2] + u[3] * v[3];
}

__device__ __forceinline__ int group_of(const BwdArgs& a, int h) { return h < a.G * a.k ? h / a.k : a.skv; }

// ---------------------------------------------------------------- head-output and router gradients
// Sum over the four lanes of a quad (DPP row permutations xor 1, xor 2).
__device__ __forceinline__ float quad_add(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, false));
    return v;
}

// Four lanes per (token, group), each a quarter of the head dims (four elements in every 16; the
// dot products summed over the quad); group 0 also handles the shared head.  Every lane of a quad
// forms the router gradients (n <= 16 values), its first lane stores them.
template <typename T>
__global__ void bwd_route_kernel(BwdArgs a) {
    const int64_t q = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 2;
    const int qd = threadIdx.x & 3;
    const bool lead = qd == 0;
    if (q >= a.T * a.G) return;  // whole quads leave together (T G quads, blocks of 64 quads)
    const int64_t t = q / a.G;
    const int g = (int)(q % a.G);
    const int n = a.n, k = a.k, dh = a.dh, H = a.H, nr = a.G * a.k;
    const int64_t b = t / a.S, s = t % a.S;
    const bool rslot = !a.dense && a.variant == GQE_VARIANT_GQE;
    // rows of d_h (a multiple of 16) read and written four elements at a time
    const float* Ut = a.U + t * a.NS * dh;
    auto U4 = [&](int slot, int j) { return *reinterpret_cast<const f32x4_t*>(Ut + slot * dh + j); };
    // U slots: the routed heads' (by choice rank, or by expert on the whole-product path), then the
    // renormalised group slots, then the shared head
    const int ub = a.wgp ? a.N : nr;
    auto O4 = [&](int h, int j) { return ld4<T>(a.O, ((b * a.S + s) * H + h) * dh + j); };
    auto dO4 = [&](int h, int j) -> f32x4_t& { return *reinterpret_cast<f32x4_t*>(a.dO + (t * H + h) * dh + j); };
    if (g == 0 && a.s) {  // shared head: do = dy W_os^T
        const int hs = nr, ls = ub + (rslot ? a.G : 0);
        float D = 0.f;
        for (int j = 4 * qd; j < dh; j += 16) {
            const f32x4_t v = U4(ls, j);
            dO4(hs, j) = v;
            D += dot4(v, O4(hs, j));
        }
        D = quad_add(D);
        if (lead) a.Dd[t * H + hs] = D;
    }
    if (a.dense) {  // all-active GQA: hard concatenation, no router
        for (int r = 0; r < k; ++r) {
            const int h = g * k + r;
            float D = 0.f;
            for (int j = 4 * qd; j < dh; j += 16) {
                const f32x4_t v = U4(a.wgp ? g * n + r : h, j);
                dO4(h, j) = v;
                D += dot4(v, O4(h, j));
            }
            D = quad_add(D);
            if (lead) {
                a.Dd[t * H + h] = D;
                a.cf[t * H + h] = 1.f;
                a.wn[t * H + h] = 0.f;
            }
        }
        return;
    }
    // the group's router probabilities, as the forward pass formed them
    float p[16], dp[16];
    for (int jj = 0; jj < n; ++jj) {
        p[jj] = a.probs[t * a.N + g * n + jj];
        dp[jj] = 0.f;
    }
    const int32_t* id = a.idx + (t * a.G + g) * k;
    float psel = 0.f;
    for (int r = 0; r < k; ++r) psel += p[id[r] - g * n];
    float dw[16];
    for (int r = 0; r < k; ++r) {
        const int h = g * k + r, jr = id[r] - g * n;
        const float coef = a.variant == GQE_VARIANT_WEIGHTED_CONCAT ? p[jr] : 1.f;
        const float w = p[jr] / psel;
        float D = 0.f, ou = 0.f, ov = 0.f;
        for (int j = 4 * qd; j < dh; j += 16) {
            const f32x4_t u = U4(a.wgp ? id[r] : h, j);
            const f32x4_t v = rslot ? U4(ub + g, j) : f32x4_t{0.f, 0.f, 0.f, 0.f};
            const f32x4_t o = O4(h, j);
            const f32x4_t dov = coef * u + w * v;
            dO4(h, j) = dov;
            D += dot4(dov, o);
            ou += dot4(o, u);
            ov += dot4(o, v);
        }
        D = quad_add(D);
        ou = quad_add(ou);
        ov = quad_add(ov);
        if (lead) {
            a.Dd[t * H + h] = D;
            a.cf[t * H + h] = coef;
            a.wn[t * H + h] = w;
        }
        if (a.variant == GQE_VARIANT_WEIGHTED_CONCAT) dp[jr] += ou;
        dw[r] = ov;
    }
    if (rslot) {
        float sw = 0.f;
        for (int r = 0; r < k; ++r) sw += (p[id[r] - g * n] / psel) * dw[r];
        for (int r = 0; r < k; ++r) dp[id[r] - g * n] += (dw[r] - sw) / psel;
    }
    // aux = (1/G) sum_g n sum_e f_e P_e, P_e = mean_t p[t, e]: dp[t, e] += aux_coef n f_e / (G T)
    for (int jj = 0; jj < n; ++jj) {
        const double f = (double)a.counts[g * n + jj] / ((double)a.T * (double)k);
        dp[jj] += (float)(a.aux_coef * (double)n * f / ((double)a.G * (double)a.T));
    }
    float sdp = 0.f;
    for (int jj = 0; jj < n; ++jj) sdp += p[jj] * dp[jj];
    if (lead)
        for (int jj = 0; jj < n; ++jj) a.dl[t * a.N + g * n + jj] = p[jj] * (dp[jj] - sdp);
}

// ---------------------------------------------------------------- attention
// Both kernels: four lanes per row, each holding a quarter of the head dims (DQ = d_h / 4); dot
// products are summed over the four lanes with DPP quad permutations.  Tiles of 64 keys or queries
// are staged in LDS as float32.

__device__ __forceinline__ float quad_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false));  // xor 1
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, false));  // xor 2
    return v;
}

constexpr int kPitch = 132;  // LDS row pitch (floats): 16-byte aligned rows, d_h <= 128

// dq for a block of 64 queries of one (sequence, head): pass 1 recomputes each row's log-sum-exp
// over the causal keys (online, log2 units), pass 2 sums dz_j k_j with dz_j = p_j (do . v_j - D).
template <typename T, int DQ>
__global__ void __launch_bounds__(256) bwd_dq_kernel(BwdArgs a) {
    __shared__ __align__(16) float ks[64][kPitch];
    __shared__ __align__(16) float vs[64][kPitch];
    const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int g = group_of(a, h);
    const int dh = a.dh;
    const int qi = tid >> 2, qd = tid & 3, d0 = qd * DQ;
    const int64_t s = (int64_t)qb * 64 + qi;
    const bool valid = s < a.S;
    const int64_t sq = valid ? s : a.S - 1;
    const int64_t t = b * a.S + sq;
    float q[DQ], dov[DQ], dq[DQ];
    const int64_t qo = ((b * a.H + h) * a.S + sq) * dh + d0;
#pragma unroll
    for (int i = 0; i < DQ; ++i) {
        q[i] = ld<T>(a.Q, qo + i);
        dov[i] = a.dO[(t * a.H + h) * dh + d0 + i];
        dq[i] = 0.f;
    }
    const float D = a.Dd[t * a.H + h];
    const int64_t kbase = (b * a.G + g) * a.S_pad * dh;
    const int64_t vbase = (b * a.G + g) * dh * a.S_pad;
    const int ntiles = qb + 1;  // causal: key tiles up to the diagonal
    auto stage = [&](int kt, bool withv) {
        __syncthreads();
        for (int i = tid; i < 64 * dh; i += 256) {
            const int kk = i / dh, c = i - kk * dh;
            const int64_t kp = (int64_t)kt * 64 + kk;
            ks[kk][c] = kp < a.S ? ld<T>(a.K, kbase + kp * dh + c) : 0.f;
        }
        if (withv)
            for (int i = tid; i < 64 * dh; i += 256) {
                const int c = i / 64, kk = i & 63;  // neighbouring threads: neighbouring keys of V^T
                const int64_t kp = (int64_t)kt * 64 + kk;
                vs[kk][c] = kp < a.S ? ld<T>(a.Vt, vbase + (int64_t)c * a.S_pad + vt_pos(kp)) : 0.f;
            }
        __syncthreads();
    };
    // pass 1: log-sum-exp of the row
    float m = -INFINITY, l = 0.f;
    for (int kt = 0; kt < ntiles; ++kt) {
        stage(kt, false);
        const int nk = (int)min<int64_t>(64, sq + 1 - (int64_t)kt * 64);
        for (int kk = 0; kk < 64; ++kk) {
            float p = 0.f;
#pragma unroll
            for (int i = 0; i < DQ; i += 4) {
                const f32x4_t kv = *reinterpret_cast<const f32x4_t*>(&ks[kk][d0 + i]);
                p += q[i] * kv[0] + q[i + 1] * kv[1] + q[i + 2] * kv[2] + q[i + 3] * kv[3];
            }
            const float sc = kk < nk ? quad_sum(p) : -INFINITY;
            const float mn = fmaxf(m, sc);
            l = l * __builtin_amdgcn_exp2f(m - mn) + __builtin_amdgcn_exp2f(sc - mn);
            m = mn;
        }
    }
    const float L = m + __builtin_amdgcn_logf(l);
    // pass 2
    for (int kt = 0; kt < ntiles; ++kt) {
        stage(kt, true);
        const int nk = (int)min<int64_t>(64, sq + 1 - (int64_t)kt * 64);
        for (int kk = 0; kk < 64; ++kk) {
            float p = 0.f, da = 0.f;
            f32x4_t kr[DQ / 4];
#pragma unroll
            for (int i = 0; i < DQ; i += 4) {
                kr[i / 4] = *reinterpret_cast<const f32x4_t*>(&ks[kk][d0 + i]);
                const f32x4_t vv = *reinterpret_cast<const f32x4_t*>(&vs[kk][d0 + i]);
#pragma unroll
                for (int z = 0; z < 4; ++z) {
                    p += q[i + z] * kr[i / 4][z];
                    da += dov[i + z] * vv[z];
                }
            }
            const float sc = quad_sum(p), dA = quad_sum(da);
            const float dz = kk < nk ? __builtin_amdgcn_exp2f(sc - L) * (dA - D) : 0.f;
#pragma unroll
            for (int i = 0; i < DQ; ++i) dq[i] += dz * kr[i / 4][i % 4];
        }
    }
    if (!valid) return;
    const float sc = 1.f / sqrtf((float)dh);
#pragma unroll
    for (int i = 0; i < DQ; ++i) dq[i] *= sc;
    if (a.rope)
#pragma unroll
        for (int i = 0; i < DQ; i += 2) rope_pair(dq[i], dq[i + 1], -s, a.rope[(d0 + i) >> 1]);
#pragma unroll
    for (int i = 0; i < DQ; ++i) gwrite<T>(a.dQ, (t * a.H + h) * dh + d0 + i, dq[i]);
    if (qd == 0) a.lse[t * a.H + h] = L;
}

// dk, dv for a block of 64 keys of one (sequence, group): every later query of every head of the
// group, query tiles of 64 staged in LDS with their log-sum-exp and D.
template <typename T, int DQ>
__global__ void __launch_bounds__(256) bwd_dkv_kernel(BwdArgs a) {
    __shared__ __align__(16) float qs[64][kPitch];
    __shared__ __align__(16) float ds[64][kPitch];
    __shared__ float ls[64], dd[64];
    const int kb = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int dh = a.dh;
    const int kj = tid >> 2, qd = tid & 3, d0 = qd * DQ;
    const int64_t j = (int64_t)kb * 64 + kj;
    const bool valid = j < a.S;
    const int64_t jk = valid ? j : a.S - 1;
    float k[DQ], v[DQ], dk[DQ], dv[DQ];
    const int64_t kbase = ((b * a.G + g) * a.S_pad + jk) * dh + d0;
    const int64_t vbase = (b * a.G + g) * dh * a.S_pad;
#pragma unroll
    for (int i = 0; i < DQ; ++i) {
        k[i] = ld<T>(a.K, kbase + i);
        v[i] = ld<T>(a.Vt, vbase + (int64_t)(d0 + i) * a.S_pad + vt_pos(jk));
        dk[i] = dv[i] = 0.f;
    }
    const int nqt = (int)ceil_div(a.S, 64);
    for (int h = 0; h < a.H; ++h) {
        if (group_of(a, h) != g) continue;  // uniform over the work group
        for (int qt = kb; qt < nqt; ++qt) {
            __syncthreads();
            for (int i = tid; i < 64 * dh; i += 256) {
                const int qq = i / dh, c = i - qq * dh;
                const int64_t sp = (int64_t)qt * 64 + qq;
                const bool in = sp < a.S;
                qs[qq][c] = in ? ld<T>(a.Q, ((b * a.H + h) * a.S + sp) * dh + c) : 0.f;
                ds[qq][c] = in ? a.dO[((b * a.S + sp) * a.H + h) * dh + c] : 0.f;
            }
            if (tid < 64) {
                const int64_t sp = (int64_t)qt * 64 + tid;
                const int64_t ti = (b * a.S + (sp < a.S ? sp : 0)) * a.H + h;
                ls[tid] = a.lse[ti];
                dd[tid] = a.Dd[ti];
            }
            __syncthreads();
            for (int qq = 0; qq < 64; ++qq) {
                const int64_t sp = (int64_t)qt * 64 + qq;
                float p = 0.f, da = 0.f;
                f32x4_t qr[DQ / 4], dr[DQ / 4];
#pragma unroll
                for (int i = 0; i < DQ; i += 4) {
                    qr[i / 4] = *reinterpret_cast<const f32x4_t*>(&qs[qq][d0 + i]);
                    dr[i / 4] = *reinterpret_cast<const f32x4_t*>(&ds[qq][d0 + i]);
#pragma unroll
                    for (int z = 0; z < 4; ++z) {
                        p += qr[i / 4][z] * k[i + z];
                        da += dr[i / 4][z] * v[i + z];
                    }
                }
                const float sc = quad_sum(p), dA = quad_sum(da);
                const bool on = sp < a.S && sp >= jk;
                const float pj = on ? __builtin_amdgcn_exp2f(sc - ls[qq]) : 0.f;
                const float dz = pj * (dA - dd[qq]);
#pragma unroll
                for (int i = 0; i < DQ; ++i) {
                    dk[i] += dz * qr[i / 4][i % 4];
                    dv[i] += pj * dr[i / 4][i % 4];
                }
            }
        }
    }
    if (!valid) return;
    // the stored queries carry log2(e)/sqrt(d_h): q / sqrt(d_h) = q~ / log2(e)
#pragma unroll
    for (int i = 0; i < DQ; ++i) dk[i] *= 1.f / kLog2e;
    if (a.rope)
#pragma unroll
        for (int i = 0; i < DQ; i += 2) rope_pair(dk[i], dk[i + 1], -j, a.rope[(d0 + i) >> 1]);
    const int64_t t = b * a.S + j;
#pragma unroll
    for (int i = 0; i < DQ; ++i) {
        gwrite<T>(a.dK, (t * a.G + g) * dh + d0 + i, dk[i]);
        gwrite<T>(a.dV, (t * a.G + g) * dh + d0 + i, dv[i]);
    }
}

// ---------------------------------------------------------------- attention on matrix cores (bf16)
// v_mfma_f32_16x16x16_bf16: A lane l = row l % 16, k 4 (l / 16) .. +3; B lane l = column l % 16, same
// k; C lane l = column l % 16, rows 4 (l / 16) .. +3.  The C tile of S = Q K^T (rows = queries,
// columns = keys) is, lane for lane, the A operand of a product whose rows are the keys and whose k
// index runs over the queries (P^T dO, dS^T Q): probabilities and score gradients go from the
// accumulators to the next product without any exchange; likewise S^T = K Q^T feeds dS K.  P and dS
// are rounded to bf16 for the products (the forward pass feeds P to its P.V product the same way).
typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mma16(const s16x4_t& a, const s16x4_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ s16x4_t lds8(const uint16_t* p) { return *reinterpret_cast<const s16x4_t*>(p); }
// sixteen bytes (eight bf16) from LDS or global memory, and two four-element pieces joined
__device__ __forceinline__ bf16x8_t ld16b(const uint16_t* p) { return *reinterpret_cast<const bf16x8_t*>(p); }
__device__ __forceinline__ bf16x8_t join8(const s16x4_t& lo, const s16x4_t& hi) {
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ f32x4_t mma32(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// c + A B for a 16 x 16 x 16 product whose sum c a 16 x 16 x 32 product may have just written: the
// 16 x 16 x 16 product goes to its own zero accumulator and the two are added on the vector ALU.
// Chained through the accumulator operand instead (no wait states between the two in the generated
// code), the pair gave wrong sums on gfx950 in the parity tests.
__device__ __forceinline__ f32x4_t mma16_add(const s16x4_t& a, const s16x4_t& b, const f32x4_t& c) {
    return c + mma16(a, b, f32x4_t{0.f, 0.f, 0.f, 0.f});
}
__device__ __forceinline__ s16x4_t gld8(const uint16_t* p) { return *reinterpret_cast<const s16x4_t*>(p); }
__device__ __forceinline__ float swap_x1(float v) {  // the value of lane ^ 1
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false));
}

// row-major V and bf16 dO (rows past the sequence zero) for the matrix-core kernels
// thread per eight head dims of one row: V rows gathered from V^T with neighbouring threads on
// neighbouring keys (coalesced reads), dO rows converted with neighbouring threads on neighbouring
// dims; one 16-byte store each
__global__ void bwd_mprep_kernel(BwdArgs a, uint16_t* __restrict__ Vr, uint16_t* __restrict__ dOb) {
    const int c8n = a.dh / 8;
    const int64_t nv = a.B * a.G * a.S_pad * c8n, no = a.B * a.H * a.S_pad * c8n;
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q < nv) {
        const int64_t s = q % a.S_pad, rem = q / a.S_pad;
        const int c8 = (int)(rem % c8n);
        const int64_t bg = rem / c8n;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (s < a.S) {
            const uint16_t* src = reinterpret_cast<const uint16_t*>(a.Vt) + (bg * a.dh + 8 * c8) * a.S_pad + vt_pos(s);
#pragma unroll
            for (int e = 0; e < 8; e += 2)
                v[e >> 1] = (uint32_t)src[(int64_t)e * a.S_pad] | ((uint32_t)src[(int64_t)(e + 1) * a.S_pad] << 16);
        }
        *reinterpret_cast<u32x4_t*>(Vr + (bg * a.S_pad + s) * a.dh + 8 * c8) = v;
    } else if (q < nv + no) {
        const int64_t i = q - nv;
        const int c8 = (int)(i % c8n);
        const int64_t r = i / c8n, s = r % a.S_pad, bh = r / a.S_pad, b = bh / a.H, h = bh % a.H;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (s < a.S) {
            float f[8];
            ld8f(a.dO + ((b * a.S + s) * a.H + h) * a.dh + 8 * c8, f);
            v = pack8(f);
        }
        *reinterpret_cast<u32x4_t*>(dOb + (bh * a.S_pad + s) * a.dh + 8 * c8) = v;
    }
}

// dk, dv of 128 keys (wave w: keys 32 w .. 32 w + 31, two 16-key column groups) of one (sequence,
// group) over the later queries of every head of the group, query tiles of 64 staged in LDS
// row-major (the gradient products read them transposed with ds_read_b64_tr_b16); every fragment
// read from LDS feeds the products of both column groups.
// 16 x 16 products in v_mfma_f32_16x16x32_bf16 (v_mfma_f32_16x16x16_bf16 for a last 16 head dims):
// the score products contract the head dims, the gradient products P^T dO and dS^T Q contract 32
// queries at a time -- the lane's four queries of two consecutive 16-query blocks, the transposed
// tiles read in the same order.
// Two waves per SIMD up to d_h = 48 (the compiler fits the registers in 256 with a few dwords of
// spill; one wave per SIMD left the matrix core idle during every wait); larger head dims keep one
// wave per SIMD (their spills at 256 registers are larger).
template <int DH>
__global__ void __launch_bounds__(256, DH <= 48 ? 2 : 1) bwd_dkv_mfma_kernel(BwdArgs a, const uint16_t* __restrict__ Vr,
                                                           const uint16_t* __restrict__ dOb) {
    constexpr int NC = DH / 16, N32 = DH / 32, R16 = (DH % 32) / 16, P1 = DH + 8;
    constexpr int F32 = N32 > 0 ? N32 : 1;
    __shared__ __align__(16) uint16_t Qs[64 * P1], dOs[64 * P1];
    __shared__ float lss[64], dds[64];
    // longest first: key block 0 (every query tile after it) of every (group, sequence) leads
    // one work group per (key block, group, sequence), and one more per (key block, sequence) for
    // the shared head: the shared head's group would otherwise carry twice the work of the others
    // on the longest (first) key blocks; the two parts of that group go to float32 partials
    const int GS = a.G + a.s;
    const int kb = (int)(blockIdx.x / (GS * a.B)), gi = (int)(blockIdx.x % GS), b = (int)(blockIdx.x / GS % a.B);
    const bool shared_part = gi == a.G;
    const int g = shared_part ? a.skv : gi;
    const bool split = a.s && g == a.skv;
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, j4 = lane >> 4;
    const int64_t S = a.S;
    const uint16_t* Kb = reinterpret_cast<const uint16_t*>(a.K) + ((int64_t)(b * a.G + g) * a.S_pad) * DH;
    const uint16_t* Vb = Vr + ((int64_t)(b * a.G + g) * a.S_pad) * DH;
    int64_t key[2];  // this lane's key column in each group
    bool kin[2];
    // key and value fragments of the score products: head dims 32 c + 8 j4 .. + 7, and of a last
    // 16 (R16) dims 32 N32 + 4 j4 .. + 3
    bf16x8_t kf[2][F32], vf[2][F32];
    s16x4_t kt16[2], vt16[2];
    f32x4_t dk[2][NC], dv[2][NC];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        key[u] = (int64_t)kb * 128 + w * 32 + 16 * u + l16;
        kin[u] = key[u] < S;
#pragma unroll
        for (int c = 0; c < N32; ++c) {
            kf[u][c] = kin[u] ? ld16b(Kb + key[u] * DH + 32 * c + 8 * j4) : bf16x8_t{};
            vf[u][c] = kin[u] ? ld16b(Vb + key[u] * DH + 32 * c + 8 * j4) : bf16x8_t{};
        }
        kt16[u] = vt16[u] = s16x4_t{0, 0, 0, 0};
        if (R16 && kin[u]) {
            kt16[u] = gld8(Kb + key[u] * DH + 32 * N32 + 4 * j4);
            vt16[u] = gld8(Vb + key[u] * DH + 32 * N32 + 4 * j4);
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) dk[u][c] = dv[u][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const int nqt = (int)ceil_div(S, 64);
    const uint16_t* Qg = reinterpret_cast<const uint16_t*>(a.Q);
    // (head of the group, query tile) pairs in order; the next pair's Q, dO, log-sum-exp and D are
    // loaded into registers while the current pair multiplies
    const int nh = shared_part ? 1 : a.k;
    const int qt0 = 2 * kb, ntl = nqt - qt0, total = nh * ntl;
    auto head = [&](int hi) { return shared_part ? a.G * a.k : g * a.k + hi; };
    // staging: thread = (four neighbouring rows, one 8-dim chunk); R = the four rows.  Up to d_h = 64
    // (SPLIT) waves 0-1 stage Q and waves 2-3 dO, so a staging thread does half the work and holds
    // half the prefetch registers; above, every staging thread does both
    constexpr int NQC = 16 * (DH / 8), R = 4;
    constexpr bool SPLIT = NQC <= 128;
    static_assert(NQC <= 256, "d_h <= 128");
    const bool dorole = SPLIT && tid >= 128;  // this thread stages dO (wave-uniform)
    const int sid = SPLIT ? (tid & 127) : tid;
    const bool stager = sid < NQC;
    const int rq = (sid / (DH / 8)) * 4, cq = sid % (DH / 8);
    u32x4_t pq[R], pd[SPLIT ? 1 : R];
    float pl = 0.f, pdd = 0.f;
    auto fetch = [&](int it) {
        const int h = head(it / ntl), qt = qt0 + it % ntl;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int q = rq + r, c8 = cq;
            const int64_t qp = (int64_t)qt * 64 + q;
            pq[r] = u32x4_t{0u, 0u, 0u, 0u};
            if (!SPLIT) pd[SPLIT ? 0 : r] = u32x4_t{0u, 0u, 0u, 0u};
            if (stager && qp < S) {
                const uint16_t* qsrc = Qg + (((int64_t)b * a.H + h) * S + qp) * DH + 8 * c8;
                const uint16_t* dsrc = dOb + (((int64_t)b * a.H + h) * a.S_pad + qp) * DH + 8 * c8;
                if (SPLIT) {
                    pq[r] = *reinterpret_cast<const u32x4_t*>(dorole ? dsrc : qsrc);
                } else {
                    pq[r] = *reinterpret_cast<const u32x4_t*>(qsrc);
                    pd[SPLIT ? 0 : r] = *reinterpret_cast<const u32x4_t*>(dsrc);
                }
            }
        }
        if (tid < 64) {
            const int64_t qp = (int64_t)qt * 64 + tid;
            const int64_t ti = (b * S + (qp < S ? qp : 0)) * a.H + h;
            pl = a.lse[ti];
            pdd = a.Dd[ti];
        }
    };
    if (total > 0) fetch(0);
    for (int it = 0; it < total; ++it) {
        const int qt = qt0 + it % ntl;
        __syncthreads();  // the previous pair's products are done with the tiles
        if (stager) {
            if (SPLIT) {
                uint16_t* const rowm = dorole ? dOs : Qs;
#pragma unroll
                for (int r = 0; r < R; ++r) *reinterpret_cast<u32x4_t*>(&rowm[(rq + r) * P1 + 8 * cq]) = pq[r];
            } else {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    *reinterpret_cast<u32x4_t*>(&Qs[(rq + r) * P1 + 8 * cq]) = pq[r];
                    *reinterpret_cast<u32x4_t*>(&dOs[(rq + r) * P1 + 8 * cq]) = pd[SPLIT ? 0 : r];
                }
            }
        }
        if (tid < 64) {
            lss[tid] = pl;
            dds[tid] = pdd;
        }
        __syncthreads();
        if (it + 1 < total) fetch(it + 1);
        // a query tile wholly after the block's last key and inside the sequence masks nothing
        const bool inside = (int64_t)qt * 64 >= (int64_t)kb * 128 + 128 && (int64_t)qt * 64 + 64 <= S;
        // pairs of 16-query blocks: queries qp .. qp + 31 of the tile
#pragma unroll
        for (int qp = 0; qp < 64; qp += 32) {
            bf16x8_t qa[2][F32], da_[2][F32];
            s16x4_t qa16[2], da16[2];
            float lq[2][4], dq4[2][4];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int q0 = qp + 16 * h2;
#pragma unroll
                for (int c = 0; c < N32; ++c) {
                    qa[h2][c] = ld16b(&Qs[(q0 + l16) * P1 + 32 * c + 8 * j4]);
                    da_[h2][c] = ld16b(&dOs[(q0 + l16) * P1 + 32 * c + 8 * j4]);
                }
                qa16[h2] = da16[h2] = s16x4_t{0, 0, 0, 0};
                if (R16) {
                    qa16[h2] = lds8(&Qs[(q0 + l16) * P1 + 32 * N32 + 4 * j4]);
                    da16[h2] = lds8(&dOs[(q0 + l16) * P1 + 32 * N32 + 4 * j4]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    lq[h2][i] = lss[q0 + 4 * j4 + i];
                    dq4[h2][i] = dds[q0 + 4 * j4 + i];
                }
            }
            // Q and dO transposed on the read (ds_read_b64_tr_b16): lane j of a 16-lane group
            // addresses row row0 + j / 4, columns col0 + 4 (j % 4) .. + 3, and lane i receives rows
            // row0 .. row0 + 3 of column col0 + i -- head dim 16 c + l16, the lane's four queries of
            // each of the two blocks
            typedef __attribute__((address_space(3))) s16x4_t* lds_s4;
            auto trq = [&](const uint16_t* T, int row0, int col0) {
                return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s4)(&T[(row0 + (l16 >> 2)) * P1 + col0 + 4 * (l16 & 3)]));
            };
            bf16x8_t qtb[NC], dtb[NC];
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                qtb[c] = join8(trq(Qs, qp + 4 * j4, 16 * c), trq(Qs, qp + 16 + 4 * j4, 16 * c));
                dtb[c] = join8(trq(dOs, qp + 4 * j4, 16 * c), trq(dOs, qp + 16 + 4 * j4, 16 * c));
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                float p[8], ds[8];
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int c = 0; c < N32; ++c) {
                        sacc = mma32(qa[h2][c], kf[u][c], sacc);
                        dp = mma32(da_[h2][c], vf[u][c], dp);
                    }
                    if (R16) {
                        sacc = mma16_add(qa16[h2], kt16[u], sacc);
                        dp = mma16_add(da16[h2], vt16[u], dp);
                    }
                    if (inside) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            p[4 * h2 + i] = __builtin_amdgcn_exp2f(sacc[i] - lq[h2][i]);
                            ds[4 * h2 + i] = p[4 * h2 + i] * (dp[i] - dq4[h2][i]);
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int64_t qpos = (int64_t)qt * 64 + qp + 16 * h2 + 4 * j4 + i;
                            const bool on = kin[u] && qpos < S && qpos >= key[u];
                            p[4 * h2 + i] = on ? __builtin_amdgcn_exp2f(sacc[i] - lq[h2][i]) : 0.f;
                            ds[4 * h2 + i] = on ? p[4 * h2 + i] * (dp[i] - dq4[h2][i]) : 0.f;
                        }
                    }
                }
                const bf16x8_t pa = __builtin_bit_cast(bf16x8_t, pack8(p));
                const bf16x8_t dsa = __builtin_bit_cast(bf16x8_t, pack8(ds));
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    dv[u][c] = mma32(pa, dtb[c], dv[u][c]);
                    dk[u][c] = mma32(dsa, qtb[c], dk[u][c]);
                }
            }
        }
    }
    // C layout: lane column = head dim 16 c + l16, rows = keys 32 w + 16 u + 4 j4 + i
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t kp = (int64_t)kb * 128 + w * 32 + 16 * u + 4 * j4 + i;
                const int col = 16 * c + l16;
                float kv = dk[u][c][i] * (1.f / kLog2e);
                if (a.rope) {
                    const float other = swap_x1(kv);  // pair partner: the neighbouring column
                    float lo = (l16 & 1) ? other : kv, hi = (l16 & 1) ? kv : other;
                    rope_pair(lo, hi, -kp, a.rope[col >> 1]);
                    kv = (l16 & 1) ? hi : lo;
                }
                if (kp < S) {
                    if (split) {
                        const int64_t T = a.T, o = (b * S + kp) * DH + col;
                        a.kvp[(shared_part ? 1 : 0) * T * DH + o] = kv;
                        a.kvp[(shared_part ? 3 : 2) * T * DH + o] = dv[u][c][i];
                    } else {
                        gwrite<bf16_t>(a.dK, ((b * S + kp) * a.G + g) * DH + col, kv);
                        gwrite<bf16_t>(a.dV, ((b * S + kp) * a.G + g) * DH + col, dv[u][c][i]);
                    }
                }
            }
}

// the shared head's group: dK = routed part + shared part, dV likewise, rounded once to bf16
__global__ void bwd_kv_sum_kernel(BwdArgs a) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t n = a.T * a.dh;
    if (q >= n) return;
    const int64_t t = q / a.dh;
    const int c = (int)(q % a.dh);
    const int64_t o = (t * a.G + a.skv) * a.dh + c;
    gwrite<bf16_t>(a.dK, o, a.kvp[q] + a.kvp[n + q]);
    gwrite<bf16_t>(a.dV, o, a.kvp[2 * n + q] + a.kvp[3 * n + q]);
}

constexpr int kDqWaves = 8;  // waves of the query-block kernel (16 queries each)

// dq of 16 kDqWaves queries (wave w: queries 16 w ..) of one (sequence, head): pass 1 the row log-sum-exp,
// pass 2 dS^T = P^T (dP^T - D) and dq += dS K over the causal key tiles.
template <int DH>
__global__ void __launch_bounds__(64 * kDqWaves) bwd_dq_mfma_kernel(BwdArgs a, const uint16_t* __restrict__ Vr,
                                                                    const uint16_t* __restrict__ dOb) {
    constexpr int NC = DH / 16, N32 = DH / 32, R16 = (DH % 32) / 16, P1 = DH + 8;
    constexpr int F32 = N32 > 0 ? N32 : 1;
    constexpr int QB = 16 * kDqWaves;  // queries per work group, 16 per wave
    __shared__ __align__(16) uint16_t Ks[64 * P1], Vs[64 * P1];
    // longest first: the last query block (every key tile before it) of every (head, sequence) leads
    const int nqb = (int)ceil_div(a.S, QB);
    const int qb = nqb - 1 - (int)(blockIdx.x / (a.H * a.B));
    const int h = (int)(blockIdx.x % a.H), b = (int)(blockIdx.x / a.H % a.B);
    const int tid = threadIdx.x;
    const int g = group_of(a, h);
    const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, j4 = lane >> 4;
    const int64_t S = a.S;
    const int64_t qpos = (int64_t)qb * QB + w * 16 + l16;  // this lane's query column
    const bool qin = qpos < S;
    const uint16_t* Qg = reinterpret_cast<const uint16_t*>(a.Q);
    // query and dO fragments of the score products: head dims 32 c + 8 j4 .. + 7, and of a last 16
    // (R16) dims 32 N32 + 4 j4 .. + 3
    bf16x8_t qf[F32], df[F32];
    s16x4_t qf16 = {0, 0, 0, 0}, df16 = {0, 0, 0, 0};
    {
        const uint16_t* qrow = Qg + (((int64_t)b * a.H + h) * S + qpos) * DH;
        const uint16_t* drow = dOb + (((int64_t)b * a.H + h) * a.S_pad + qpos) * DH;
#pragma unroll
        for (int c = 0; c < N32; ++c) {
            qf[c] = qin ? ld16b(qrow + 32 * c + 8 * j4) : bf16x8_t{};
            df[c] = qin ? ld16b(drow + 32 * c + 8 * j4) : bf16x8_t{};
        }
        if (R16 && qin) {
            qf16 = gld8(qrow + 32 * N32 + 4 * j4);
            df16 = gld8(drow + 32 * N32 + 4 * j4);
        }
    }
    const float Dq = qin ? a.Dd[(b * S + qpos) * a.H + h] : 0.f;
    const uint16_t* Kb = reinterpret_cast<const uint16_t*>(a.K) + ((int64_t)(b * a.G + g) * a.S_pad) * DH;
    const uint16_t* Vb = Vr + ((int64_t)(b * a.G + g) * a.S_pad) * DH;
    const int ntile = (int)((min((int64_t)qb * QB + QB, S) - 1) / 64) + 1;  // key tiles up to the last query
    // pass 1 (iterations 0 .. ntile - 1): each lane folds its four keys of every sub-tile into
    // (m, l); then the four lanes of a query column are combined into the row log-sum-exp L.
    // Skipped when the forward's attention stored L (the same scores, with its row sums).
    // pass 2 (ntile .. 2 ntile - 1): dS^T = P^T (dP^T - D), dq += dS K.  The next iteration's key
    // (and value) tile is loaded into registers while the current one multiplies.  16 x 16 products in
    // v_mfma_f32_16x16x32_bf16 (v_mfma_f32_16x16x16_bf16 for a last 16 head dims); dq += dS K
    // contracts 32 keys at a time (the lane's four keys of two consecutive 16-key sub-tiles, K read
    // transposed in the same order with ds_read_b64_tr_b16).
    // staging: thread = (four neighbouring rows, one 8-dim chunk); R = the four rows.  Up to d_h = 64
    // (SPLIT) threads 0 .. 127 stage K and threads 128 .. 255 stage V
    // (pass 2); above, every staging thread does both
    constexpr int NQC = 16 * (DH / 8), R = 4;
    constexpr bool SPLIT = NQC <= 128 && 64 * kDqWaves >= 256;
    static_assert(NQC <= 256, "d_h <= 128");
    const bool vrole = SPLIT && tid >= 128 && tid < 256;  // this thread stages V (wave-uniform)
    const int sid = SPLIT ? (tid & 127) : tid;
    const bool stager = (SPLIT ? tid < 256 : true) && sid < NQC;
    const int rq = (sid / (DH / 8)) * 4, cq = sid % (DH / 8);
    u32x4_t pk[R], pv[SPLIT ? 1 : R];
    auto fetch = [&](int it) {
        const int kt = it % ntile;
        const bool full = it >= ntile;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int kk = rq + r, c8 = cq;
            const int64_t kp = (int64_t)kt * 64 + kk;
            pk[r] = u32x4_t{0u, 0u, 0u, 0u};
            if (!SPLIT) pv[SPLIT ? 0 : r] = u32x4_t{0u, 0u, 0u, 0u};
            if (stager && kp < S) {
                if (SPLIT) {
                    if (!vrole || full) pk[r] = *reinterpret_cast<const u32x4_t*>((vrole ? Vb : Kb) + kp * DH + 8 * c8);
                } else {
                    pk[r] = *reinterpret_cast<const u32x4_t*>(Kb + kp * DH + 8 * c8);
                    if (full) pv[SPLIT ? 0 : r] = *reinterpret_cast<const u32x4_t*>(Vb + kp * DH + 8 * c8);
                }
            }
        }
    };
    float m = -INFINITY, l = 0.f, L = 0.f;
    f32x4_t dq[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) dq[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // with the forward's log-sum-exp the first pass is skipped
    const int it0 = a.lse_fwd ? ntile : 0;
    if (a.lse_fwd) L = qin ? a.lse[(b * S + qpos) * a.H + h] : 0.f;
    fetch(it0);
    for (int it = it0; it < 2 * ntile; ++it) {
        const int kt = it % ntile;
        const bool full = it >= ntile;
        __syncthreads();  // the previous tile's products are done
        if (stager && (!vrole || full)) {
            uint16_t* const rowm = vrole ? Vs : Ks;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                *reinterpret_cast<u32x4_t*>(&rowm[(rq + r) * P1 + 8 * cq]) = pk[r];
                if (!SPLIT && full) *reinterpret_cast<u32x4_t*>(&Vs[(rq + r) * P1 + 8 * cq]) = pv[SPLIT ? 0 : r];
            }
        }
        __syncthreads();
        if (it + 1 < 2 * ntile) fetch(it + 1);
        if (it == ntile && !a.lse_fwd) {  // first pass-2 tile: finish the log-sum-exp
#pragma unroll
            for (int o = 0; o < 2; ++o) {
                float mo, lo;
                if (o == 0) {
                    const auto sm = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
                    const auto sl = __builtin_amdgcn_permlane16_swap(__float_as_uint(l), __float_as_uint(l), false, false);
                    mo = (j4 & 1) ? __uint_as_float(sm[0]) : __uint_as_float(sm[1]);
                    lo = (j4 & 1) ? __uint_as_float(sl[0]) : __uint_as_float(sl[1]);
                } else {
                    const auto sm = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
                    const auto sl = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
                    mo = (j4 & 2) ? __uint_as_float(sm[0]) : __uint_as_float(sm[1]);
                    lo = (j4 & 2) ? __uint_as_float(sl[0]) : __uint_as_float(sl[1]);
                }
                if (mo != -INFINITY) {
                    if (m == -INFINITY) {
                        m = mo;
                        l = lo;
                    } else {
                        const float mn = fmaxf(m, mo);
                        l = l * __builtin_amdgcn_exp2f(m - mn) + lo * __builtin_amdgcn_exp2f(mo - mn);
                        m = mn;
                    }
                }
            }
            L = m + __builtin_amdgcn_logf(l);
        }
        typedef __attribute__((address_space(3))) s16x4_t* lds_s4;
        // lane j of a 16-lane group addresses key row0 + j / 4, dims col0 + 4 (j % 4) .. + 3; lane i
        // receives keys row0 .. row0 + 3 of dim col0 + i
        auto trk = [&](int row0, int col0) {
            return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(&Ks[(row0 + (l16 >> 2)) * P1 + col0 + 4 * (l16 & 3)]));
        };
        // S^T (rows keys k0 + 4 j4 + i, column the lane's query) of one 16-key sub-tile
        auto scores = [&](const uint16_t* Tl, int k0, const bf16x8_t (&f)[F32], const s16x4_t& f16) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < N32; ++c) acc = mma32(ld16b(&Tl[(k0 + l16) * P1 + 32 * c + 8 * j4]), f[c], acc);
            if (R16) acc = mma16_add(lds8(&Tl[(k0 + l16) * P1 + 32 * N32 + 4 * j4]), f16, acc);
            return acc;
        };
        if (!full) {
#pragma unroll
            for (int sub = 0; sub < 4; ++sub) {
                const int k0 = sub * 16;
                const f32x4_t st = scores(Ks, k0, qf, qf16);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t kp = (int64_t)kt * 64 + k0 + 4 * j4 + i;
                    if (kp <= qpos && kp < S) {
                        const float mn = fmaxf(m, st[i]);
                        l = l * __builtin_amdgcn_exp2f(m - mn) + __builtin_amdgcn_exp2f(st[i] - mn);
                        m = mn;
                    }
                }
            }
        } else {
            // a key tile wholly before the query block masks nothing but the rows past the end
            const bool inside = (int64_t)kt * 64 + 64 <= (int64_t)qb * QB;
#pragma unroll
            for (int sp = 0; sp < 64; sp += 32) {
                float ds[8];
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const int k0 = sp + 16 * h2;
                    const f32x4_t st = scores(Ks, k0, qf, qf16), dpt = scores(Vs, k0, df, df16);
                    if (inside) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) ds[4 * h2 + i] = qin ? __builtin_amdgcn_exp2f(st[i] - L) * (dpt[i] - Dq) : 0.f;
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int64_t kp = (int64_t)kt * 64 + k0 + 4 * j4 + i;
                            const bool on = qin && kp <= qpos && kp < S;
                            ds[4 * h2 + i] = on ? __builtin_amdgcn_exp2f(st[i] - L) * (dpt[i] - Dq) : 0.f;
                        }
                    }
                }
                const bf16x8_t da = __builtin_bit_cast(bf16x8_t, pack8(ds));
                // K transposed on the read (ds_read_b64_tr_b16): head dim 16 c + l16, the lane's
                // four keys of each of the two 16-key sub-tiles
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    dq[c] = mma32(da, join8(trk(sp + 4 * j4, 16 * c), trk(sp + 16 + 4 * j4, 16 * c)), dq[c]);
            }
        }
    }
    // C layout: lane column = head dim 16 c + l16, rows = queries 16 w + 4 j4 + i
    const float sc = 1.f / sqrtf((float)DH);
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t qr = (int64_t)qb * QB + w * 16 + 4 * j4 + i;
            const int col = 16 * c + l16;
            float v = dq[c][i] * sc;
            if (a.rope) {
                const float other = swap_x1(v);
                float lo = (l16 & 1) ? other : v, hi = (l16 & 1) ? v : other;
                rope_pair(lo, hi, -qr, a.rope[col >> 1]);
                v = (l16 & 1) ? hi : lo;
            }
            if (qr < S) gwrite<bf16_t>(a.dQ, ((b * S + qr) * a.H + h) * DH + col, v);
        }
    if (j4 == 0 && qin && !a.lse_fwd) a.lse[(b * S + qpos) * a.H + h] = L;
}

// ---------------------------------------------------------------- tiled float32 GEMM
// C[M][N] (=, +=) sum_k A(m, k) B(k, n) for a set of sub-problems (blockIdx.z): 64 x 64 tiles of C,
// K in chunks of 16 staged in LDS, 256 threads with a 4 x 4 block each.  The problem type supplies
// the sizes (possibly read on the device: gathered token lists), the element loaders and the
// store; AK / BK say whether A / B are contiguous along k (then 16 neighbouring threads read 16
// consecutive k of one row), else along m / n.
template <class Prob, bool AK, bool BK>
__global__ void __launch_bounds__(256) tgemm_kernel(Prob pr, int splits, float* part, int64_t pstride) {
    __shared__ float As[16][68];
    __shared__ float Bs[16][68];
    typename Prob::Sub sp;
    const int sub = blockIdx.z / splits, piece = blockIdx.z % splits;
    if (!pr.begin(sub, sp)) return;
    const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
    if (m0 >= sp.M || n0 >= sp.N) return;
    // split-K: this work group sums k in [kb, ke) (16-aligned pieces)
    const int kc = ((sp.K + splits - 1) / splits + 15) & ~15;
    const int kb = piece * kc, ke = min(sp.K, kb + kc);
    const int tid = threadIdx.x, tm = tid >> 4, tn = tid & 15;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
    for (int k0 = kb; k0 < ke; k0 += 16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = tid + 256 * q;
            const int m = AK ? i >> 4 : i & 63, kk = AK ? i & 15 : i >> 6;
            As[kk][m] = (m0 + m < sp.M && k0 + kk < ke) ? pr.lda(sp, m0 + m, k0 + kk) : 0.f;
            const int n = BK ? i >> 4 : i & 63, kq = BK ? i & 15 : i >> 6;
            Bs[kq][n] = (n0 + n < sp.N && k0 + kq < ke) ? pr.ldb(sp, k0 + kq, n0 + n) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            const f32x4_t av = *reinterpret_cast<const f32x4_t*>(&As[kk][tm * 4]);
            const f32x4_t bv = *reinterpret_cast<const f32x4_t*>(&Bs[kk][tn * 4]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] += av[i] * bv[j];
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + tm * 4 + i, n = n0 + tn * 4 + j;
            if (m >= sp.M || n >= sp.N) continue;
            if (splits == 1) pr.store(sp, m, n, acc[i][j]);
            else part[(int64_t)blockIdx.z * pstride + (int64_t)m * sp.N + n] = acc[i][j];
        }
}

// split-K: the pieces of every element added in piece order (deterministic), then stored
template <class Prob>
__global__ void __launch_bounds__(256) tgemm_reduce_kernel(Prob pr, int splits, const float* part, int64_t pstride) {
    typename Prob::Sub sp;
    const int sub = blockIdx.y;
    if (!pr.begin(sub, sp)) return;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)sp.M * sp.N) return;
    float v = 0.f;
    for (int p = 0; p < splits; ++p) v += part[((int64_t)sub * splits + p) * pstride + e];
    pr.store(sp, (int)(e / sp.N), (int)(e % sp.N), v);
}


// The same sub-problems on matrix cores (bf16 layers): operands rounded once to bf16 as they are
// staged (rows k-contiguous in LDS for both A and B), 16x16x16 products into float32 accumulators,
// wave w owning the 32 x 32 quarter (w / 2, w % 2) of the 64 x 64 tile.
template <class Prob, bool AK, bool BK>
__global__ void __launch_bounds__(256) tgemm_mfma_kernel(Prob pr, int splits, float* part, int64_t pstride) {
    // k chunk: 32 for operands contiguous along k (one 16-byte vector per thread and operand), 64
    // for operands contiguous along m and n (two tokens of eight rows per thread).  LDS row pitch
    // 40 / 72 bf16 (80 / 144 bytes): the 8-byte fragment reads of 16 rows x 2 k-quads hit distinct
    // banks.
    static_assert(AK == BK, "both operands contiguous along k, or neither");
    constexpr int KC = AK ? 32 : 64, KP = AK ? 40 : 72, NQ = KC / 32;
    __shared__ __align__(16) uint16_t As[64 * KP];  // [m][k]
    __shared__ __align__(16) uint16_t Bs[64 * KP];  // [n][k]
    typename Prob::Sub sp;
    const int sub = blockIdx.z / splits, piece = blockIdx.z % splits;
    if (!pr.begin(sub, sp)) return;
    const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
    if (m0 >= sp.M || n0 >= sp.N) return;
    const int kc = ((sp.K + splits - 1) / splits + KC - 1) / KC * KC;
    const int kb = piece * kc, ke = min(sp.K, kb + kc);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, j4 = lane >> 4;
    const int wm = (w >> 1) * 32, wn = (w & 1) * 32;
    f32x4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int k0 = kb; k0 < ke; k0 += KC) {
        // 64 x KC of A and of B.  Operands contiguous along k: eight neighbouring k of one row per
        // load, one 16-byte LDS store.  Operands contiguous along m (n): eight neighbouring m of
        // four neighbouring k per thread, regrouped in registers into eight 8-byte LDS stores of
        // four k each.  Vector loads where the problem offers them for the whole run, else
        // element by element (ragged edges).
        if (AK) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                float v[8];
                const int idx = tid + 256 * q, m = idx / (KC / 8), ka = (idx % (KC / 8)) * 8;
                const bool in = m0 + m < sp.M;
                if (!(in && k0 + ka + 8 <= ke && pr.lda8(sp, m0 + m, k0 + ka, v)))
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = (in && k0 + ka + e < ke) ? pr.lda(sp, m0 + m, k0 + ka + e) : 0.f;
                *reinterpret_cast<u32x4_t*>(&As[m * KP + ka]) = pack8(v);
            }
        } else {
            float v[2][8];
            const int kq = (tid >> 3) * 2, m8 = (tid & 7) * 8;
#pragma unroll
            for (int z = 0; z < 2; ++z) {
                const bool in = k0 + kq + z < ke;
                if (!(in && m0 + m8 + 8 <= sp.M && pr.lda8(sp, m0 + m8, k0 + kq + z, v[z])))
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        v[z][e] = (in && m0 + m8 + e < sp.M) ? pr.lda(sp, m0 + m8 + e, k0 + kq + z) : 0.f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e)
                *reinterpret_cast<uint32_t*>(&As[(m8 + e) * KP + kq]) = pack_bf16x2(v[0][e], v[1][e]);
        }
        if (BK) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                float v[8];
                const int idx = tid + 256 * q, n = idx / (KC / 8), kq = (idx % (KC / 8)) * 8;
                const bool in = n0 + n < sp.N;
                if (!(in && k0 + kq + 8 <= ke && pr.ldb8(sp, k0 + kq, n0 + n, v)))
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = (in && k0 + kq + e < ke) ? pr.ldb(sp, k0 + kq + e, n0 + n) : 0.f;
                *reinterpret_cast<u32x4_t*>(&Bs[n * KP + kq]) = pack8(v);
            }
        } else {
            float v[2][8];
            const int kq = (tid >> 3) * 2, n8 = (tid & 7) * 8;
#pragma unroll
            for (int z = 0; z < 2; ++z) {
                const bool in = k0 + kq + z < ke;
                if (!(in && n0 + n8 + 8 <= sp.N && pr.ldb8(sp, k0 + kq + z, n0 + n8, v[z])))
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        v[z][e] = (in && n0 + n8 + e < sp.N) ? pr.ldb(sp, k0 + kq + z, n0 + n8 + e) : 0.f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e)
                *reinterpret_cast<uint32_t*>(&Bs[(n8 + e) * KP + kq]) = pack_bf16x2(v[0][e], v[1][e]);
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < KC; ks += 16) {
            s16x4_t af[2], bq[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                af[t] = lds8(&As[(wm + 16 * t + l16) * KP + ks + 4 * j4]);
                bq[t] = lds8(&Bs[(wn + 16 * t + l16) * KP + ks + 4 * j4]);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mma16(af[i], bq[j], acc[i][j]);
        }
        __syncthreads();
    }
    // C layout: lane column n = l16 of each 16 x 16 block, rows 4 j4 .. 4 j4 + 3
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm + 16 * i + 4 * j4 + r, n = n0 + wn + 16 * j + l16;
                if (m >= sp.M || n >= sp.N) continue;
                if (splits == 1) pr.store(sp, m, n, acc[i][j][r]);
                else part[(int64_t)blockIdx.z * pstride + (int64_t)m * sp.N + n] = acc[i][j][r];
            }
}

// Token lists of the routed experts (global bucketing of the forward's routing): the m-th token of
// expert e is perm[offs[e] + m]; its rank r is where e sits in idx[t][g].
struct Lists {
    const int32_t* offs;  // [N + 1]
    const int32_t* perm;  // [T G k]: token of every list position
    const int32_t* rank;  // [T G k]: choice rank of every list position
};

// rank of every list position, from the inverse map of the bucketing: thread per (t, g, r)
__global__ void list_rank_kernel(const int32_t* __restrict__ inv, int64_t n, int k, int32_t* __restrict__ rank) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q < n) rank[inv[q]] = (int)(q % k);
}

// U[t][slot] = dy_t W_slot^T: sub-problem = slot matrix (expert e, group slot g, shared head);
// M = its tokens, N = d_h, K = d.
template <typename T>
struct ProbU {
    BwdArgs a;
    Lists L;
    struct Sub {
        int M, N, K, kind, e, g, base;
    };
    __device__ bool begin(int z, Sub& s) const {
        const bool rslot = !a.dense && a.variant == GQE_VARIANT_GQE;
        s.N = a.dh;
        s.K = a.d;
        s.e = s.g = s.base = 0;
        if (z < a.N) {
            s.kind = 0;
            s.e = z;
            s.g = z / a.n;
            if (a.dense) {
                s.M = (int)a.T;
            } else {
                s.base = L.offs[z];
                s.M = L.offs[z + 1] - s.base;
            }
        } else if (rslot && z < a.N + a.G) {
            s.kind = 1;
            s.g = z - a.N;
            s.M = (int)a.T;
        } else {
            s.kind = 2;
            s.M = (int)a.T;
        }
        return s.M > 0;
    }
    __device__ int64_t tok(const Sub& s, int m) const { return (s.kind == 0 && !a.dense) ? L.perm[s.base + m] : m; }
    __device__ float lda(const Sub& s, int m, int k) const { return ld<T>(a.dy, tok(s, m) * a.d + k); }
    __device__ const T* wslot(const Sub& s) const {
        return s.kind == 0 ? (const T*)a.wo + (int64_t)s.e * a.dh * a.d
                           : (s.kind == 1 ? (const T*)a.wor + (int64_t)s.g * a.dh * a.d : (const T*)a.wos);
    }
    __device__ float ldb(const Sub& s, int k, int n) const { return to_f32(wslot(s)[(int64_t)n * a.d + k]); }
    // k .. k + 7 (8-aligned; rows aligned when d % 8 == 0)
    __device__ bool lda8(const Sub& s, int m, int k, float (&v)[8]) const {
        if (a.d & 7) return false;
        ld8<T>(a.dy, tok(s, m) * a.d + k, v);
        return true;
    }
    __device__ bool ldb8(const Sub& s, int k, int n, float (&v)[8]) const {
        if (a.d & 7) return false;
        ld8<T>(wslot(s), (int64_t)n * a.d + k, v);
        return true;
    }
    __device__ void store(const Sub& s, int m, int n, float v) const {
        const int64_t t = tok(s, m);
        const bool rslot = !a.dense && a.variant == GQE_VARIANT_GQE;
        int ls;
        if (s.kind == 0) ls = s.g * a.k + (a.dense ? s.e % a.n : L.rank[s.base + m]);
        else if (s.kind == 1) ls = a.G * a.k + s.g;
        else ls = a.G * a.k + (rslot ? a.G : 0);
        a.U[(t * a.NS + ls) * a.dh + n] = v;
    }
};

// weight gradients of the output slots: dW[j][c] = sum_t v_t[j] dy_t[c]; M = d_h, N = d, K = tokens
template <typename T>
struct ProbWo {
    BwdArgs a;
    Lists L;
    typedef typename ProbU<T>::Sub Sub;
    __device__ bool begin(int z, Sub& s) const {
        ProbU<T> u{a, L};
        if (!u.begin(z, s)) {
            // no token: the gradient block is zero
            s.K = 0;
            s.M = a.dh;
            s.N = a.d;
            return true;
        }
        s.K = s.M;
        s.M = a.dh;
        s.N = a.d;
        return true;
    }
    __device__ int64_t tok(const Sub& s, int k) const { return (s.kind == 0 && !a.dense) ? L.perm[s.base + k] : k; }
    __device__ float lda(const Sub& s, int j, int k) const {
        const int64_t t = tok(s, k);
        const int64_t ob = t * a.H * a.dh;  // O is token-major
        if (s.kind == 0) {
            const int h = s.g * a.k + (a.dense ? s.e % a.n : L.rank[s.base + k]);
            return a.cf[t * a.H + h] * ld<T>(a.O, ob + h * a.dh + j);
        }
        if (s.kind == 1) {
            float v = 0.f;
            for (int r = 0; r < a.k; ++r) {
                const int h = s.g * a.k + r;
                v += a.wn[t * a.H + h] * ld<T>(a.O, ob + h * a.dh + j);
            }
            return v;
        }
        return ld<T>(a.O, ob + a.G * a.k * a.dh + j);
    }
    __device__ float ldb(const Sub& s, int k, int n) const { return ld<T>(a.dy, tok(s, k) * a.d + n); }
    // j .. j + 7 of token k (d_h is a multiple of 16)
    __device__ bool lda8(const Sub& s, int j, int k, float (&v)[8]) const {
        const int64_t t = tok(s, k);
        const int64_t ob = t * a.H * a.dh;
        if (s.kind == 0) {
            const int h = s.g * a.k + (a.dense ? s.e % a.n : L.rank[s.base + k]);
            ld8<T>(a.O, ob + h * a.dh + j, v);
            const float c = a.cf[t * a.H + h];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] *= c;
        } else if (s.kind == 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = 0.f;
            for (int r = 0; r < a.k; ++r) {
                const int h = s.g * a.k + r;
                float o[8];
                ld8<T>(a.O, ob + h * a.dh + j, o);
                const float c = a.wn[t * a.H + h];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] += c * o[e];
            }
        } else {
            ld8<T>(a.O, ob + a.G * a.k * a.dh + j, v);
        }
        return true;
    }
    __device__ bool ldb8(const Sub& s, int k, int n, float (&v)[8]) const {
        if (a.d & 7) return false;
        ld8<T>(a.dy, tok(s, k) * a.d + n, v);
        return true;
    }
    __device__ void store(const Sub& s, int m, int n, float v) const {
        const int per = a.dh * a.d;
        float* dst = s.kind == 0 ? a.dwo + (int64_t)s.e * per : (s.kind == 1 ? a.dwor + (int64_t)s.g * per : a.dwos);
        dst[(int64_t)m * a.d + n] = v;
    }
};

// input-side weight gradients dW[i][j] = sum_t x_t[i] g_t[j]: sub-problem = head block (K_g, V_g,
// shared query, expert e); M = d, N = d_h, K = tokens
template <typename T>
struct ProbWx {
    BwdArgs a;
    Lists L;
    struct Sub {
        int M, N, K, hb, e, g, base;
    };
    __device__ bool begin(int z, Sub& s) const {
        const int ebase = 2 * a.G + a.s;
        s.hb = z;
        s.M = a.d;
        s.N = a.dh;
        s.K = (int)a.T;
        s.e = s.g = s.base = 0;
        if (z >= ebase) {
            s.e = z - ebase;
            s.g = s.e / a.n;
            if (!a.dense) {
                s.base = L.offs[s.e];
                s.K = L.offs[s.e + 1] - s.base;
            }
        }
        return true;
    }
    __device__ int64_t tok(const Sub& s, int k) const {
        return (s.hb >= 2 * a.G + a.s && !a.dense) ? L.perm[s.base + k] : k;
    }
    __device__ float lda(const Sub& s, int i, int k) const { return ld<T>(a.x, tok(s, k) * a.d + i); }
    __device__ bool lda8(const Sub& s, int i, int k, float (&v)[8]) const {
        if (a.d & 7) return false;
        ld8<T>(a.x, tok(s, k) * a.d + i, v);
        return true;
    }
    // the gradient row of token list entry k: buffer and element offset
    __device__ const void* grow(const Sub& s, int k, int64_t& off) const {
        const int ebase = 2 * a.G + a.s;
        const int64_t t = tok(s, k);
        if (s.hb < a.G) {
            off = (t * a.G + s.hb) * a.dh;
            return a.dK;
        }
        if (s.hb < 2 * a.G) {
            off = (t * a.G + s.hb - a.G) * a.dh;
            return a.dV;
        }
        if (s.hb < ebase) {
            off = (t * a.H + a.G * a.k) * a.dh;
            return a.dQ;
        }
        const int h = s.g * a.k + (a.dense ? s.e % a.n : L.rank[s.base + k]);
        off = (t * a.H + h) * a.dh;
        return a.dQ;
    }
    __device__ bool ldb8(const Sub& s, int k, int j, float (&v)[8]) const {
        int64_t off;
        const void* p = grow(s, k, off);
        gread8<T>(p, off + j, v);
        return true;
    }
    __device__ float ldb(const Sub& s, int k, int j) const {
        int64_t off;
        const void* p = grow(s, k, off);
        return gread<T>(p, off + j);
    }
    __device__ void store(const Sub& s, int i, int j, float v) const {
        const int ebase = 2 * a.G + a.s;
        if (s.hb < a.G) a.dwk[(int64_t)i * a.G * a.dh + s.hb * a.dh + j] = v;
        else if (s.hb < 2 * a.G) a.dwv[(int64_t)i * a.G * a.dh + (s.hb - a.G) * a.dh + j] = v;
        else if (s.hb < ebase) a.dwqs[(int64_t)i * a.dh + j] = v;
        else a.dwq[((int64_t)s.e * a.d + i) * a.dh + j] = v;
    }
};

// dx, dense part: K = [dK (G d_h) | dV (G d_h) | shared dq (d_h)] written (which = 0), then the
// router logits' part, K = N, added (which = 1).  With `expand` the which = 0 product also takes
// the routed query heads as N more d_h-wide segments, one per expert: a token's segment holds its
// dq for that expert where it chose it and zeros elsewhere (n / k times the routed work, in one
// pass over dx instead of one read-modify-write per (group, rank)).
template <typename T>
struct ProbDxDense {
    BwdArgs a;
    int which;
    int expand;
    struct Sub {
        int M, N, K;
    };
    __device__ int kd() const { return 2 * a.G * a.dh + a.s * a.dh; }
    __device__ bool begin(int, Sub& s) const {
        s.M = (int)a.T;
        s.N = a.d;
        s.K = which ? (a.dense ? 0 : a.N) : kd() + (expand ? a.N * a.dh : 0);
        return s.K > 0;
    }
    // routed segment element kk' = e d_h + j: the head of token t that chose expert e, or -1
    __device__ int routed_head(int t, int e) const {
        const int g = e / a.n;
        if (a.dense) return g * a.k + e % a.n;
        const int32_t* id = a.idx + ((int64_t)t * a.G + g) * a.k;
        for (int r = 0; r < a.k; ++r)
            if (id[r] == e) return g * a.k + r;
        return -1;
    }
    __device__ float lda(const Sub&, int t, int kk) const {
        if (!which && kk >= kd()) {
            const int e = (kk - kd()) / a.dh, j = (kk - kd()) % a.dh;
            const int h = routed_head(t, e);
            return h < 0 ? 0.f : gread<T>(a.dQ, ((int64_t)t * a.H + h) * a.dh + j);
        }
        if (which) kk += kd();
        const int GD = a.G * a.dh;
        if (kk < GD) return gread<T>(a.dK, (int64_t)t * GD + kk);
        if (kk < 2 * GD) return gread<T>(a.dV, (int64_t)t * GD + kk - GD);
        kk -= 2 * GD;
        if (a.s && kk < a.dh) return gread<T>(a.dQ, ((int64_t)t * a.H + a.G * a.k) * a.dh + kk);
        kk -= a.s * a.dh;
        return a.dl[(int64_t)t * a.N + kk];
    }
    __device__ float ldb(const Sub&, int kk, int i) const {
        if (!which && kk >= kd()) {
            const int e = (kk - kd()) / a.dh, j = (kk - kd()) % a.dh;
            return ld<T>(a.wq, ((int64_t)e * a.d + i) * a.dh + j);
        }
        if (which) kk += kd();
        const int GD = a.G * a.dh;
        if (kk < GD) return ld<T>(a.wk, (int64_t)i * GD + kk);
        if (kk < 2 * GD) return ld<T>(a.wv, (int64_t)i * GD + kk - GD);
        kk -= 2 * GD;
        if (a.s && kk < a.dh) return ld<T>(a.wqs, (int64_t)i * a.dh + kk);
        kk -= a.s * a.dh;
        return a.wr[(int64_t)i * a.N + kk];
    }
    // kk .. kk + 7 inside one segment (segment lengths G d_h, d_h are multiples of 16)
    __device__ bool lda8(const Sub&, int t, int kk, float (&v)[8]) const {
        if (which) return false;
        const int GD = a.G * a.dh;
        if (kk >= kd()) {
            const int e = (kk - kd()) / a.dh, j = (kk - kd()) % a.dh;
            const int h = routed_head(t, e);
            if (h < 0) {
#pragma unroll
                for (int z = 0; z < 8; ++z) v[z] = 0.f;
            } else {
                gread8<T>(a.dQ, ((int64_t)t * a.H + h) * a.dh + j, v);
            }
            return true;
        }
        if (kk < GD) gread8<T>(a.dK, (int64_t)t * GD + kk, v);
        else if (kk < 2 * GD) gread8<T>(a.dV, (int64_t)t * GD + kk - GD, v);
        else gread8<T>(a.dQ, ((int64_t)t * a.H + a.G * a.k) * a.dh + kk - 2 * GD, v);
        return true;
    }
    __device__ bool ldb8(const Sub&, int kk, int i, float (&v)[8]) const {
        if (which) return false;
        const int GD = a.G * a.dh;
        if (kk >= kd()) {
            const int e = (kk - kd()) / a.dh, j = (kk - kd()) % a.dh;
            ld8<T>(a.wq, ((int64_t)e * a.d + i) * a.dh + j, v);
            return true;
        }
        if (kk < GD) ld8<T>(a.wk, (int64_t)i * GD + kk, v);
        else if (kk < 2 * GD) ld8<T>(a.wv, (int64_t)i * GD + kk - GD, v);
        else ld8<T>(a.wqs, (int64_t)i * a.dh + kk - 2 * GD, v);
        return true;
    }
    __device__ void store(const Sub&, int t, int i, float v) const {
        if (which) a.dx[(int64_t)t * a.d + i] += v;
        else a.dx[(int64_t)t * a.d + i] = v;
    }
};

// dx, routed part (added): one launch per (group g, choice rank r), sub-problem = expert e of the
// group; M = its tokens (those whose rank-r choice is another expert load zeros and store nothing),
// N = d, K = d_h.  Inside one launch every token has exactly one such expert, so the adds never
// collide; the launches follow each other on the stream.
template <typename T>
struct ProbDxRouted {
    BwdArgs a;
    Lists L;
    int g, r;
    struct Sub {
        int M, N, K, e, base;
    };
    __device__ bool begin(int z, Sub& s) const {
        s.e = g * a.n + z;
        s.N = a.d;
        s.K = a.dh;
        if (a.dense) {
            s.base = 0;
            s.M = (z == r) ? (int)a.T : 0;
        } else {
            s.base = L.offs[s.e];
            s.M = L.offs[s.e + 1] - s.base;
        }
        return s.M > 0;
    }
    __device__ int64_t tok(const Sub& s, int m) const { return a.dense ? m : L.perm[s.base + m]; }
    __device__ bool mine(const Sub& s, int m) const { return a.dense || L.rank[s.base + m] == r; }
    __device__ float lda(const Sub& s, int m, int j) const {
        const int64_t t = tok(s, m);
        if (!mine(s, m)) return 0.f;
        return gread<T>(a.dQ, (t * a.H + g * a.k + r) * a.dh + j);
    }
    __device__ float ldb(const Sub& s, int j, int i) const { return ld<T>(a.wq, ((int64_t)s.e * a.d + i) * a.dh + j); }
    __device__ bool lda8(const Sub& s, int m, int j, float (&v)[8]) const {
        if (!mine(s, m)) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = 0.f;
        } else {
            gread8<T>(a.dQ, (tok(s, m) * a.H + g * a.k + r) * a.dh + j, v);
        }
        return true;
    }
    __device__ bool ldb8(const Sub& s, int j, int i, float (&v)[8]) const {
        ld8<T>(a.wq, ((int64_t)s.e * a.d + i) * a.dh + j, v);
        return true;
    }
    __device__ void store(const Sub& s, int m, int i, float v) const {
        if (mine(s, m)) a.dx[tok(s, m) * a.d + i] += v;
    }
};

// Router weight and bias gradients, dW_r[i][e] = sum_t x_t[i] dl_t[e] and db_r[e] = sum_t dl_t[e]
// (row i = d, where x counts as 1), in float32: work group = (256 rows i, 16 experts, token chunk);
// the chunk's logit gradients pass through LDS 128 tokens at a time and every lane reads them as
// a broadcast; per-chunk partial sums ([chunk][expert][row]: neighbouring lanes store neighbouring
// rows) are added in chunk order.
constexpr int kRgTok = 128;
template <typename T>
__global__ void __launch_bounds__(256) bwd_router_wgrad_kernel(BwdArgs a, int nchunk, float* __restrict__ part) {
    __shared__ __align__(16) float dls[kRgTok][16];
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int e0 = blockIdx.y * 16, ne = min(16, a.N - e0);
    const int c = blockIdx.z;
    const int64_t per = ceil_div(a.T, nchunk);
    const int64_t t0 = (int64_t)c * per, t1 = min(a.T, t0 + per);
    float acc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.f;
    for (int64_t tb = t0; tb < t1; tb += kRgTok) {
        __syncthreads();
        for (int q = threadIdx.x; q < kRgTok * 16; q += 256) {
            const int tt = q >> 4, e = q & 15;
            const int64_t t = tb + tt;
            dls[tt][e] = (t < t1 && e < ne) ? a.dl[t * a.N + e0 + e] : 0.f;
        }
        __syncthreads();
        const int nt = (int)min<int64_t>(kRgTok, t1 - tb);
        if (i <= a.d)
            for (int t8 = 0; t8 < nt; t8 += 8) {
                // eight tokens' x loads in flight together (tokens past the chunk count as 0)
                float xv[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    xv[u] = t8 + u < nt ? (i < a.d ? ld<T>(a.x, (tb + t8 + u) * a.d + i) : 1.f) : 0.f;
#pragma unroll
                for (int u = 0; u < 8; ++u)
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4) {
                        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(&dls[t8 + u][4 * e4]);
#pragma unroll
                        for (int z = 0; z < 4; ++z) acc[4 * e4 + z] += xv[u] * v[z];
                    }
            }
    }
    if (i <= a.d)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            if (e < ne) part[((int64_t)c * a.N + e0 + e) * (a.d + 1) + i] = acc[e];
}

// eight lanes per output element, each adding every eighth chunk in chunk order, then the eight
// partial sums added in lane order (a fixed order: the result does not depend on the schedule)
__global__ void bwd_router_wgrad_reduce(BwdArgs a, int nchunk, const float* __restrict__ part) {
    const int64_t q = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 3;  // e (d + 1) + i
    const int sl = threadIdx.x & 7;
    const int64_t n = (int64_t)(a.d + 1) * a.N;
    float v = 0.f;
    if (q < n)
        for (int c = sl; c < nchunk; c += 8) v += part[(int64_t)c * n + q];
    // lanes 8 j .. 8 j + 7: add lane 0's partial first, then lanes 1 .. 7, in that order
    float tot = 0.f;
#pragma unroll
    for (int o = 0; o < 8; ++o) tot += __shfl(v, (threadIdx.x & ~7) + o);
    if (q >= n || sl != 0) return;
    const int e = (int)(q / (a.d + 1)), i = (int)(q % (a.d + 1));
    if (i < a.d) a.dwr[(int64_t)i * a.N + e] = tot;
    else a.dbr[e] = tot;
}

// ---------------------------------------------------------------- token-contracted products (bf16)
// C[m][n] = sum_t A[t][m] B[t][n] with A and B token-major (the weight gradients: x^T g and
// slot^T dy), for bf16 layers.  Work group = 128 x 128 tile of C and a range of tokens (ordered
// split-K); per 32 tokens the two 32 x 128 operand tiles go straight from global memory into LDS
// (global_load_lds_dwordx4, token rows as they are, 16-byte chunks XOR-swizzled by the row), three
// stages deep.  The matrix core wants eight consecutive tokens per lane for one column, which
// ds_read_b64_tr_b16 delivers from the token-major tile: within 16 lanes, lane i receives halfword
// i % 4 of the 8-byte pieces addressed by lanes i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4, so
// lane j addressing row kk + j / 4, column c0 + 4 (j % 4) hands lane i the four tokens kk .. kk + 3
// of column c0 + i.  Four waves, each a 64 x 64 quarter in 16 x 16 blocks, v_mfma_f32_16x16x32_bf16.
struct WgJob {
    const uint16_t* A;  // [T][lda], columns [0, M) used
    const uint16_t* B;  // [T][ldb], columns [0, N) used
    int lda, ldb, M, N;
    int tiles_n, tile0;  // 128-column tiles of N; first tile of the job in the launch
    int64_t part;        // float offset of the job's partial sums [split][M][N]
    float* dst;          // reduce: destination
    int mode;            // 0: dst[m N + n]; 1: dst[((n / dh) M + m) dh + n % dh] (per-expert blocks)
};
constexpr int kWgMaxJobs = 4;
struct WgArgs {
    WgJob job[kWgMaxJobs];
    int njobs, ntiles;
    int64_t T;
    int splits, kc;  // token range per split (a multiple of 32)
    int dh;
    float* part;
};

__device__ __forceinline__ int wg_swz(int r) { return 2 * (r & 3) + 8 * ((r >> 3) & 1); }

__global__ void __launch_bounds__(256) wg_gemm_kernel(WgArgs a) {
    constexpr int BM = 128, BN = 128, KC = 32, NST = 3;
    __shared__ __align__(1024) uint16_t As[NST][KC * BM];
    __shared__ __align__(1024) uint16_t Bs[NST][KC * BN];
    int t = blockIdx.x, jn = 0;
    for (int q = 1; q < a.njobs; ++q)
        if (t >= a.job[q].tile0) jn = q;
    const WgJob& J = a.job[jn];
    t -= J.tile0;
    const int m0 = (t / J.tiles_n) * BM, n0 = (t % J.tiles_n) * BN;
    const int piece = blockIdx.y;
    const int64_t kb = (int64_t)piece * a.kc, ke = min(a.T, kb + a.kc);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // LDS destinations of the loads are scalar
    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (kb < ke) {
        // loads: wave w fills 1 KB segments w and w + 4 of each operand tile (4 token rows each);
        // lane: row 4 seg + lane / 16, LDS chunk lane % 16 holding global chunk (lane % 16) ^ swz(row);
        // columns past M (N) read column 0 of the row, tokens past the range read the range's last
        int aoff[2], boff[2], rowv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int seg = w + 4 * h, r = 4 * seg + (lane >> 4), c = (lane & 15) ^ wg_swz(r);
            rowv[h] = r;
            aoff[h] = (m0 + 8 * c < J.M) ? m0 + 8 * c : 0;
            boff[h] = (n0 + 8 * c < J.N) ? n0 + 8 * c : 0;
        }
        auto issue = [&](int64_t k0, int stage) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t tok = min(k0 + rowv[h], ke - 1);
                dma16(J.A + tok * J.lda + aoff[h], &As[stage][(w + 4 * h) * 512]);
                dma16(J.B + tok * J.ldb + boff[h], &Bs[stage][(w + 4 * h) * 512]);
            }
        };
        const int nchunk = (int)((ke - kb + KC - 1) / KC);
        issue(kb, 0);
        if (nchunk > 1) issue(kb + KC, 1);
        // fragment addresses (element offsets in a stage): lane j of its 16-lane group addresses
        // token row 8 q + 4 h + j / 4 (q = lane / 16, h = read), column base + 4 (j % 4)
        const int q = lane >> 4, gi = lane & 15;
        const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
        auto faddr = [&](int col0, int h) {
            const int r = 8 * q + 4 * h + (gi >> 2);
            const int col = col0 + 4 * (gi & 3);
            return r * 128 + 8 * ((col >> 3) ^ wg_swz(r)) + (col & 7);
        };
        typedef __attribute__((address_space(3))) s16x4_t* lds_s4;
        for (int c = 0; c < nchunk; ++c) {
            const int stage = c % NST;
            if (c + 2 < nchunk) {
                issue(kb + (int64_t)(c + 2) * KC, (c + 2) % NST);
                __builtin_amdgcn_s_waitcnt(vmcnt_wait(8));   // chunk c landed, c + 1 and c + 2 in flight
            } else if (c + 1 < nchunk) {
                __builtin_amdgcn_s_waitcnt(vmcnt_wait(4));
            } else {
                __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
            }
            __syncthreads();
            bf16x8_t af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(&As[stage][faddr(wm + 16 * i, 0)]));
                const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(&As[stage][faddr(wm + 16 * i, 1)]));
                af[i] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                const s16x4_t lb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(&Bs[stage][faddr(wn + 16 * i, 0)]));
                const s16x4_t hb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(&Bs[stage][faddr(wn + 16 * i, 1)]));
                bfr[i] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lb, hb, 0, 1, 2, 3, 4, 5, 6, 7));
            }
            const int64_t k0 = kb + (int64_t)c * KC;
            if (k0 + KC > ke) {
                // the range's last, partial chunk: tokens past its end (rows re-read from the last
                // token) contribute nothing
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (k0 + 8 * q + e >= ke) bfr[i][e] = (__bf16)0.0f;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
            __syncthreads();  // the stage is free for the load three chunks on
        }
    }
    // C layout: lane holds rows 4 (lane / 16) + 0..3 of each 16 x 16 block, column lane % 16
    float* pp = a.part + J.part + (int64_t)piece * J.M * J.N;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + ((w >> 1) * 64) + 16 * i + 4 * (lane >> 4) + r;
                const int n = n0 + ((w & 1) * 64) + 16 * j + (lane & 15);
                if (m < J.M && n < J.N) pp[(int64_t)m * J.N + n] = acc[i][j][r];
            }
}

// The split-K pieces of every element added in piece order, then stored (blockIdx.y = job).
__global__ void __launch_bounds__(256) wg_reduce_kernel(WgArgs a) {
    const WgJob& J = a.job[blockIdx.y];
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t MN = (int64_t)J.M * J.N;
    if (e >= MN) return;
    float v = 0.f;
    for (int p = 0; p < a.splits; ++p) v += a.part[J.part + p * MN + e];
    const int m = (int)(e / J.N), n = (int)(e % J.N);
    if (J.mode == 0) J.dst[e] = v;
    else J.dst[((int64_t)(n / a.dh) * J.M + m) * a.dh + n % a.dh] = v;
}

// Token-major bf16 operands of the weight and input gradients, with the routed experts
// zero-expanded (an expert's block is zero where the token did not choose it).  gcat: [T][kp], the
// concatenated gradients [dK (G d_h) | dV (G d_h) | shared dq (s d_h) | routed dq per expert (N d_h) |
// zeros up to kp]; ocat: [T][N + nslot][d_h], the output-slot vectors: expert slots (coefficient times
// the head output where chosen), the renormalised group slots (sum_r w_r o_r), the shared head's
// output.  Thread = (token, eight columns).
template <typename T>
__global__ void __launch_bounds__(256) wg_expand_kernel(BwdArgs a, uint16_t* __restrict__ gcat, int kp,
                                                        uint16_t* __restrict__ ocat, int nslot) {
    // work group: four tokens (blockIdx.y) x 64 consecutive 16-byte chunks of their rows (blockIdx.x)
    const int ng = kp / 8, no = (a.N + nslot) * a.dh / 8;
    const int64_t t = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6);
    const int u = (int)blockIdx.x * 64 + (int)(threadIdx.x & 63);
    if (t >= a.T || u >= ng + no) return;
    const uint16_t* dQ = reinterpret_cast<const uint16_t*>(a.dQ);
    const int GD = a.G * a.dh, kd = 2 * GD + a.s * a.dh;
    // the head of token t that chose expert e (all-active GQA: head e % n of its group), or -1
    auto routed_head = [&](int e) {
        const int g = e / a.n;
        if (a.dense) return g * a.k + e % a.n;
        const int32_t* id = a.idx + (t * a.G + g) * a.k;
        int h = -1;
        for (int r = 0; r < a.k; ++r)
            if (id[r] == e) h = g * a.k + r;
        return h;
    };
    if (u < ng) {
        const int c = 8 * u;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (c < GD) v = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(a.dK) + t * GD + c);
        else if (c < 2 * GD) v = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(a.dV) + t * GD + c - GD);
        else if (c < kd) v = *reinterpret_cast<const u32x4_t*>(dQ + (t * a.H + a.G * a.k) * a.dh + c - 2 * GD);
        else if (c < kd + a.N * a.dh) {
            const int e = (c - kd) / a.dh, j = (c - kd) % a.dh;
            const int h = routed_head(e);
            if (h >= 0) v = *reinterpret_cast<const u32x4_t*>(dQ + (t * a.H + h) * a.dh + j);
        }
        *reinterpret_cast<u32x4_t*>(gcat + t * kp + c) = v;
        return;
    }
    const int c = 8 * (u - ng);
    const int blk = c / a.dh, j = c % a.dh;
    float o[8];
    if (blk < a.N) {
        const int h = routed_head(blk);
        if (h < 0) {
#pragma unroll
            for (int z = 0; z < 8; ++z) o[z] = 0.f;
        } else {
            ld8<bf16_t>(a.O, (t * a.H + h) * a.dh + j, o);
            const float cf = a.cf[t * a.H + h];
#pragma unroll
            for (int z = 0; z < 8; ++z) o[z] *= cf;
        }
    } else if (blk - a.N < nslot - a.s) {
        const int g = blk - a.N;
#pragma unroll
        for (int z = 0; z < 8; ++z) o[z] = 0.f;
        for (int r = 0; r < a.k; ++r) {
            const int h = g * a.k + r;
            float v[8];
            ld8<bf16_t>(a.O, (t * a.H + h) * a.dh + j, v);
            const float w = a.wn[t * a.H + h];
#pragma unroll
            for (int z = 0; z < 8; ++z) o[z] += w * v[z];
        }
    } else {
        ld8<bf16_t>(a.O, (t * a.H + a.G * a.k) * a.dh + j, o);
    }
    *reinterpret_cast<u32x4_t*>(ocat + t * (a.N + nslot) * a.dh + c) = pack8(o);
}

// The input-side weights transposed to match gcat: wcat[i][kk] = the weight that multiplies gcat
// column kk in dx[t][i] (W_k, W_v, W_qs, then W_q of every expert; zeros up to kp).  Thread = (i,
// eight columns).
__global__ void __launch_bounds__(256) wg_wcat_kernel(BwdArgs a, uint16_t* __restrict__ wcat, int kp) {
    const int ng = kp / 8;
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= (int64_t)a.d * ng) return;
    const int i = (int)(q / ng), c = 8 * (int)(q % ng);
    const int GD = a.G * a.dh, kd = 2 * GD + a.s * a.dh;
    const uint16_t* src = nullptr;
    if (c < GD) src = reinterpret_cast<const uint16_t*>(a.wk) + (int64_t)i * GD + c;
    else if (c < 2 * GD) src = reinterpret_cast<const uint16_t*>(a.wv) + (int64_t)i * GD + c - GD;
    else if (c < kd) src = reinterpret_cast<const uint16_t*>(a.wqs) + (int64_t)i * a.dh + c - 2 * GD;
    else if (c < kd + a.N * a.dh) {
        const int e = (c - kd) / a.dh, j = (c - kd) % a.dh;
        src = reinterpret_cast<const uint16_t*>(a.wq) + ((int64_t)e * a.d + i) * a.dh + j;
    }
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (src) {
        // two 8-byte halves (the weights are only assumed 8-byte aligned, as by ld8)
        const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(src), hi = *reinterpret_cast<const u32x2_t*>(src + 4);
        v = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    }
    *reinterpret_cast<u32x4_t*>(wcat + (int64_t)i * kp + c) = v;
}

// The output-slot weights as one [NS d_h][d] matrix: W_o of every expert, W_oR of every group (when
// the renormalised slot exists), W_os.  Thread = (row, eight columns).
__global__ void __launch_bounds__(256) wg_wslot_kernel(BwdArgs a, uint16_t* __restrict__ wsl) {
    const int ng = a.d / 8;
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= (int64_t)a.NS * a.dh * ng) return;
    const int row = (int)(q / ng), c = 8 * (int)(q % ng);
    const int ro = a.N * a.dh, rg = (a.NS - a.N - a.s) * a.dh;
    const uint16_t* src;
    if (row < ro) src = reinterpret_cast<const uint16_t*>(a.wo) + (int64_t)row * a.d + c;
    else if (row < ro + rg) src = reinterpret_cast<const uint16_t*>(a.wor) + (int64_t)(row - ro) * a.d + c;
    else src = reinterpret_cast<const uint16_t*>(a.wos) + (int64_t)(row - ro - rg) * a.d + c;
    const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(src), hi = *reinterpret_cast<const u32x2_t*>(src + 4);
    *reinterpret_cast<u32x4_t*>(wsl + (int64_t)row * a.d + c) = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
}

// C = A B^T (+ dl W_r^T) in float32 for bf16 A [M][kp] and B [N][kp], both contiguous along the
// contraction (the U and dx products): 256 x (64 NB) tiles, eight waves of 128 x 16 NB in
// v_mfma_f32_16x16x32_bf16, the operand tiles copied straight into LDS in 64-wide slices
// (XOR-swizzled 16-byte chunks, two stages).  Against 128 x 128 tiles this re-reads each operand
// fewer times: these products are bound by their global -> LDS copies, not by the matrix cores.
// NB is chosen per product so that the tiles fill the CUs in the fewest rounds.  The router's term
// (float32 logit gradients and router weights, nr <= 64 columns; nr = 0: none) is added in the same
// accumulators by v_mfma_f32_16x16x4_f32 from float32 tiles staged in the freed LDS.
template <int NB>
__global__ void __launch_bounds__(512, 1) bt_gemm_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                       float* __restrict__ C, int64_t M, int N, int kp,
                                                       const float* __restrict__ dl, const float* __restrict__ wr,
                                                       int nr) {
    constexpr int BM = 256, BN = 64 * NB, KC = 64;
    constexpr int SA = BM * KC / 512, SB = BN * KC / 512;  // 1 KB segments per operand tile
    __shared__ __align__(1024) uint16_t As[2][BM * KC];
    __shared__ __align__(1024) uint16_t Bs[2][BN * KC];
    static_assert(SA % 8 == 0 && SB % 8 == 0, "whole segments per wave");
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tiles_n = (N + BN - 1) / BN;
    const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * BM;
    const int n0 = (int)(blockIdx.x % tiles_n) * BN;
    // segment s: rows 8 s .. 8 s + 7, eight chunks each; wave w takes segments w, w + 8, ...;
    // LDS chunk p of row r holds global chunk p ^ ((r >> 1) & 7); rows past the edge repeat the last
    uint32_t aoff[SA / 8], boff[SB / 8];
#pragma unroll
    for (int i = 0; i < SA / 8; ++i) {
        const int qq = (w + 8 * i) * 64 + lane;
        const int r = qq >> 3, c = (qq & 7) ^ ((r >> 1) & 7);
        const int64_t ra = min(m0 + r, M - 1) - m0;
        aoff[i] = (uint32_t)((ra * kp + 8 * c) * 2);
    }
#pragma unroll
    for (int i = 0; i < SB / 8; ++i) {
        const int qq = (w + 8 * i) * 64 + lane;
        const int r = qq >> 3, c = (qq & 7) ^ ((r >> 1) & 7);
        const int rb = min(n0 + r, N - 1) - n0;
        boff[i] = (uint32_t)(((int64_t)rb * kp + 8 * c) * 2);
    }
    const uint16_t* abase = A + m0 * kp;
    const uint16_t* bbase = B + (int64_t)n0 * kp;
    auto issue = [&](int kc, int stage) {
#pragma unroll
        for (int i = 0; i < SA / 8; ++i) dma16(abase + kc * KC, aoff[i], &As[stage][(w + 8 * i) * 512]);
#pragma unroll
        for (int i = 0; i < SB / 8; ++i) dma16(bbase + kc * KC, boff[i], &Bs[stage][(w + 8 * i) * 512]);
    };
    f32x4_t acc[8][NB];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int wm = (w >> 2) * 128, wn = (w & 3) * 16 * NB;
    auto swz = [](int row, int c) { return (row * 8 + (c ^ ((row >> 1) & 7))) * 8; };
    const int nk = kp / KC;
    issue(0, 0);
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    __syncthreads();
    for (int kc = 0; kc < nk; ++kc) {
        const int stage = kc & 1;
        if (kc + 1 < nk) issue(kc + 1, stage ^ 1);
#pragma unroll
        for (int ks = 0; ks < KC / 32; ++ks) {
            const int c = 4 * ks + (lane >> 4);
            bf16x8_t bfr[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[stage][swz(wn + 16 * j + (lane & 15), c)]);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(&As[stage][swz(wm + 16 * i + (lane & 15), c)]);
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[j], acc[i][j], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
        __syncthreads();
    }
    if (nr > 0) {
        // dl [256 tokens][nr4] and W_r [BN columns][nr4] of the tile in float32 (zero past the
        // edges and past nr), then k-steps of four router columns
        const int nr4 = (nr + 3) & ~3;
        float* dls = reinterpret_cast<float*>(&As[0][0]);
        float* wrs = reinterpret_cast<float*>(&Bs[0][0]);
        for (int q = tid; q < BM * nr4; q += 512) {
            const int r = q / nr4, e = q % nr4;
            dls[q] = (m0 + r < M && e < nr) ? dl[(m0 + r) * nr + e] : 0.f;
        }
        for (int q = tid; q < BN * nr4; q += 512) {
            const int r = q / nr4, e = q % nr4;
            wrs[q] = (n0 + r < N && e < nr) ? wr[(int64_t)(n0 + r) * nr + e] : 0.f;
        }
        __syncthreads();
        for (int e0 = 0; e0 < nr4; e0 += 4) {
            float bq[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j) bq[j] = wrs[(wn + 16 * j + (lane & 15)) * nr4 + e0 + (lane >> 4)];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float af = dls[(wm + 16 * i + (lane & 15)) * nr4 + e0 + (lane >> 4)];
#pragma unroll
                for (int j = 0; j < NB; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af, bq[j], acc[i][j], 0, 0, 0);
            }
        }
    }
    // lane: rows (tokens) 4 (lane / 16) + 0..3 of each 16 x 16 block, column lane % 16
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t m = m0 + wm + 16 * i + 4 * (lane >> 4) + r;
                const int n = n0 + wn + 16 * j + (lane & 15);
                if (m < M && n < N) C[m * N + n] = acc[i][j][r];
            }
}

// CUs of the current device (cached per device)
int device_cus() {
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// C [M][N] = A B^T (+ dl W_r^T) with the tile width that fills the CUs in the fewest rounds (time of
// a round taken as proportional to the tile width; ties to the wider tile)
hipError_t launch_bt_gemm(const uint16_t* A, const uint16_t* B, float* C, int64_t M, int N, int kp, const float* dl,
                          const float* wr, int nr, hipStream_t st) {
    const int64_t cus = device_cus(), tm = ceil_div(M, 256);
    int nb = 3;
    double best = 1e300;
    for (int b = 2; b <= 5; ++b) {
        const double cost = (double)ceil_div(tm * ceil_div(N, 64 * b), cus) * b;
        if (cost <= best) {
            best = cost;
            nb = b;
        }
    }
    const unsigned tiles = (unsigned)(tm * ceil_div(N, 64 * nb));
    switch (nb) {
        case 2: bt_gemm_kernel<2><<<tiles, 512, 0, st>>>(A, B, C, M, N, kp, dl, wr, nr); break;
        case 3: bt_gemm_kernel<3><<<tiles, 512, 0, st>>>(A, B, C, M, N, kp, dl, wr, nr); break;
        case 4: bt_gemm_kernel<4><<<tiles, 512, 0, st>>>(A, B, C, M, N, kp, dl, wr, nr); break;
        default: bt_gemm_kernel<5><<<tiles, 512, 0, st>>>(A, B, C, M, N, kp, dl, wr, nr); break;
    }
    return hipGetLastError();
}


// Columns of gcat / wcat: the concatenated input-side blocks rounded up to whole 64-wide slices.
int wg_kp(const BwdArgs& a) { return (int)round_up((int64_t)(2 * a.G + a.s + a.N) * a.dh, 64); }

// Launches one token-contracted product set (jobs in order) and its reduce.
hipError_t wg_launch(WgArgs wa, hipStream_t st) {
    int tiles = 0;
    int64_t off = 0;
    for (int i = 0; i < wa.njobs; ++i) {
        WgJob& J = wa.job[i];
        J.tiles_n = (int)ceil_div(J.N, 128);
        J.tile0 = tiles;
        tiles += (int)ceil_div(J.M, 128) * J.tiles_n;
        J.part = off;
        off += (int64_t)wa.splits * J.M * J.N;
    }
    wa.ntiles = tiles;
    wg_gemm_kernel<<<dim3((unsigned)tiles, (unsigned)wa.splits), 256, 0, st>>>(wa);
    int64_t mn = 0;
    for (int i = 0; i < wa.njobs; ++i) mn = std::max(mn, (int64_t)wa.job[i].M * wa.job[i].N);
    wg_reduce_kernel<<<dim3((unsigned)ceil_div(mn, 256), (unsigned)wa.njobs), 256, 0, st>>>(wa);
    return hipGetLastError();
}

template <class Prob, bool AK, bool BK>
void tgemm(bool mfma, const Prob& p, int maxM, int maxN, int nsub, hipStream_t st, int splits = 1,
           float* part = nullptr) {
    if (nsub <= 0) return;
    const int64_t pstride = (int64_t)maxM * maxN;
    const dim3 grid((unsigned)ceil_div(maxN, 64), (unsigned)ceil_div(maxM, 64), (unsigned)(nsub * splits));
    if (mfma) tgemm_mfma_kernel<Prob, AK, BK><<<grid, 256, 0, st>>>(p, splits, part, pstride);
    else tgemm_kernel<Prob, AK, BK><<<grid, 256, 0, st>>>(p, splits, part, pstride);
    if (splits > 1)
        tgemm_reduce_kernel<Prob><<<dim3((unsigned)ceil_div(pstride, 256), (unsigned)nsub), 256, 0, st>>>(p, splits, part,
                                                                                                           pstride);
}

template <typename T>
hipError_t run(const BwdArgs& a, const Lists& L, hipStream_t st, KernelMarks* km) {
    auto blocks = [](int64_t n) { return (unsigned)ceil_div(n, 256); };
    const bool rslot = !a.dense && a.variant == GQE_VARIANT_GQE;
    const int nsm = a.N + (rslot ? a.G : 0) + a.s;
    const int nt = (int)a.T;
    if (km) km->begin(KT_BWD_OUT);
    // bf16 layers: the GEMM-shaped steps on matrix cores, except the router's (float32 weights and
    // logit gradients stay float32)
    const bool mm = sizeof(T) == 2;
    // bf16: the output-slot, weight and input gradients as whole products over zero-expanded
    // operands (conditions in launch_backward)
    const bool wgp = a.wgp != 0;
    if (wgp) {
        // U = dy W_slots^T for every slot of every token (the experts zero-expanded: slots the token
        // did not choose are computed and not read), one product
        const int nso = a.NS * a.dh;
        wg_wslot_kernel<<<blocks((int64_t)nso * (a.d / 8)), 256, 0, st>>>(a, a.wg_wslot);
        const hipError_t e = launch_bt_gemm(reinterpret_cast<const uint16_t*>(a.dy), a.wg_wslot, a.U, a.T, nso, a.d,
                                            nullptr, nullptr, 0, st);
        if (e != hipSuccess) return e;
    } else {
        tgemm<ProbU<T>, true, true>(mm, ProbU<T>{a, L}, nt, a.dh, nsm, st);
    }
    bwd_route_kernel<T><<<blocks(4 * a.T * a.G), 256, 0, st>>>(a);
    if (km) km->mark(KT_BWD_OUT);
    if (km) km->begin(KT_BWD_ATTN);
    const unsigned nblk = (unsigned)ceil_div(a.S, 64);
    const dim3 gq(nblk, (unsigned)a.H, (unsigned)a.B), gk(nblk, (unsigned)a.G, (unsigned)a.B);
    if (sizeof(T) == 2) {
        // bf16: matrix cores
        const int64_t n = a.B * (a.G + a.H) * a.S_pad * (a.dh / 8);
        bwd_mprep_kernel<<<(unsigned)ceil_div(n, 256), 256, 0, st>>>(a, a.vr, a.dob);
        const dim3 gq1((unsigned)(ceil_div(a.S, 16 * kDqWaves) * a.H * a.B)),
            gk1((unsigned)(ceil_div(a.S, 128) * (a.G + a.s) * a.B));
#define GQE_BWD_MFMA(DHV)                                                     \
    bwd_dq_mfma_kernel<DHV><<<gq1, 64 * kDqWaves, 0, st>>>(a, a.vr, a.dob);   \
    bwd_dkv_mfma_kernel<DHV><<<gk1, 256, 0, st>>>(a, a.vr, a.dob);
        switch (a.dh / 16) {  // d_h: a multiple of 16, at most 128
            case 1: GQE_BWD_MFMA(16) break;
            case 2: GQE_BWD_MFMA(32) break;
            case 3: GQE_BWD_MFMA(48) break;
            case 4: GQE_BWD_MFMA(64) break;
            case 5: GQE_BWD_MFMA(80) break;
            case 6: GQE_BWD_MFMA(96) break;
            case 7: GQE_BWD_MFMA(112) break;
            default: GQE_BWD_MFMA(128) break;
        }
#undef GQE_BWD_MFMA
        if (a.s) bwd_kv_sum_kernel<<<(unsigned)ceil_div(a.T * a.dh, 256), 256, 0, st>>>(a);
        if (km) km->mark(KT_BWD_ATTN);
        goto weights;
    }
#define GQE_BWD_ATTN(DQV)                                     \
    bwd_dq_kernel<T, DQV><<<gq, 256, 0, st>>>(a);             \
    bwd_dkv_kernel<T, DQV><<<gk, 256, 0, st>>>(a);
    switch (a.dh / 4) {
        case 4: GQE_BWD_ATTN(4) break;
        case 8: GQE_BWD_ATTN(8) break;
        case 12: GQE_BWD_ATTN(12) break;
        case 16: GQE_BWD_ATTN(16) break;
        case 20: GQE_BWD_ATTN(20) break;
        case 24: GQE_BWD_ATTN(24) break;
        case 28: GQE_BWD_ATTN(28) break;
        default: GQE_BWD_ATTN(32) break;
    }
#undef GQE_BWD_ATTN
    if (km) km->mark(KT_BWD_ATTN);
weights:
    if (km) km->begin(KT_BWD_WGRAD);
    // weight gradients reduce over the tokens: split-K pieces summed in order
    if (wgp) {
        // bf16: two token-contracted products over zero-expanded operands (routed experts as
        // blocks that are zero where the token did not choose them)
        const int nslot = (rslot ? a.G : 0) + a.s;
        const int kp = wg_kp(a);
        const int nch = kp / 8 + (a.N + nslot) * a.dh / 8;  // 16-byte chunks of a token's two rows
        const dim3 ge((unsigned)ceil_div(nch, 64), (unsigned)ceil_div(a.T, 4));
        wg_expand_kernel<T><<<ge, 256, 0, st>>>(a, a.wg_gcat, kp, a.wg_ocat, nslot);
        WgArgs wa{};
        wa.T = a.T;
        wa.splits = kWgSplits;
        wa.kc = (int)round_up(ceil_div(a.T, kWgSplits), 32);
        wa.dh = a.dh;
        wa.part = a.part;
        const int no = (a.N + nslot) * a.dh;  // slot columns of a token
        const uint16_t* dyb = reinterpret_cast<const uint16_t*>(a.dy);
        const uint16_t* xb = reinterpret_cast<const uint16_t*>(a.x);
        // output side: dW_o / dW_oR / dW_os [slot d_h][d] = slot^T dy
        wa.job[0] = WgJob{a.wg_ocat, dyb, no, a.d, a.N * a.dh, a.d, 0, 0, 0, a.dwo, 0};
        wa.njobs = 1;
        if (rslot) wa.job[wa.njobs++] = WgJob{a.wg_ocat + a.N * a.dh, dyb, no, a.d, a.G * a.dh, a.d, 0, 0, 0, a.dwor, 0};
        if (a.s) wa.job[wa.njobs++] = WgJob{a.wg_ocat + (no - a.dh), dyb, no, a.d, a.dh, a.d, 0, 0, 0, a.dwos, 0};
        hipError_t e = wg_launch(wa, st);
        if (e != hipSuccess) return e;
        // input side: dW_k, dW_v [d][G d_h], dW_qs [d][d_h] = x^T g; dW_q [N][d][d_h] from the
        // zero-expanded routed gradients
        const int gd = a.G * a.dh;
        const uint16_t* gc = a.wg_gcat;
        wa.job[0] = WgJob{xb, gc, a.d, kp, a.d, gd, 0, 0, 0, a.dwk, 0};
        wa.job[1] = WgJob{xb, gc + gd, a.d, kp, a.d, gd, 0, 0, 0, a.dwv, 0};
        wa.job[2] = WgJob{xb, gc + 2 * gd + a.s * a.dh, a.d, kp, a.d, a.N * a.dh, 0, 0, 0, a.dwq, 1};
        wa.njobs = 3;
        if (a.s) wa.job[wa.njobs++] = WgJob{xb, gc + 2 * gd, a.d, kp, a.d, a.dh, 0, 0, 0, a.dwqs, 0};
        e = wg_launch(wa, st);
        if (e != hipSuccess) return e;
    } else {
        tgemm<ProbWo<T>, false, false>(mm, ProbWo<T>{a, L}, a.dh, a.d, nsm, st, kWgradSplits, a.part);
        const int nwx = 2 * a.G + a.s + a.N;  // head blocks and experts (the router has its own kernel)
        tgemm<ProbWx<T>, false, false>(mm, ProbWx<T>{a, L}, a.d, a.dh, nwx, st, kWgradSplits, a.part);
    }
    if (!a.dense) {
        const int nchunk = (int)std::min<int64_t>(kRouterChunks, ceil_div(a.T, kRgTok));
        const dim3 gr((unsigned)ceil_div(a.d + 1, 256), (unsigned)ceil_div(a.N, 16), (unsigned)nchunk);
        bwd_router_wgrad_kernel<T><<<gr, 256, 0, st>>>(a, nchunk, a.part);
        bwd_router_wgrad_reduce<<<(unsigned)ceil_div((int64_t)(a.d + 1) * a.N * 8, 256), 256, 0, st>>>(a, nchunk,
                                                                                                     a.part);
    }
    if (km) km->mark(KT_BWD_WGRAD);
    if (km) km->begin(KT_BWD_DX);
    if (wgp) {
        // bf16: dx = gcat wcat^T + dl W_r^T in one kernel (gcat from the weights stage)
        const int kp = wg_kp(a);
        wg_wcat_kernel<<<blocks((int64_t)a.d * (kp / 8)), 256, 0, st>>>(a, a.wg_wcat, kp);
        const hipError_t e = launch_bt_gemm(a.wg_gcat, a.wg_wcat, a.dx, a.T, a.d, kp, a.dl, a.wr, a.dense ? 0 : a.N, st);
        if (e != hipSuccess) return e;
    } else {
        // routed heads inside the dense product while that costs at most 4x their own work
        const int expand = a.n <= 4 * a.k ? 1 : 0;
        tgemm<ProbDxDense<T>, true, true>(mm, ProbDxDense<T>{a, 0, expand}, nt, a.d, 1, st);
        if (!a.dense) tgemm<ProbDxDense<T>, true, true>(false, ProbDxDense<T>{a, 1, 0}, nt, a.d, 1, st);
        if (!expand)
            for (int g = 0; g < a.G; ++g)
                for (int r = 0; r < a.k; ++r)
                    tgemm<ProbDxRouted<T>, true, true>(mm, ProbDxRouted<T>{a, L, g, r}, nt, a.d, a.n, st);
    
    }
    if (km) km->mark(KT_BWD_DX);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const GqeDims& D, const WorkPlan& P, const BwdPlan& BP, const gqe_weights_t& w,
                           const void* packed, const PackedLayout& pl, const void* x, const void* dy, double aux_coef,
                           const char* fws, char* ws, const gqe_grads_t& gr, hipStream_t st, KernelMarks* km) {
    BwdArgs a{};
    a.x = x;
    a.dy = dy;
    a.idx = (const int32_t*)(fws + P.idx);
    a.counts = (const int64_t*)(fws + P.stats);
    a.Q = fws + P.q;
    a.K = fws + P.kk;
    a.Vt = fws + P.vt;
    a.O = fws + P.o;
    a.wq = w.w_q;
    a.wqs = w.w_q_shared;
    a.wk = w.w_k;
    a.wv = w.w_v;
    a.wo = w.w_o;
    a.wor = w.w_o_rslot;
    a.wos = w.w_o_shared;
    a.wr = w.w_router;
    a.probs = (const float*)(fws + P.probs);
    a.rope = D.rope > 0.f ? (const double*)((const char*)packed + pl.rope) : nullptr;
    a.U = (float*)(ws + BP.U);
    a.dO = (float*)(ws + BP.dO);
    a.Dd = (float*)(ws + BP.Dd);
    a.lse = (float*)(ws + BP.lse);
    if (D.dtype == GQE_DTYPE_BF16 && P.lse_ok) {
        // the forward's attention stored every row's log-sum-exp: the query-block kernel skips its
        // first pass and both attention kernels read it from the forward workspace
        a.lse = const_cast<float*>(reinterpret_cast<const float*>(fws + P.lse));
        a.lse_fwd = 1;
    }
    a.dl = (float*)(ws + BP.dl);
    a.cf = (float*)(ws + BP.cf);
    a.wn = (float*)(ws + BP.wn);
    a.dQ = ws + BP.dQ;
    a.dK = ws + BP.dK;
    a.dV = ws + BP.dV;
    a.part = (float*)(ws + BP.part);
    a.vr = (uint16_t*)(ws + BP.vr);
    a.dob = (uint16_t*)(ws + BP.dob);
    a.kvp = (float*)(ws + BP.kvp);
    a.wg_gcat = (uint16_t*)(ws + BP.wg_gcat);
    a.wg_wcat = (uint16_t*)(ws + BP.wg_wcat);
    a.wg_wslot = (uint16_t*)(ws + BP.wg_wslot);
    a.wg_ocat = (uint16_t*)(ws + BP.wg_ocat);
    a.dx = gr.dx;
    a.dwr = gr.d_router;
    a.dbr = gr.d_router_bias;
    a.dwq = gr.d_q;
    a.dwqs = gr.d_q_shared;
    a.dwk = gr.d_k;
    a.dwv = gr.d_v;
    a.dwo = gr.d_o;
    a.dwor = gr.d_o_rslot;
    a.dwos = gr.d_o_shared;
    a.aux_coef = aux_coef;
    a.B = P.B;
    a.S = P.S;
    a.T = P.T;
    a.S_pad = P.S_pad;
    a.d = D.d;
    a.N = D.N;
    a.G = D.G;
    a.k = D.k;
    a.n = D.n;
    a.dh = D.dh;
    a.H = D.H;
    a.s = D.s;
    a.skv = D.skv;
    a.variant = D.variant;
    a.dense = D.dense;
    // bf16 whole products over zero-expanded operands while the routed part costs at most 4x its
    // own work (n <= 4k), the router term fits the dx product's epilogue (N <= 64) and the hidden
    // size tiles the 64-wide slices of the U and dx products (d % 64 == 0)
    a.wgp = (D.dtype == GQE_DTYPE_BF16 && D.d % 64 == 0 && D.n <= 4 * D.k && D.N <= 64) ? 1 : 0;
    a.NS = a.wgp ? BP.NSX : BP.NS;
    a.Np = (int)round_up(D.N, 16);
    Lists L{(const int32_t*)(ws + BP.offs), (const int32_t*)(ws + BP.perm), (const int32_t*)(ws + BP.rank)};
    if (!D.dense) {
        hipError_t e = launch_bucket(D, P, const_cast<char*>(fws), (int32_t*)(ws + BP.offs), (int32_t*)(ws + BP.perm),
                                     (int32_t*)(ws + BP.inv), st);
        if (e != hipSuccess) return e;
        const int64_t n = P.T * D.G * D.k;
        list_rank_kernel<<<(unsigned)ceil_div(n, 256), 256, 0, st>>>((const int32_t*)(ws + BP.inv), n, D.k,
                                                                     (int32_t*)(ws + BP.rank));
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return D.dtype == GQE_DTYPE_BF16 ? run<bf16_t>(a, L, st, km) : run<float>(a, L, st, km);
}
