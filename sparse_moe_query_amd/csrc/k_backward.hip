// Backward pass of the GQE layer (gfx950): gradients of L = sum(dy * y) + aux_coef * aux with
// respect to x and every weight, the routing decisions of the forward pass held fixed.
//
// GQE README "Usage" trains with lm_loss + 0.01 * collect_aux_loss(attn); the explainer's "Output
// Construction" notes that the renormalised weighted-sum slot is the language-modelling loss's
// differentiable path to the router (top-k itself is piecewise constant), and its "Training and
// Loss" adds the load-balancing loss.  The steps are the chain rule through the forward definition,
// in reverse order:
//
//   bwd_u_kernel      U[t][slot] = dy_t W_slot^T for every output slot of the token (routed expert
//                     e: W_o[e]; group g: W_oR[g]; shared head: W_os)
//   bwd_route_kernel  per (token, group): head-output gradients do = c U_e + w U_g, D = do . o for
//                     the attention, the router probabilities again (float64 logits, as in the
//                     forward), the probability gradients (weighted_concat coefficient,
//                     renormalisation w = p / sum_sel p, aux loss), and the logit gradients through
//                     the in-group softmax
//   bwd_lse_kernel    log-sum-exp of every query row (log2 units, from the stored queries and keys)
//   bwd_dq_kernel     dq = sum_j p_j (do . v_j - D) k_j / sqrt(d_h), rotated back (rotary embedding)
//   bwd_dkv_kernel    dk_j, dv_j summed over the later queries of every head of the group
//   bwd_wgrad_kernels weight gradients as sums over the tokens that use each weight block
//   bwd_dx_kernel     dx = sum over the token's head blocks of dq W^T (+ dk, dv, router logits)
//
// This is the first, scalar form of the backward pass: one thread per output element (or per
// query / key row), float32 arithmetic over the forward's stored Q, K, V^T and O.  It reads the
// forward pass's workspace (routing, statistics, Q, K, V^T, O), which must be unchanged.
#include <math.h>

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
    // weights (gqe_init layouts) and the packed router / rotary tables
    const void *wq, *wqs, *wk, *wv, *wo, *wor, *wos;
    const float* wr;        // [d][N]
    const double* wr64;     // packed router weights
    const double* br64;     // [N]
    int router_fast;        // lane-ordered packed router layout
    const double* rope;     // rotary frequencies (cycles per position) or null
    // backward workspace
    float* U;               // [T][NS][dh]
    float* dO;              // [T][H][dh]
    float* Dd;              // [T][H]
    float* lse;             // [T][H]
    float* dl;              // [T][N]
    float* cf;              // [T][H]: output coefficient of each routed head (p for weighted_concat, else 1)
    float* wn;              // [T][H]: renormalised weight of each routed head (variant gqe)
    float* dQ;              // [T][H][dh] (before the rotation)
    float* dK;              // [T][G][dh] (before the rotation)
    float* dV;              // [T][G][dh]
    // outputs (float32)
    float *dx, *dwr, *dbr, *dwq, *dwqs, *dwk, *dwv, *dwo, *dwor, *dwos;
    double aux_coef;
    int64_t B, S, T, S_pad;
    int d, N, G, k, n, dh, H, s, skv, variant, dense, NS, Np;
};

template <typename T>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
    return to_f32(reinterpret_cast<const T*>(p)[i]);
}

// routed head h = g k + r of token t -> expert; the shared head -> -1
__device__ __forceinline__ int expert_of(const BwdArgs& a, int64_t t, int h) {
    if (h >= a.G * a.k) return -1;
    const int g = h / a.k, r = h % a.k;
    return a.dense ? g * a.n + r : a.idx[(t * a.G + g) * a.k + r];
}
__device__ __forceinline__ int group_of(const BwdArgs& a, int h) { return h < a.G * a.k ? h / a.k : a.skv; }

// ---------------------------------------------------------------- U = dy W_slot^T
// slot ls of token t: routed (g, r) -> ls = g k + r (W_o[e]); group slot -> G k + g (W_oR[g]);
// shared head -> G k + G (gqe) or G k
template <typename T>
__global__ void bwd_u_kernel(BwdArgs a) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per = (int64_t)a.NS * a.dh;
    if (q >= a.T * per) return;
    const int64_t t = q / per;
    const int ls = (int)((q % per) / a.dh), j = (int)(q % a.dh);
    const int nr = a.G * a.k;
    const bool rslot = !a.dense && a.variant == GQE_VARIANT_GQE;
    const T* W;
    if (ls < nr) W = (const T*)a.wo + (int64_t)expert_of(a, t, ls) * a.dh * a.d;
    else if (rslot && ls < nr + a.G) W = (const T*)a.wor + (int64_t)(ls - nr) * a.dh * a.d;
    else W = (const T*)a.wos;
    const T* w = W + (int64_t)j * a.d;
    const T* g = (const T*)a.dy + t * a.d;
    float acc = 0.f;
    for (int c = 0; c < a.d; ++c) acc += to_f32(g[c]) * to_f32(w[c]);
    a.U[q] = acc;
}

// ---------------------------------------------------------------- head-output and router gradients
// thread per (token, group); group 0 also handles the shared head.
template <typename T>
__global__ void bwd_route_kernel(BwdArgs a) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= a.T * a.G) return;
    const int64_t t = q / a.G;
    const int g = (int)(q % a.G);
    const int n = a.n, k = a.k, dh = a.dh, H = a.H, nr = a.G * a.k;
    const int64_t b = t / a.S, s = t % a.S;
    const bool rslot = !a.dense && a.variant == GQE_VARIANT_GQE;
    const float* Ut = a.U + t * a.NS * dh;
    auto O_at = [&](int h, int j) { return ld<T>(a.O, ((b * a.S + s) * H + h) * dh + j); };
    if (g == 0 && a.s) {  // shared head: do = dy W_os^T
        const int hs = nr, ls = nr + (rslot ? a.G : 0);
        float D = 0.f;
        for (int j = 0; j < dh; ++j) {
            const float v = Ut[ls * dh + j];
            a.dO[(t * H + hs) * dh + j] = v;
            D += v * O_at(hs, j);
        }
        a.Dd[t * H + hs] = D;
    }
    if (a.dense) {  // all-active GQA: hard concatenation, no router
        for (int r = 0; r < k; ++r) {
            const int h = g * k + r;
            float D = 0.f;
            for (int j = 0; j < dh; ++j) {
                const float v = Ut[h * dh + j];
                a.dO[(t * H + h) * dh + j] = v;
                D += v * O_at(h, j);
            }
            a.Dd[t * H + h] = D;
            a.cf[t * H + h] = 1.f;
            a.wn[t * H + h] = 0.f;
        }
        return;
    }
    // router probabilities of the group, as the forward pass forms them
    double l[16];
    const T* xr = (const T*)a.x + t * a.d;
    for (int jj = 0; jj < n; ++jj) {
        const int e = g * n + jj;
        double acc = 0.0;
        for (int i = 0; i < a.d; ++i) {
            const double w = a.router_fast ? a.wr64[((int64_t)(i >> 3) * 16 + e) * 8 + (i & 7)]
                                           : a.wr64[(int64_t)i * a.Np + e];
            acc = __builtin_fma((double)to_f32(xr[i]), w, acc);
        }
        l[jj] = acc + a.br64[e];
    }
    double m = l[0];
    for (int jj = 1; jj < n; ++jj) m = fmax(m, l[jj]);
    float den = 0.f;
    for (int jj = 0; jj < n; ++jj) den += expf((float)(l[jj] - m));
    const float inv = 1.0f / den;
    float p[16], dp[16];
    for (int jj = 0; jj < n; ++jj) {
        p[jj] = expf((float)(l[jj] - m)) * inv;
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
        for (int j = 0; j < dh; ++j) {
            const float u = Ut[h * dh + j];
            const float v = rslot ? Ut[(nr + g) * dh + j] : 0.f;
            const float o = O_at(h, j);
            const float dov = coef * u + w * v;
            a.dO[(t * H + h) * dh + j] = dov;
            D += dov * o;
            ou += o * u;
            ov += o * v;
        }
        a.Dd[t * H + h] = D;
        a.cf[t * H + h] = coef;
        a.wn[t * H + h] = w;
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
    for (int jj = 0; jj < n; ++jj) a.dl[t * a.N + g * n + jj] = p[jj] * (dp[jj] - sdp);
}

// ---------------------------------------------------------------- attention
template <typename T>
__global__ void bwd_lse_kernel(BwdArgs a) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= a.T * a.H) return;
    const int64_t t = q / a.H;
    const int h = (int)(q % a.H), g = group_of(a, h);
    const int64_t b = t / a.S, s = t % a.S;
    const int64_t qo = ((b * a.H + h) * a.S + s) * a.dh;
    const int64_t kb = (b * a.G + g) * a.S_pad * a.dh;
    float m = -INFINITY, l = 0.f;
    for (int64_t j = 0; j <= s; ++j) {
        float sc = 0.f;
        for (int i = 0; i < a.dh; ++i) sc += ld<T>(a.Q, qo + i) * ld<T>(a.K, kb + j * a.dh + i);
        if (sc > m) {
            l = l * exp2f(m - sc) + 1.f;
            m = sc;
        } else {
            l += exp2f(sc - m);
        }
    }
    a.lse[q] = m + log2f(l);
}

__device__ __forceinline__ void rope_back(float* v, int n, int64_t pos, const double* rope, int j0) {
    // rotation by the opposite angle: the rotation is orthogonal
    for (int i = 0; i + 1 < n; i += 2) rope_pair(v[i], v[i + 1], -pos, rope[(j0 + i) >> 1]);
}

// thread per (query token, head): dq in registers (d_h <= 128)
template <typename T>
__global__ void bwd_dq_kernel(BwdArgs a) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= a.T * a.H) return;
    const int64_t t = q / a.H;
    const int h = (int)(q % a.H), g = group_of(a, h);
    const int64_t b = t / a.S, s = t % a.S;
    const int dh = a.dh;
    const int64_t qo = ((b * a.H + h) * a.S + s) * dh;
    const int64_t kb = (b * a.G + g) * a.S_pad * dh;
    const int64_t vb = (b * a.G + g) * dh * a.S_pad;
    const float L = a.lse[q], D = a.Dd[q];
    const float* dov = a.dO + q * dh;
    float dq[128];
    for (int i = 0; i < dh; ++i) dq[i] = 0.f;
    for (int64_t j = 0; j <= s; ++j) {
        float sc = 0.f, dA = 0.f;
        for (int i = 0; i < dh; ++i) {
            sc += ld<T>(a.Q, qo + i) * ld<T>(a.K, kb + j * dh + i);
            dA += dov[i] * ld<T>(a.Vt, vb + (int64_t)i * a.S_pad + vt_pos(j));
        }
        const float pj = exp2f(sc - L);
        const float dz = pj * (dA - D);  // gradient of the natural-log score q.k / sqrt(d_h)
        for (int i = 0; i < dh; ++i) dq[i] += dz * ld<T>(a.K, kb + j * dh + i);
    }
    const float sc = 1.f / sqrtf((float)dh);
    for (int i = 0; i < dh; ++i) dq[i] *= sc;
    if (a.rope) rope_back(dq, dh, s, a.rope, 0);
    for (int i = 0; i < dh; ++i) a.dQ[q * dh + i] = dq[i];
}

// thread per (key token, group, 16 head dims): dk, dv of those dims over every later query and
// every head of the group
template <typename T>
__global__ void bwd_dkv_kernel(BwdArgs a) {
    const int parts = a.dh / 16;
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= a.T * a.G * parts) return;
    const int part = (int)(q % parts);
    const int64_t tg = q / parts;
    const int64_t t = tg / a.G;
    const int g = (int)(tg % a.G);
    const int64_t b = t / a.S, j = t % a.S;
    const int dh = a.dh, j0 = 16 * part;
    const int64_t kb = ((b * a.G + g) * a.S_pad + j) * dh;
    const int64_t vb = (b * a.G + g) * dh * a.S_pad;
    const float qs = 1.f / (kLog2e);  // stored queries carry log2(e)/sqrt(d_h): q/sqrt(d_h) = q~ / log2(e)
    float dk[16], dv[16];
    for (int i = 0; i < 16; ++i) dk[i] = dv[i] = 0.f;
    for (int h = 0; h < a.H; ++h) {
        if (group_of(a, h) != g) continue;
        for (int64_t s = j; s < a.S; ++s) {
            const int64_t qo = ((b * a.H + h) * a.S + s) * dh;
            const int64_t qi = (b * a.S + s) * a.H + h;
            const float* dov = a.dO + qi * dh;
            float sc = 0.f, dA = 0.f;
            for (int i = 0; i < dh; ++i) {
                sc += ld<T>(a.Q, qo + i) * ld<T>(a.K, kb + i);
                dA += dov[i] * ld<T>(a.Vt, vb + (int64_t)i * a.S_pad + vt_pos(j));
            }
            const float pj = exp2f(sc - a.lse[qi]);
            const float dz = pj * (dA - a.Dd[qi]);
            for (int i = 0; i < 16; ++i) {
                dk[i] += dz * ld<T>(a.Q, qo + j0 + i) * qs;
                dv[i] += pj * dov[j0 + i];
            }
        }
    }
    if (a.rope) rope_back(dk, 16, j, a.rope, j0);
    for (int i = 0; i < 16; ++i) {
        a.dK[(t * a.G + g) * dh + j0 + i] = dk[i];
        a.dV[(t * a.G + g) * dh + j0 + i] = dv[i];
    }
}

// ---------------------------------------------------------------- weight gradients
// W_o[e] / W_oR[g] / W_os: thread per (slot matrix, j, c), summed over the tokens in order
template <typename T>
__global__ void bwd_wgrad_o_kernel(BwdArgs a) {
    const bool rslot = !a.dense && a.variant == GQE_VARIANT_GQE;
    const int nsm = a.N + (rslot ? a.G : 0) + a.s;
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per = (int64_t)a.dh * a.d;
    if (q >= nsm * per) return;
    const int sm = (int)(q / per), j = (int)((q % per) / a.d), c = (int)(q % a.d);
    const int nr = a.G * a.k;
    float acc = 0.f;
    for (int64_t t = 0; t < a.T; ++t) {
        const float g = ld<T>(a.dy, t * a.d + c);
        const int64_t ob = t * a.H * a.dh;  // O is token-major: [B][S][H][dh]
        float v = 0.f;
        if (sm < a.N) {
            const int gg = sm / a.n;
            for (int r = 0; r < a.k; ++r) {
                const int h = gg * a.k + r;
                if (expert_of(a, t, h) == sm) v += a.cf[t * a.H + h] * ld<T>(a.O, ob + h * a.dh + j);
            }
        } else if (rslot && sm < a.N + a.G) {
            const int gg = sm - a.N;
            for (int r = 0; r < a.k; ++r) {
                const int h = gg * a.k + r;
                v += a.wn[t * a.H + h] * ld<T>(a.O, ob + h * a.dh + j);
            }
        } else {
            v = ld<T>(a.O, ob + nr * a.dh + j);
        }
        acc += v * g;
    }
    float* dst = sm < a.N ? a.dwo + (int64_t)sm * per
                          : (rslot && sm < a.N + a.G ? a.dwor + (int64_t)(sm - a.N) * per : a.dwos);
    dst[(int64_t)j * a.d + c] = acc;
}

// W_k, W_v (per group), W_qs, W_q[e]: thread per (head block, i, j), summed over the tokens
template <typename T>
__global__ void bwd_wgrad_x_kernel(BwdArgs a) {
    const int nhb = 2 * a.G + a.s + a.N;
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per = (int64_t)a.d * a.dh;
    if (q >= nhb * per) return;
    const int hb = (int)(q / per), i = (int)((q % per) / a.dh), j = (int)(q % a.dh);
    const int ebase = 2 * a.G + a.s, nr = a.G * a.k;
    float acc = 0.f;
    for (int64_t t = 0; t < a.T; ++t) {
        const float xv = ld<T>(a.x, t * a.d + i);
        float gv = 0.f;
        if (hb < a.G) gv = a.dK[(t * a.G + hb) * a.dh + j];
        else if (hb < 2 * a.G) gv = a.dV[(t * a.G + hb - a.G) * a.dh + j];
        else if (hb < ebase) gv = a.dQ[(t * a.H + nr) * a.dh + j];
        else {
            const int e = hb - ebase, gg = e / a.n;
            for (int r = 0; r < a.k; ++r) {
                const int h = gg * a.k + r;
                if (expert_of(a, t, h) == e) gv += a.dQ[(t * a.H + h) * a.dh + j];
            }
        }
        acc += xv * gv;
    }
    if (hb < a.G) a.dwk[(int64_t)i * a.G * a.dh + hb * a.dh + j] = acc;
    else if (hb < 2 * a.G) a.dwv[(int64_t)i * a.G * a.dh + (hb - a.G) * a.dh + j] = acc;
    else if (hb < ebase) a.dwqs[(int64_t)i * a.dh + j] = acc;
    else a.dwq[((int64_t)(hb - ebase) * a.d + i) * a.dh + j] = acc;
}

// W_r (thread per (i, e)) and b_r (i == d)
template <typename T>
__global__ void bwd_wgrad_r_kernel(BwdArgs a) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= (int64_t)(a.d + 1) * a.N) return;
    const int i = (int)(q / a.N), e = (int)(q % a.N);
    float acc = 0.f;
    for (int64_t t = 0; t < a.T; ++t) acc += (i < a.d ? ld<T>(a.x, t * a.d + i) : 1.f) * a.dl[t * a.N + e];
    if (i < a.d) a.dwr[(int64_t)i * a.N + e] = acc;
    else a.dbr[e] = acc;
}

// dx[t][i]: every head block of the token (dq W^T, dk W_k^T, dv W_v^T) and the router logits
template <typename T>
__global__ void bwd_dx_kernel(BwdArgs a) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= a.T * a.d) return;
    const int64_t t = q / a.d;
    const int i = (int)(q % a.d);
    const int dh = a.dh, GD = a.G * dh, nr = a.G * a.k;
    float acc = 0.f;
    for (int h = 0; h < a.H; ++h) {
        const float* g = a.dQ + (t * a.H + h) * dh;
        const T* w = h < nr ? (const T*)a.wq + ((int64_t)expert_of(a, t, h) * a.d + i) * dh
                            : (const T*)a.wqs + (int64_t)i * dh;
        for (int j = 0; j < dh; ++j) acc += g[j] * to_f32(w[j]);
    }
    const T* wk = (const T*)a.wk + (int64_t)i * GD;
    const T* wv = (const T*)a.wv + (int64_t)i * GD;
    for (int c = 0; c < GD; ++c) acc += a.dK[t * GD + c] * to_f32(wk[c]) + a.dV[t * GD + c] * to_f32(wv[c]);
    if (!a.dense)
        for (int e = 0; e < a.N; ++e) acc += a.dl[t * a.N + e] * a.wr[(int64_t)i * a.N + e];
    a.dx[q] = acc;
}

template <typename T>
hipError_t run(const BwdArgs& a, hipStream_t st, KernelMarks* km) {
    auto blocks = [](int64_t n) { return (unsigned)ceil_div(n, 256); };
    const bool rslot = !a.dense && a.variant == GQE_VARIANT_GQE;
    if (km) km->begin(KT_BWD_OUT);
    bwd_u_kernel<T><<<blocks(a.T * a.NS * a.dh), 256, 0, st>>>(a);
    bwd_route_kernel<T><<<blocks(a.T * a.G), 256, 0, st>>>(a);
    if (km) km->mark(KT_BWD_OUT);
    if (km) km->begin(KT_BWD_ATTN);
    bwd_lse_kernel<T><<<blocks(a.T * a.H), 256, 0, st>>>(a);
    bwd_dq_kernel<T><<<blocks(a.T * a.H), 256, 0, st>>>(a);
    bwd_dkv_kernel<T><<<blocks(a.T * a.G * (a.dh / 16)), 256, 0, st>>>(a);
    if (km) km->mark(KT_BWD_ATTN);
    if (km) km->begin(KT_BWD_WGRAD);
    const int nsm = a.N + (rslot ? a.G : 0) + a.s;
    bwd_wgrad_o_kernel<T><<<blocks((int64_t)nsm * a.dh * a.d), 256, 0, st>>>(a);
    bwd_wgrad_x_kernel<T><<<blocks((int64_t)(2 * a.G + a.s + a.N) * a.d * a.dh), 256, 0, st>>>(a);
    if (!a.dense) bwd_wgrad_r_kernel<T><<<blocks((int64_t)(a.d + 1) * a.N), 256, 0, st>>>(a);
    if (km) km->mark(KT_BWD_WGRAD);
    if (km) km->begin(KT_BWD_DX);
    bwd_dx_kernel<T><<<blocks(a.T * a.d), 256, 0, st>>>(a);
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
    a.wr64 = (const double*)((const char*)packed + pl.wr64);
    a.br64 = (const double*)((const char*)packed + pl.br64);
    a.router_fast = router_uses_mfma(D) ? 1 : 0;
    a.rope = D.rope > 0.f ? (const double*)((const char*)packed + pl.rope) : nullptr;
    a.U = (float*)(ws + BP.U);
    a.dO = (float*)(ws + BP.dO);
    a.Dd = (float*)(ws + BP.Dd);
    a.lse = (float*)(ws + BP.lse);
    a.dl = (float*)(ws + BP.dl);
    a.cf = (float*)(ws + BP.cf);
    a.wn = (float*)(ws + BP.wn);
    a.dQ = (float*)(ws + BP.dQ);
    a.dK = (float*)(ws + BP.dK);
    a.dV = (float*)(ws + BP.dV);
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
    a.NS = BP.NS;
    a.Np = (int)round_up(D.N, 16);
    return D.dtype == GQE_DTYPE_BF16 ? run<bf16_t>(a, st, km) : run<float>(a, st, km);
}
