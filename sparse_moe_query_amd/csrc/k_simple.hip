// Scalar GPU path of the GQE forward pass: one thread per output element, float32 arithmetic.
// It serves float32 layers and every shape the matrix-core path does not tile (any d, d_h <= 128).
// Same workspace layouts as the matrix-core path:
//   Q_act [B, H, S, d_h]; K [B, G, S_pad, d_h]; V^T [B, G, d_h, S_pad] (keys slotted by vt_pos);
//   O_act [B, S, H, d_h]; virtual head v = g*k + r for the r-th choice of group g, v = G*k for
//   the shared head.
#include "gqe_common.h"
#include "gqe_internal.h"

namespace {

struct Args {
    int64_t B, S, T, S_pad;
    int d, N, G, k, n, dh, H, s, skv, variant, dense;
};

// Projections (GQE README "Algorithm Overview": dense, unchanged K/V for every group; only the
// selected query heads are computed; plus the always-on shared query head).
// With the rotary embedding each query / key element also computes its pair partner (j ^ 1).
template <typename T>
__global__ void proj_simple_kernel(Args a, const T* __restrict__ x, const T* __restrict__ wk,
                                   const T* __restrict__ wv, const T* __restrict__ wqs,
                                   const T* __restrict__ wq, const int32_t* __restrict__ idx,
                                   const double* __restrict__ rope, int use_rope,
                                   T* __restrict__ Q, T* __restrict__ K, T* __restrict__ Vt) {
    const int64_t C = (int64_t)(2 * a.G + a.s + a.G * a.k) * a.dh;
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= a.T * C) return;
    const int64_t t = q / C;
    const int c = (int)(q % C);
    const int64_t b = t / a.S, s = t % a.S;
    const T* xr = x + t * a.d;
    const int GD = a.G * a.dh;
    float acc = 0.f;
    if (c < 2 * GD) {
        const T* w = c < GD ? wk : wv;
        const int cc = c % GD;
        for (int i = 0; i < a.d; ++i) acc += to_f32(xr[i]) * to_f32(w[(int64_t)i * GD + cc]);
        const int g = cc / a.dh, j = cc % a.dh;
        if (c < GD && use_rope) {
            float pr = 0.f;
            for (int i = 0; i < a.d; ++i) pr += to_f32(xr[i]) * to_f32(w[(int64_t)i * GD + (cc ^ 1)]);
            float lo = (j & 1) ? pr : acc, hi = (j & 1) ? acc : pr;
            rope_pair(lo, hi, s, rope[j >> 1]);
            acc = (j & 1) ? hi : lo;
        }
        if (c < GD) K[((b * a.G + g) * a.S_pad + s) * a.dh + j] = from_f32<T>(acc);
        else Vt[((b * a.G + g) * a.dh + j) * a.S_pad + vt_pos(s)] = from_f32<T>(acc);
        return;
    }
    int cc = c - 2 * GD;
    int v, j;
    const T* w;
    if (a.s && cc < a.dh) {
        v = a.G * a.k;
        j = cc;
        w = wqs;
    } else {
        cc -= a.s * a.dh;
        v = cc / a.dh;
        j = cc % a.dh;
        const int g = v / a.k, r = v % a.k;
        const int e = a.dense ? g * a.n + r : idx[(t * a.G + g) * a.k + r];
        w = wq + (int64_t)e * a.d * a.dh;
    }
    for (int i = 0; i < a.d; ++i) acc += to_f32(xr[i]) * to_f32(w[(int64_t)i * a.dh + j]);
    if (use_rope) {
        float pr = 0.f;
        for (int i = 0; i < a.d; ++i) pr += to_f32(xr[i]) * to_f32(w[(int64_t)i * a.dh + (j ^ 1)]);
        float lo = (j & 1) ? pr : acc, hi = (j & 1) ? acc : pr;
        rope_pair(lo, hi, s, rope[j >> 1]);
        acc = (j & 1) ? hi : lo;
    }
    // stored pre-scaled by log2(e)/sqrt(d_h): the attention works in log2 units
    Q[((b * a.H + v) * a.S + s) * a.dh + j] = from_f32<T>(acc * (1.44269504088896341f / sqrtf((float)a.dh)));
}

// Causal attention of one query row (online softmax over keys 0..s of its group).
template <typename T>
__global__ void attn_simple_kernel(Args a, const T* __restrict__ Q, const T* __restrict__ K,
                                   const T* __restrict__ Vt, T* __restrict__ O) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= a.B * a.H * a.S) return;
    const int64_t s = q % a.S;
    const int v = (int)((q / a.S) % a.H);
    const int64_t b = q / (a.S * a.H);
    const int g = v < a.G * a.k ? v / a.k : a.skv;
    float qv[128], o[128];
    const T* qr = Q + ((b * a.H + v) * a.S + s) * a.dh;
    for (int j = 0; j < a.dh; ++j) {
        qv[j] = to_f32(qr[j]);
        o[j] = 0.f;
    }
    float m = -INFINITY, l = 0.f;  // scores are already in log2 units
    const T* Kg = K + (b * a.G + g) * a.S_pad * a.dh;
    const T* Vg = Vt + (b * a.G + g) * a.dh * a.S_pad;
    for (int64_t kk = 0; kk <= s; ++kk) {
        float sc = 0.f;
        for (int j = 0; j < a.dh; ++j) sc += qv[j] * to_f32(Kg[kk * a.dh + j]);
        const float mn = fmaxf(m, sc);
        const float alpha = exp2f(m - mn);
        const float p = exp2f(sc - mn);
        l = l * alpha + p;
        const int64_t pos = vt_pos(kk);
        for (int j = 0; j < a.dh; ++j) o[j] = o[j] * alpha + p * to_f32(Vg[(int64_t)j * a.S_pad + pos]);
        m = mn;
    }
    T* orow = O + ((b * a.S + s) * a.H + v) * a.dh;
    const float inv = 1.0f / l;
    for (int j = 0; j < a.dh; ++j) orow[j] = from_f32<T>(o[j] * inv);
}

// Key norms for the matrix-core attention kernel's range test (when the projection ran here).
template <typename T>
__global__ void kn_simple_kernel(Args a, const T* __restrict__ K, float* __restrict__ kn) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= a.B * a.G * a.S) return;
    const int64_t s = q % a.S, bg = q / a.S;
    const T* kr = K + (bg * a.S_pad + s) * a.dh;
    float ss = 0.f;
    for (int j = 0; j < a.dh; ++j) ss += to_f32(kr[j]) * to_f32(kr[j]);
    kn[bg * a.S_pad + s] = sqrtf(ss) * 1.01f;  // margin for the float32 rounding of the sum
}

// Output construction (README "Parameters"/"Ablations"; explainer "Output Construction").
template <typename T>
__global__ void combine_simple_kernel(Args a, const T* __restrict__ O, const int32_t* __restrict__ idx,
                                      const float* __restrict__ wsel, const float* __restrict__ psel,
                                      const T* __restrict__ wo, const T* __restrict__ wor,
                                      const T* __restrict__ wos, T* __restrict__ y) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= a.T * a.d) return;
    const int64_t t = q / a.d;
    const int col = (int)(q % a.d);
    const T* ot = O + t * a.H * a.dh;
    float acc = 0.f;
    for (int g = 0; g < a.G; ++g) {
        for (int r = 0; r < a.k; ++r) {
            const int v = g * a.k + r;
            const int64_t o = (t * a.G + g) * a.k + r;
            const int e = a.dense ? g * a.n + r : idx[o];
            const float coef = (!a.dense && a.variant == GQE_VARIANT_WEIGHTED_CONCAT) ? psel[o] : 1.f;
            float part = 0.f;
            for (int j = 0; j < a.dh; ++j)
                part += to_f32(ot[v * a.dh + j]) * to_f32(wo[((int64_t)e * a.dh + j) * a.d + col]);
            acc += coef * part;
        }
        if (!a.dense && a.variant == GQE_VARIANT_GQE) {
            float part = 0.f;
            for (int j = 0; j < a.dh; ++j) {
                float slot = 0.f;
                for (int r = 0; r < a.k; ++r)
                    slot += wsel[(t * a.G + g) * a.k + r] * to_f32(ot[(g * a.k + r) * a.dh + j]);
                part += slot * to_f32(wor[((int64_t)g * a.dh + j) * a.d + col]);
            }
            acc += part;
        }
    }
    if (a.s) {
        const int v = a.G * a.k;
        float part = 0.f;
        for (int j = 0; j < a.dh; ++j) part += to_f32(ot[v * a.dh + j]) * to_f32(wos[(int64_t)j * a.d + col]);
        acc += part;
    }
    y[q] = from_f32<T>(acc);
}

template <typename T>
Args make_args(const GqeDims& D, const WorkPlan& P) {
    return Args{P.B, P.S, P.T, P.S_pad, D.d, D.N, D.G, D.k, D.n, D.dh, D.H, D.s, D.skv, D.variant, D.dense};
}

template <typename T>
hipError_t proj(const GqeDims& D, const WorkPlan& P, const gqe_weights_t& w, const void* x, const double* rope,
                char* ws, hipStream_t st) {
    const Args a = make_args<T>(D, P);
    const int64_t C = (int64_t)(2 * D.G + D.s + D.G * D.k) * D.dh;
    proj_simple_kernel<T><<<(unsigned)ceil_div(P.T * C, 256), 256, 0, st>>>(
        a, (const T*)x, (const T*)w.w_k, (const T*)w.w_v, (const T*)w.w_q_shared, (const T*)w.w_q,
        (const int32_t*)(ws + P.idx), rope, D.rope > 0.f ? 1 : 0, (T*)(ws + P.q), (T*)(ws + P.kk),
        (T*)(ws + P.vt));
    return hipGetLastError();
}

template <typename T>
hipError_t attn(const GqeDims& D, const WorkPlan& P, char* ws, hipStream_t st) {
    const Args a = make_args<T>(D, P);
    attn_simple_kernel<T><<<(unsigned)ceil_div(P.B * D.H * P.S, 128), 128, 0, st>>>(
        a, (const T*)(ws + P.q), (const T*)(ws + P.kk), (const T*)(ws + P.vt), (T*)(ws + P.o));
    return hipGetLastError();
}

template <typename T>
hipError_t combine(const GqeDims& D, const WorkPlan& P, const gqe_weights_t& w, void* y, char* ws,
                   hipStream_t st) {
    const Args a = make_args<T>(D, P);
    combine_simple_kernel<T><<<(unsigned)ceil_div(P.T * D.d, 256), 256, 0, st>>>(
        a, (const T*)(ws + P.o), (const int32_t*)(ws + P.idx), (const float*)(ws + P.wsel),
        (const float*)(ws + P.psel), (const T*)w.w_o, (const T*)w.w_o_rslot, (const T*)w.w_o_shared, (T*)y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_proj_simple(const GqeDims& D, const WorkPlan& P, const gqe_weights_t& w, const void* x,
                              const double* rope, char* ws, hipStream_t st, KernelMarks* km) {
    if (km) km->begin(KT_PROJ);
    const hipError_t e = D.dtype == GQE_DTYPE_BF16 ? proj<bf16_t>(D, P, w, x, rope, ws, st)
                                                   : proj<float>(D, P, w, x, rope, ws, st);
    if (km) km->mark(KT_PROJ);
    return e;
}
hipError_t launch_attn_simple(const GqeDims& D, const WorkPlan& P, char* ws, hipStream_t st, KernelMarks* km) {
    if (km) km->begin(KT_ATTN);
    const hipError_t e = D.dtype == GQE_DTYPE_BF16 ? attn<bf16_t>(D, P, ws, st) : attn<float>(D, P, ws, st);
    if (km) km->mark(KT_ATTN);
    return e;
}
hipError_t launch_kn_simple(const GqeDims& D, const WorkPlan& P, char* ws, hipStream_t st, KernelMarks* km) {
    const Args a = make_args<bf16_t>(D, P);
    if (km) km->begin(KT_KEYNORM);
    if (D.dtype == GQE_DTYPE_BF16)
        kn_simple_kernel<bf16_t><<<(unsigned)ceil_div(P.B * D.G * P.S, 256), 256, 0, st>>>(
            a, (const bf16_t*)(ws + P.kk), (float*)(ws + P.kn));
    else
        kn_simple_kernel<float><<<(unsigned)ceil_div(P.B * D.G * P.S, 256), 256, 0, st>>>(
            a, (const float*)(ws + P.kk), (float*)(ws + P.kn));
    if (km) km->mark(KT_KEYNORM);
    return hipGetLastError();
}
hipError_t launch_combine_simple(const GqeDims& D, const WorkPlan& P, const gqe_weights_t& w, void* y,
                                 char* ws, hipStream_t st, KernelMarks* km) {
    if (km) km->begin(KT_COMBINE);
    const hipError_t e = D.dtype == GQE_DTYPE_BF16 ? combine<bf16_t>(D, P, w, y, ws, st) : combine<float>(D, P, w, y, ws, st);
    if (km) km->mark(KT_COMBINE);
    return e;
}
