// Decode step of the GQE layer on gfx950: one new token per sequence against a dense KV cache.
//
// GQE README "Algorithm Overview" and the gist.science explainer ("Technical Summary" ->
// "Architecture and Routing", "Dense KV Path"): the key/value projections and the KV cache stay
// dense and unchanged; routing only chooses which query heads a token computes.  So the output of
// the token at position p of a sequence is row p of the causal forward pass over positions 0..p,
// and the keys and values of positions 0..p-1 are exactly what the forward pass (or earlier decode
// steps) computed for them: they are read from the cache instead of being recomputed.
//
// Cache layout: K and V each [cache rows][G][s_max][d_h] in the layer's storage type; sequence b
// of a decode batch uses cache row b.  Everything here is bound by memory or latency (one token
// per sequence: a query row meets its keys once), so the kernels use the vector ALU in float32:
//
//   kv_export_kernel   K [B][G][S_pad][d_h] and the slotted V^T of a forward pass -> cache rows
//   dec_proj_kernel    work group = (head block, up to 8 tokens that use it): head block = K_g,
//                      V_g, the shared query head or routed expert e (the tokens that chose e);
//                      d_h dot products of length d per token, the weights read once per group
//                      of 8 tokens; K and V go to the cache at the token's position, queries
//                      (times log2(e)/sqrt(d_h)) to a float32 buffer
//   dec_attn_kernel    work group = (token, KV group, chunk of C cached keys): the V chunk is
//                      staged in LDS by 16-byte loads, each thread scores one key for all active
//                      heads of the group, then chunk maximum, exp2, row sums and P.V; writes a
//                      float32 partial result (O, maximum, row sum) per head
//   dec_merge_kernel   one wave per (token, head): online-softmax merge of the chunk partials
//   dec_combine_kernel work group = (token, 256 output columns): the variant's output
//                      construction (routed slots, renormalised slot, shared head) fused with the
//                      output projection, weights in their "x @ W" layout
//
// A sequence whose position is outside [0, s_max) is not processed: nothing is written to the
// cache, and its output row is NaN.
#include <math.h>

#include <cmath>

#include "gqe_common.h"
#include "gqe_internal.h"

namespace {

constexpr int kTok = 8;     // tokens per projection work group
constexpr int kDC = 512;    // hidden-dim chunk of the token rows staged in LDS by the projection
constexpr int kMaxH = GQE_DEC_MAX_HEADS;

struct DecArgs {
    const void* x;
    void* y;
    const int32_t* pos;
    void* kc;
    void* vc;
    const void *wq, *wqs, *wk, *wv, *wo, *wor, *wos;
    const int32_t* idx;
    const float* wsel;
    const float* psel;
    float* qd;     // [B][H][dh]
    float* part;   // [B][G][NC][MH][dh + 2]
    float* od;     // [B][H][dh]
    int64_t s_max;
    int B, d, N, G, k, n, dh, H, s, skv, variant, dense, NC, MH, C;
    float qscale;
};

__device__ __forceinline__ bool pos_ok(int p, int64_t s_max) { return p >= 0 && (int64_t)p < s_max; }

// 16 bytes of storage -> float32 values
__device__ __forceinline__ void widen16(const u32x4_t& u, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(u[i] << 16);
        f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void widen16(const u32x4_t& u, float (&f)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(u[i]);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// ---------------------------------------------------------------- forward pass -> cache
template <typename T>
__global__ void __launch_bounds__(256) kv_export_kernel(const T* __restrict__ K, const T* __restrict__ Vt,
                                                        T* __restrict__ kc, T* __restrict__ vc, int64_t S,
                                                        int64_t S_pad, int G, int dh, int64_t s_max, int64_t b0) {
    __shared__ float tile[64][129];  // 64 keys of V, d_h <= 128
    const int b = blockIdx.z, g = blockIdx.y, tid = threadIdx.x;
    const int64_t s0 = (int64_t)blockIdx.x * 64;
    const int ns = (int)(S - s0 < 64 ? S - s0 : 64);
    const int64_t src = (int64_t)b * G + g;
    const int64_t dst = ((b0 + b) * G + g) * s_max + s0;
    const T* ks = K + (src * S_pad + s0) * dh;
    T* kd = kc + dst * dh;
    for (int i = tid; i < ns * dh; i += 256) kd[i] = ks[i];
    const T* vs = Vt + src * dh * S_pad;
    for (int i = tid; i < 64 * dh; i += 256) {
        const int j = i >> 6, o = i & 63;  // neighbouring threads read neighbouring keys
        if (o < ns) tile[o][j] = to_f32(vs[(int64_t)j * S_pad + vt_pos(s0 + o)]);
    }
    __syncthreads();
    T* vd = vc + dst * dh;
    for (int i = tid; i < ns * dh; i += 256) vd[i] = from_f32<T>(tile[i / dh][i % dh]);
}

// ---------------------------------------------------------------- projections of the new tokens
template <typename T>
__global__ void __launch_bounds__(256) dec_proj_kernel(DecArgs a) {
    __shared__ float xs[kTok][kDC];
    __shared__ float red[256 * kTok];
    __shared__ int list[kTok];
    __shared__ int wcount[4];
    const int hb = blockIdx.x, tg = blockIdx.y, tid = threadIdx.x;
    const int G = a.G, dh = a.dh, d = a.d;
    const int ebase = 2 * G + a.s;
    const bool is_exp = hb >= ebase;
    const int e = hb - ebase;
    const int g = is_exp ? e / a.n : (hb < G ? hb : hb - G);

    // tokens of this work group: entries [8 tg, 8 tg + 8) of the tokens that use the head block
    int ntok;
    if (!is_exp || a.dense) {
        const int r = is_exp ? e % a.n : 0;  // all-active GQA: expert j of a group is head j
        ntok = a.B - kTok * tg;
        ntok = ntok < kTok ? ntok : kTok;
        if (tid < ntok) list[tid] = (kTok * tg + tid) | (r << 24);
    } else {
        // routed expert e: its tokens in ascending order (ballot compaction over the batch)
        const int w = tid >> 6;
        int base = 0;
        for (int b0 = 0; b0 < a.B; b0 += 256) {
            const int b = b0 + tid;
            int rank = -1;
            if (b < a.B) {
                const int32_t* id = a.idx + ((int64_t)b * G + g) * a.k;
                for (int r = 0; r < a.k; ++r)
                    if (id[r] == e) rank = r;
            }
            const uint64_t m = __builtin_amdgcn_ballot_w64(rank >= 0);
            if ((tid & 63) == 0) wcount[w] = __builtin_popcountll(m);
            __syncthreads();
            int off = base;
            for (int i = 0; i < w; ++i) off += wcount[i];
            const int pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
            const int slot = off + pre - kTok * tg;
            if (rank >= 0 && slot >= 0 && slot < kTok) list[slot] = b | (rank << 24);
            base += wcount[0] + wcount[1] + wcount[2] + wcount[3];
            __syncthreads();
        }
        ntok = base - kTok * tg;
        ntok = ntok < 0 ? 0 : (ntok < kTok ? ntok : kTok);
    }
    if (ntok <= 0) return;  // uniform over the work group
    __syncthreads();
    int tok[kTok];
#pragma unroll
    for (int t = 0; t < kTok; ++t) tok[t] = t < ntok ? list[t] : list[0];

    const T* W;
    int64_t rs;
    if (hb < G) {
        W = (const T*)a.wk + hb * dh;
        rs = (int64_t)G * dh;
    } else if (hb < 2 * G) {
        W = (const T*)a.wv + (hb - G) * dh;
        rs = (int64_t)G * dh;
    } else if (!is_exp) {
        W = (const T*)a.wqs;
        rs = dh;
    } else {
        W = (const T*)a.wq + (int64_t)e * d * dh;
        rs = dh;
    }
    const int nsl = 256 / dh;  // slices of the hidden dimension (dh <= 128)
    const int j = tid % dh, sl = tid / dh;
    const bool act = sl < nsl;
    float acc[kTok];
#pragma unroll
    for (int t = 0; t < kTok; ++t) acc[t] = 0.f;
    const T* X = (const T*)a.x;
    for (int c0 = 0; c0 < d; c0 += kDC) {
        const int nc = d - c0 < kDC ? d - c0 : kDC;
        for (int i = tid; i < kTok * nc; i += 256) {
            const int t = i / nc, c = i - t * nc;
            xs[t][c] = t < ntok ? to_f32(X[(int64_t)(list[t] & 0xffffff) * d + c0 + c]) : 0.f;
        }
        __syncthreads();
        if (act) {
            const T* wp = W + (int64_t)c0 * rs + j;
            for (int i = sl; i < nc; i += nsl) {
                const float wv = to_f32(wp[(int64_t)i * rs]);
#pragma unroll
                for (int t = 0; t < kTok; ++t) acc[t] += xs[t][i] * wv;
            }
        }
        __syncthreads();
    }
    if (act) {
#pragma unroll
        for (int t = 0; t < kTok; ++t) red[(sl * dh + j) * kTok + t] = acc[t];
    }
    __syncthreads();
    for (int o = tid; o < ntok * dh; o += 256) {
        const int t = o / dh, jj = o - t * dh;
        float v = 0.f;
        for (int q = 0; q < nsl; ++q) v += red[(q * dh + jj) * kTok + t];
        int tk = tok[0];
#pragma unroll
        for (int u = 1; u < kTok; ++u)
            if (t == u) tk = tok[u];
        const int b = tk & 0xffffff, rank = tk >> 24;
        if (hb < 2 * G) {
            const int p = a.pos[b];
            if (!pos_ok(p, a.s_max)) continue;
            T* dst = (T*)(hb < G ? a.kc : a.vc);
            dst[(((int64_t)b * G + g) * a.s_max + p) * dh + jj] = from_f32<T>(v);
        } else {
            const int head = is_exp ? g * (a.dense ? a.n : a.k) + rank : G * a.k;
            a.qd[((int64_t)b * a.H + head) * dh + jj] = v * a.qscale;
        }
    }
}

// ---------------------------------------------------------------- attention over one cache chunk
template <typename T>
__global__ void __launch_bounds__(256) dec_attn_kernel(DecArgs a) {
    constexpr int E16 = 16 / (int)sizeof(T);  // elements per 16-byte load
    __shared__ __align__(16) unsigned char vbuf[32768];
    __shared__ __align__(16) float qs[kMaxH * 128];
    __shared__ float ps[kMaxH * 256];
    __shared__ float red[2048];
    __shared__ float wred[4][kMaxH];
    const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int w = tid >> 6;
    const int p = a.pos[b];
    if (!pos_ok(p, a.s_max)) return;
    const int64_t L = (int64_t)p + 1, c0 = (int64_t)chunk * a.C;
    if (c0 >= L) return;
    const int nk = (int)(L - c0 < a.C ? L - c0 : a.C);
    const int dh = a.dh, G = a.G, C = a.C;
    const int kr = a.dense ? a.n : a.k;
    const int m = kr + ((a.s && g == a.skv) ? 1 : 0);
    for (int i = tid; i < m * dh; i += 256) {
        const int h = i / dh, jj = i - h * dh;
        const int hid = h < kr ? g * kr + h : G * kr;
        qs[i] = a.qd[((int64_t)b * a.H + hid) * dh + jj];
    }
    const int64_t row0 = ((int64_t)b * G + g) * a.s_max + c0;
    {
        const unsigned char* vsrc = (const unsigned char*)a.vc + row0 * dh * (int64_t)sizeof(T);
        const int nbytes = nk * dh * (int)sizeof(T);
        for (int o = tid * 16; o < nbytes; o += 256 * 16)
            *reinterpret_cast<u32x4_t*>(vbuf + o) = *reinterpret_cast<const u32x4_t*>(vsrc + o);
    }
    __syncthreads();  // queries visible

    // scores of key c0 + tid for every active head (log2 units: queries carry log2(e)/sqrt(d_h))
    float sc[kMaxH];
#pragma unroll
    for (int h = 0; h < kMaxH; ++h) sc[h] = -INFINITY;
    if (tid < nk) {
#pragma unroll
        for (int h = 0; h < kMaxH; ++h)
            if (h < m) sc[h] = 0.f;
        const u32x4_t* krow = reinterpret_cast<const u32x4_t*>((const T*)a.kc + (row0 + tid) * dh);
        for (int u = 0; u < dh / E16; ++u) {
            float f[E16];
            widen16(krow[u], f);
#pragma unroll
            for (int h = 0; h < kMaxH; ++h) {
                if (h >= m) break;
                const float* q = qs + h * dh + u * E16;
#pragma unroll
                for (int i = 0; i < E16; ++i) sc[h] += q[i] * f[i];
            }
        }
    }
    float mx[kMaxH], ls[kMaxH];
#pragma unroll
    for (int h = 0; h < kMaxH; ++h) {
        const float v = wave_max(sc[h]);
        if ((tid & 63) == 0) wred[w][h] = v;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < kMaxH; ++h) mx[h] = fmaxf(fmaxf(wred[0][h], wred[1][h]), fmaxf(wred[2][h], wred[3][h]));
    __syncthreads();
#pragma unroll
    for (int h = 0; h < kMaxH; ++h) {
        const float pr = (h < m && tid < nk) ? exp2f(sc[h] - mx[h]) : 0.f;
        if (h < m && tid < C) ps[h * C + tid] = pr;
        const float v = wave_sum(pr);
        if ((tid & 63) == 0) wred[w][h] = v;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < kMaxH; ++h) ls[h] = (wred[0][h] + wred[1][h]) + (wred[2][h] + wred[3][h]);

    // P.V: thread (dim j, key group kg) sums keys kg, kg + KG, ...
    const int KG = 256 / dh;
    const int j = tid % dh, kg = tid / dh;
    if (kg < KG) {
        float o[kMaxH];
#pragma unroll
        for (int h = 0; h < kMaxH; ++h) o[h] = 0.f;
        const T* vb = reinterpret_cast<const T*>(vbuf);
        for (int i = kg; i < nk; i += KG) {
            const float v = to_f32(vb[i * dh + j]);
#pragma unroll
            for (int h = 0; h < kMaxH; ++h)
                if (h < m) o[h] += ps[h * C + i] * v;
        }
#pragma unroll
        for (int h = 0; h < kMaxH; ++h)
            if (h < m) red[(kg * kMaxH + h) * dh + j] = o[h];
    }
    __syncthreads();
    float* dst = a.part + ((((int64_t)b * G + g) * a.NC + chunk) * a.MH) * (dh + 2);
    for (int i = tid; i < m * dh; i += 256) {
        const int h = i / dh, jj = i - h * dh;
        float v = 0.f;
        for (int q = 0; q < KG; ++q) v += red[(q * kMaxH + h) * dh + jj];
        dst[h * (dh + 2) + jj] = v;
    }
    if (tid < m) {
        float mv = mx[0], lv = ls[0];
#pragma unroll
        for (int h = 1; h < kMaxH; ++h)
            if (tid == h) {
                mv = mx[h];
                lv = ls[h];
            }
        dst[tid * (dh + 2) + dh] = mv;
        dst[tid * (dh + 2) + dh + 1] = lv;
    }
}

// ---------------------------------------------------------------- merge of the chunk partials
__global__ void __launch_bounds__(64) dec_merge_kernel(DecArgs a) {
    const int hid = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const int dh = a.dh;
    float* out = a.od + ((int64_t)b * a.H + hid) * dh;
    const int p = a.pos[b];
    if (!pos_ok(p, a.s_max)) {
        for (int j = lane; j < dh; j += 64) out[j] = __builtin_nanf("");
        return;
    }
    const int kr = a.dense ? a.n : a.k;
    const int g = hid < a.G * kr ? hid / kr : a.skv;
    const int h = hid < a.G * kr ? hid % kr : kr;
    const int nch = (int)(((int64_t)p + a.C) / a.C);
    const int64_t cs = (int64_t)a.MH * (dh + 2);
    const float* base = a.part + (((int64_t)b * a.G + g) * a.NC * a.MH + h) * (dh + 2);
    float M = -INFINITY;
    for (int c = 0; c < nch; ++c) M = fmaxf(M, base[c * cs + dh]);
    float l = 0.f;
    for (int c = 0; c < nch; ++c) l += base[c * cs + dh + 1] * exp2f(base[c * cs + dh] - M);
    const float inv = 1.f / l;
    for (int j = lane; j < dh; j += 64) {
        float o = 0.f;
        for (int c = 0; c < nch; ++c) o += base[c * cs + j] * exp2f(base[c * cs + dh] - M);
        out[j] = o * inv;
    }
}

// ---------------------------------------------------------------- output construction + W_o
template <typename T>
__global__ void __launch_bounds__(256) dec_combine_kernel(DecArgs a) {
    __shared__ float vec[GQE_DEC_MAX_SLOT_DIMS];
    __shared__ const T* wsl[GQE_DEC_MAX_SLOTS];
    const int b = blockIdx.y, tid = threadIdx.x;
    const int c = blockIdx.x * 256 + tid;
    const int dh = a.dh, G = a.G, d = a.d;
    T* y = (T*)a.y + (int64_t)b * d;
    if (!pos_ok(a.pos[b], a.s_max)) {
        if (c < d) y[c] = from_f32<T>(__builtin_nanf(""));
        return;
    }
    const int kr = a.dense ? a.n : a.k;
    const bool rslot = !a.dense && a.variant == GQE_VARIANT_GQE;
    const int nr = G * kr;
    const int nslot = nr + (rslot ? G : 0) + a.s;
    const float* o = a.od + (int64_t)b * a.H * dh;
    const int64_t sel = (int64_t)b * G * a.k;  // [b][g][r] of the routing buffers
    for (int i = tid; i < nslot * dh; i += 256) {
        const int sl = i / dh, jj = i - sl * dh;
        float v;
        if (sl < nr) {
            const float coef = (!a.dense && a.variant == GQE_VARIANT_WEIGHTED_CONCAT) ? a.psel[sel + sl] : 1.f;
            v = coef * o[sl * dh + jj];
        } else if (rslot && sl < nr + G) {
            const int g = sl - nr;
            v = 0.f;
            for (int r = 0; r < a.k; ++r) v += a.wsel[sel + g * a.k + r] * o[(g * a.k + r) * dh + jj];
        } else {
            v = o[nr * dh + jj];  // shared head
        }
        vec[i] = v;
    }
    for (int i = tid; i < nslot; i += 256) {
        const T* wp;
        if (i < nr) {
            const int g = i / kr, r = i - g * kr;
            const int e = a.dense ? g * a.n + r : a.idx[sel + g * a.k + r];
            wp = (const T*)a.wo + (int64_t)e * dh * d;
        } else if (rslot && i < nr + G) {
            wp = (const T*)a.wor + (int64_t)(i - nr) * dh * d;
        } else {
            wp = (const T*)a.wos;
        }
        wsl[i] = wp;
    }
    __syncthreads();
    if (c >= d) return;
    float acc = 0.f;
    for (int sl = 0; sl < nslot; ++sl) {
        const T* wp = wsl[sl] + c;
        const float* v = vec + sl * dh;
        for (int jj = 0; jj < dh; ++jj) acc += v[jj] * to_f32(wp[(int64_t)jj * d]);
    }
    y[c] = from_f32<T>(acc);
}

}  // namespace

int decode_chunk(const GqeDims& D) {
    const int row = D.dh * (D.dtype == GQE_DTYPE_BF16 ? 2 : 4);
    return row <= 128 ? 256 : (row <= 256 ? 128 : 64);
}

hipError_t launch_kv_export(const GqeDims& D, const WorkPlan& P, const char* ws, void* kc, void* vc, int64_t s_max,
                            int64_t b0, hipStream_t st) {
    const dim3 grid((unsigned)ceil_div(P.S, 64), (unsigned)D.G, (unsigned)P.B);
    if (D.dtype == GQE_DTYPE_BF16)
        kv_export_kernel<bf16_t><<<grid, 256, 0, st>>>((const bf16_t*)(ws + P.kk), (const bf16_t*)(ws + P.vt),
                                                       (bf16_t*)kc, (bf16_t*)vc, P.S, P.S_pad, D.G, D.dh, s_max, b0);
    else
        kv_export_kernel<float><<<grid, 256, 0, st>>>((const float*)(ws + P.kk), (const float*)(ws + P.vt),
                                                      (float*)kc, (float*)vc, P.S, P.S_pad, D.G, D.dh, s_max, b0);
    return hipGetLastError();
}

hipError_t launch_decode(const GqeDims& D, const DecodePlan& P, const gqe_weights_t& w, const void* x, void* y,
                         const int32_t* pos, void* kc, void* vc, char* ws, hipStream_t st, KernelMarks* km) {
    DecArgs a{};
    a.x = x;
    a.y = y;
    a.pos = pos;
    a.kc = kc;
    a.vc = vc;
    a.wq = w.w_q;
    a.wqs = w.w_q_shared;
    a.wk = w.w_k;
    a.wv = w.w_v;
    a.wo = w.w_o;
    a.wor = w.w_o_rslot;
    a.wos = w.w_o_shared;
    a.idx = (const int32_t*)(ws + P.r.idx);
    a.wsel = (const float*)(ws + P.r.wsel);
    a.psel = (const float*)(ws + P.r.psel);
    a.qd = (float*)(ws + P.qd);
    a.part = (float*)(ws + P.part);
    a.od = (float*)(ws + P.od);
    a.s_max = P.s_max;
    a.B = (int)P.B;
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
    a.NC = (int)P.NC;
    a.MH = P.MH;
    a.C = P.C;
    a.qscale = (float)(1.4426950408889634 / std::sqrt((double)D.dh));
    const bool bf = D.dtype == GQE_DTYPE_BF16;
    const int HB = 2 * D.G + D.s + D.N;
    if (km) km->begin(KT_DEC_PROJ);
    const dim3 gp((unsigned)HB, (unsigned)ceil_div(P.B, kTok));
    if (bf) dec_proj_kernel<bf16_t><<<gp, 256, 0, st>>>(a);
    else dec_proj_kernel<float><<<gp, 256, 0, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (km) km->mark(KT_DEC_PROJ);
    if (km) km->begin(KT_DEC_ATTN);
    const dim3 ga((unsigned)P.NC, (unsigned)D.G, (unsigned)P.B);
    if (bf) dec_attn_kernel<bf16_t><<<ga, 256, 0, st>>>(a);
    else dec_attn_kernel<float><<<ga, 256, 0, st>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (km) km->mark(KT_DEC_ATTN);
    if (km) km->begin(KT_DEC_MERGE);
    dec_merge_kernel<<<dim3((unsigned)D.H, (unsigned)P.B), 64, 0, st>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (km) km->mark(KT_DEC_MERGE);
    if (km) km->begin(KT_DEC_COMBINE);
    const dim3 gc((unsigned)ceil_div(D.d, 256), (unsigned)P.B);
    if (bf) dec_combine_kernel<bf16_t><<<gc, 256, 0, st>>>(a);
    else dec_combine_kernel<float><<<gc, 256, 0, st>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (km) km->mark(KT_DEC_COMBINE);
    return hipSuccess;
}
