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
//   dec_oproj_kernel   work group = (weight slot, up to 8 tokens that use it, 512 output columns):
//                      the variant's output construction (routed slots, renormalised slot, shared
//                      head) fused with the output projection, weights in their "x @ W" layout;
//                      a float32 partial row per (token, slot)
//   dec_ysum_kernel    a token's slot rows added in slot order
//
// A sequence whose position is outside [0, s_max) is not processed: nothing is written to the
// cache, and its output row is NaN.
#include <math.h>

#include <cmath>

#include "gqe_common.h"
#include "gqe_internal.h"

namespace {

constexpr int kTok = 8;     // tokens per projection / output-projection work group
constexpr int kDC = 1024;   // hidden-dim chunk of the token rows staged in LDS by the projection
constexpr int kOprojRows = 12; // output projection: weight rows per batch (two batches in flight)
constexpr int kKeysPerThread = 8;  // attention: keys per thread (chunk = 256 / units x 8 keys)
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
    float* yp;     // [B][NS][d]: a token's output row per slot
    int64_t s_max;
    int B, d, N, G, k, n, dh, H, s, skv, variant, dense, NC, MH, C, NS;
    int up;        // 16-byte units of a d_h row, rounded up to a power of two
    float qscale;
    const double* rope;  // rotary embedding frequencies (cycles per position), or null when off
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

// Lane exchanges without LDS: DPP row permutations and the gfx950 row swaps.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// v[lane] + v[lane ^ 16] and v[lane] + v[lane ^ 32] (the swap of a register with itself)
__device__ __forceinline__ float add_x16(float v) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float add_x32(float v) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float max_x16(float v) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float max_x32(float v) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}

// Sum over each aligned group of S lanes (S a power of two, wave-uniform), in every lane of the
// group, for NV values at once: xor 1 and xor 2 inside quads, then mirrors of groups that are
// already uniform.  Each step is one uniform branch over all values.
template <int NV>
__device__ __forceinline__ void group_sum(float* v, int S) {
    if (S >= 2)
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] += dpp<0xB1>(v[i]);  // quad_perm [1,0,3,2]
    if (S >= 4)
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] += dpp<0x4E>(v[i]);  // quad_perm [2,3,0,1]
    if (S >= 8)
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] += dpp<0x141>(v[i]);  // row_half_mirror
    if (S >= 16)
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] += dpp<0x140>(v[i]);  // row_mirror
    if (S >= 32)
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = add_x16(v[i]);
    if (S >= 64)
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = add_x32(v[i]);
}
// Sum over the lanes congruent modulo S (S a power of two, wave-uniform), in every lane, for NV
// values: rotations by S, 2S, .. 8 inside each 16-lane row, then across rows.
template <int NV>
__device__ __forceinline__ void stride_sum(float* v, int S) {
    if (S <= 1)
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] += dpp<0x121>(v[i]);  // row_ror:1
    if (S <= 2)
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] += dpp<0x122>(v[i]);  // row_ror:2
    if (S <= 4)
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] += dpp<0x124>(v[i]);  // row_ror:4
    if (S <= 8)
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] += dpp<0x128>(v[i]);  // row_ror:8
    if (S <= 16)
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = add_x16(v[i]);
    if (S <= 32)
#pragma unroll
        for (int i = 0; i < NV; ++i) v[i] = add_x32(v[i]);
}
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    v = max_x16(v);
    return max_x32(v);
}
__device__ __forceinline__ float wave_sum(float v) {
    group_sum<1>(&v, 64);
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

// Tokens of work group `tg` among the tokens that use one weight block: every token (rank0 is
// then their choice rank), or, for routed expert e of group g, the tokens that chose e, in
// ascending order (ballot compaction over the batch).  list[i] = token | rank << 24.  Returns the
// count (at most kTok, uniform over the work group); list is visible to the whole group.
__device__ int token_group(const DecArgs& a, bool routed, int e, int g, int rank0, int tg, int* list,
                           int* wcount) {
    const int tid = threadIdx.x, nw = blockDim.x >> 6;
    if (!routed) {
        int ntok = a.B - kTok * tg;
        ntok = ntok < kTok ? ntok : kTok;
        if (tid < ntok) list[tid] = (kTok * tg + tid) | (rank0 << 24);
        __syncthreads();
        return ntok;
    }
    const int w = tid >> 6;
    int base = 0;
    for (int b0 = 0; b0 < a.B; b0 += blockDim.x) {
        const int b = b0 + tid;
        int rank = -1;
        if (b < a.B) {
            const int32_t* id = a.idx + ((int64_t)b * a.G + g) * a.k;
            for (int r = 0; r < a.k; ++r)
                if (id[r] == e) rank = r;
        }
        const uint64_t m = __builtin_amdgcn_ballot_w64(rank >= 0);
        if ((tid & 63) == 0) wcount[w] = __builtin_popcountll(m);
        __syncthreads();
        int off = base, tot = 0;
        for (int i = 0; i < nw; ++i) {
            if (i < w) off += wcount[i];
            tot += wcount[i];
        }
        const int pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        const int slot = off + pre - kTok * tg;
        if (rank >= 0 && slot >= 0 && slot < kTok) list[slot] = b | (rank << 24);
        base += tot;
        __syncthreads();
    }
    const int ntok = base - kTok * tg;
    return ntok < 0 ? 0 : (ntok < kTok ? ntok : kTok);
}

__device__ __forceinline__ u32x4_t load16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// ---------------------------------------------------------------- projections of the new tokens
// Thread (unit u of the d_h columns, row slice rs): 16-byte units of the weight rows rs, rs + RS,
// ... (RS = 256 / UP slices, UP = units per row rounded up to a power of two) against the staged
// token rows; partial sums reduced over the slices by lane exchanges inside a wave, then across
// the four waves in LDS.
template <typename T, int RPT>
__global__ void __launch_bounds__(256) dec_proj_kernel(DecArgs a) {
    constexpr int E = 16 / (int)sizeof(T);
    __shared__ float xs[kTok][kDC];
    __shared__ float wacc[4][kTok][128];
    __shared__ int list[kTok];
    __shared__ int wcount[4];
    const int hb = blockIdx.x, tg = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int G = a.G, dh = a.dh, d = a.d;
    const int ebase = 2 * G + a.s;
    const bool is_exp = hb >= ebase;
    const int e = hb - ebase;
    const int g = is_exp ? e / a.n : (hb < G ? hb : hb - G);

    const T* W;
    int64_t rstride;
    if (hb < G) {
        W = (const T*)a.wk + hb * dh;
        rstride = (int64_t)G * dh;
    } else if (hb < 2 * G) {
        W = (const T*)a.wv + (hb - G) * dh;
        rstride = (int64_t)G * dh;
    } else if (!is_exp) {
        W = (const T*)a.wqs;
        rstride = dh;
    } else {
        W = (const T*)a.wq + (int64_t)e * d * dh;
        rstride = dh;
    }
    const int U = dh / E;
    const int UP = a.up, RS = 256 / UP;
    const int CH = RS * RPT;  // rows per chunk (the launcher keeps it <= kDC)
    const int u = tid & (UP - 1), rs = tid / UP;
    const bool uact = u < U;
    const T* wbase = W + (uact ? u * E : 0);
    // the weight rows of a chunk: all loads issued at once (rows past the end repeat the last)
    u32x4_t wv[RPT];
    auto issue = [&](int c0) {
        const int nc = d - c0 < CH ? d - c0 : CH;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            int i = rs + RS * r;
            i = i < nc ? i : nc - 1;
            wv[r] = load16(wbase + (int64_t)(c0 + i) * rstride);
        }
    };
    issue(0);  // independent of the tokens: in flight during the token selection
    const int ntok = token_group(a, is_exp && !a.dense, e, g, is_exp ? e % a.n : 0, tg, list, wcount);
    if (ntok <= 0) return;  // uniform over the work group

    float acc[kTok][E];
#pragma unroll
    for (int t = 0; t < kTok; ++t)
#pragma unroll
        for (int i = 0; i < E; ++i) acc[t][i] = 0.f;
    const T* X = (const T*)a.x;
    for (int c0 = 0; c0 < d; c0 += CH) {
        const int nc = d - c0 < CH ? d - c0 : CH;
        // the chunk of the token rows, 16 bytes per load (d is a multiple of E), every load of the
        // thread issued before the first is used: one memory round trip per chunk
        constexpr int NV = kTok * kDC / E / 256;
        const int vr = CH / E;  // 16-byte units per staged row
        u32x4_t xv[NV];
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int i = tid + 256 * j;
            const int t = i / vr, c = (i - t * vr) * E;
            xv[j] = u32x4_t{0u, 0u, 0u, 0u};
            if (t < ntok && c < nc) xv[j] = load16(X + (int64_t)(list[t] & 0xffffff) * d + c0 + c);
        }
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int i = tid + 256 * j;
            const int t = i / vr, c = (i - t * vr) * E;
            if (t >= kTok) continue;
            float f[E];
            widen16(xv[j], f);
#pragma unroll
            for (int q = 0; q < E; ++q) xs[t][c + q] = f[q];  // zero past the tokens and the chunk
        }
        __syncthreads();
        if (uact) {
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const int i = rs + RS * r;  // rows past nc meet zero token values
                float f[E];
                widen16(wv[r], f);
#pragma unroll
                for (int t = 0; t < kTok; ++t) {
                    const float xv = xs[t][i];
#pragma unroll
                    for (int q = 0; q < E; ++q) acc[t][q] += xv * f[q];
                }
            }
        }
        __syncthreads();
        if (c0 + CH < d) issue(c0 + CH);
    }
    // sum over the row slices: inside the wave (lanes u, u + UP, ...), then over the waves
    stride_sum<kTok * E>(&acc[0][0], UP);
    if (lane < UP && uact)
#pragma unroll
        for (int t = 0; t < kTok; ++t)
#pragma unroll
            for (int q = 0; q < E; ++q) wacc[w][t][u * E + q] = acc[t][q];
    __syncthreads();
    const bool rot = a.rope != nullptr && (hb < G || hb >= 2 * G);  // queries and keys
    for (int o = tid; o < ntok * dh; o += 256) {
        const int t = o / dh, jj = o - t * dh;
        float v = (wacc[0][t][jj] + wacc[1][t][jj]) + (wacc[2][t][jj] + wacc[3][t][jj]);
        const int tk = list[t];
        const int b = tk & 0xffffff, rank = tk >> 24;
        if (rot) {
            const int jp = jj ^ 1;  // pair partner
            const float vp = (wacc[0][t][jp] + wacc[1][t][jp]) + (wacc[2][t][jp] + wacc[3][t][jp]);
            float lo = (jj & 1) ? vp : v, hi = (jj & 1) ? v : vp;
            rope_pair(lo, hi, a.pos[b], a.rope[jj >> 1]);
            v = (jj & 1) ? hi : lo;
        }
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
// Thread (unit u, key group kg): the 16-byte units u of keys kg, kg + KG, ... (KG = 256 / UP key
// groups, KPT keys each) of K and of V, all loaded up front.  Scores: partial dot products over
// the unit, summed over the UP lanes of a key by lane exchanges; softmax over the chunk; P.V:
// each lane scales its V units by its keys' probabilities, summed over the key groups (lane
// exchanges, then LDS across the waves).  MH bounds the active heads of a group.
template <typename T, int MH>
__global__ void __launch_bounds__(256) dec_attn_kernel(DecArgs a) {
    constexpr int E = 16 / (int)sizeof(T);
    constexpr int KPT = kKeysPerThread;
    __shared__ float wred[4][MH];
    __shared__ float osum[4][MH][128];
    const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int p = a.pos[b];
    if (!pos_ok(p, a.s_max)) return;
    const int64_t L = (int64_t)p + 1, c0 = (int64_t)chunk * a.C;
    if (c0 >= L) return;
    const int nk = (int)(L - c0 < a.C ? L - c0 : a.C);
    const int dh = a.dh, G = a.G;
    const int kr = a.dense ? a.n : a.k;
    const int m = kr + ((a.s && g == a.skv) ? 1 : 0);
    const int U = dh / E, UP = a.up, KG = 256 / UP;
    const int u = tid & (UP - 1), kg = tid / UP;
    const bool uact = u < U;
    const int64_t row0 = ((int64_t)b * G + g) * a.s_max + c0;
    const T* kb = (const T*)a.kc + row0 * dh + u * E;
    const T* vb = (const T*)a.vc + row0 * dh + u * E;
    // every lane loads (past the chunk or the row: a valid key's unit, then zeroed): no branches
    u32x4_t kv[KPT], vv[KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        const int i = kg + KG * r;
        const int64_t off = (int64_t)(i < nk ? i : nk - 1) * dh - (uact ? 0 : u * E);
        kv[r] = load16(kb + off);
        vv[r] = load16(vb + off);
    }
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        if (!uact || kg + KG * r >= nk) {
            kv[r] = u32x4_t{0u, 0u, 0u, 0u};
            vv[r] = u32x4_t{0u, 0u, 0u, 0u};
        }
    }
    float q[MH][E];
#pragma unroll
    for (int h = 0; h < MH; ++h) {
        const int hid = h < m ? (h < kr ? g * kr + h : G * kr) : 0;
        const f32x4_t* qp = reinterpret_cast<const f32x4_t*>(a.qd + ((int64_t)b * a.H + hid) * dh + (uact ? u * E : 0));
#pragma unroll
        for (int i = 0; i < E; i += 4) {
            const f32x4_t v = qp[i / 4];
#pragma unroll
            for (int z = 0; z < 4; ++z) q[h][i + z] = (h < m && uact) ? v[z] : 0.f;
        }
    }
    // scores (log2 units: the queries carry log2(e)/sqrt(d_h))
    float sc[MH][KPT];
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        float f[E];
        widen16(kv[r], f);
#pragma unroll
        for (int h = 0; h < MH; ++h) {
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < E; ++i) s += q[h][i] * f[i];
            sc[h][r] = s;
        }
    }
    group_sum<MH * KPT>(&sc[0][0], UP);
    float mx[MH];
#pragma unroll
    for (int h = 0; h < MH; ++h) {
        float v = -INFINITY;
#pragma unroll
        for (int r = 0; r < KPT; ++r)
            if (kg + KG * r < nk) v = fmaxf(v, sc[h][r]);
        v = wave_max(v);
        if (lane == 0) wred[w][h] = v;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < MH; ++h) mx[h] = fmaxf(fmaxf(wred[0][h], wred[1][h]), fmaxf(wred[2][h], wred[3][h]));
    __syncthreads();
    float ls[MH];
#pragma unroll
    for (int h = 0; h < MH; ++h) {
        float l = 0.f;
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
            const float pr = (h < m && kg + KG * r < nk) ? __builtin_amdgcn_exp2f(sc[h][r] - mx[h]) : 0.f;
            sc[h][r] = pr;
            l += pr;
        }
        l = wave_sum(u == 0 ? l : 0.f);  // one lane per key
        if (lane == 0) wred[w][h] = l;
    }
    // P.V over my keys
    float o[MH][E];
#pragma unroll
    for (int h = 0; h < MH; ++h)
#pragma unroll
        for (int i = 0; i < E; ++i) o[h][i] = 0.f;
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
        float f[E];
        widen16(vv[r], f);
#pragma unroll
        for (int h = 0; h < MH; ++h)
#pragma unroll
            for (int i = 0; i < E; ++i) o[h][i] += sc[h][r] * f[i];
    }
    stride_sum<MH * E>(&o[0][0], UP);
    if (lane < UP && uact)
#pragma unroll
        for (int h = 0; h < MH; ++h)
#pragma unroll
            for (int i = 0; i < E; ++i) osum[w][h][u * E + i] = o[h][i];
    __syncthreads();
#pragma unroll
    for (int h = 0; h < MH; ++h) ls[h] = (wred[0][h] + wred[1][h]) + (wred[2][h] + wred[3][h]);
    float* dst = a.part + ((((int64_t)b * G + g) * a.NC + chunk) * a.MH) * (dh + 2);
    for (int i = tid; i < m * dh; i += 256) {
        const int h = i / dh, jj = i - h * dh;
        dst[h * (dh + 2) + jj] = (osum[0][h][jj] + osum[1][h][jj]) + (osum[2][h][jj] + osum[3][h][jj]);
    }
    if (tid < m) {
        float mv = mx[0], lv = ls[0];
#pragma unroll
        for (int h = 1; h < MH; ++h)
            if (tid == h) {
                mv = mx[h];
                lv = ls[h];
            }
        dst[tid * (dh + 2) + dh] = mv;
        dst[tid * (dh + 2) + dh + 1] = lv;
    }
}

// ---------------------------------------------------------------- merge of the chunk partials
// One wave per (token, head): chunk weights 2^(m_c - M) / l from the lanes (64 chunks at a time),
// then every lane sums its head dims over those chunks.
__global__ void __launch_bounds__(64) dec_merge_kernel(DecArgs a) {
    __shared__ float scl[64];
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
    // the lane's first chunk's (m, l), loaded together and kept: with at most 64 chunks (every
    // cache up to 64 C positions) nothing is read twice
    const float m0 = lane < nch ? base[lane * cs + dh] : -INFINITY;
    const float l0 = lane < nch ? base[lane * cs + dh + 1] : 0.f;
    float M = m0;
    for (int c = lane + 64; c < nch; c += 64) M = fmaxf(M, base[c * cs + dh]);
    M = wave_max(M);
    const float e0 = lane < nch ? __builtin_amdgcn_exp2f(m0 - M) : 0.f;
    float l = l0 * e0;
    for (int c = lane + 64; c < nch; c += 64) l += base[c * cs + dh + 1] * __builtin_amdgcn_exp2f(base[c * cs + dh] - M);
    const float inv = 1.f / wave_sum(l);
    float o0 = 0.f, o1 = 0.f;
    for (int cb = 0; cb < nch; cb += 64) {
        const int c = cb + lane;
        scl[lane] = cb == 0 ? e0 * inv : (c < nch ? __builtin_amdgcn_exp2f(base[c * cs + dh] - M) * inv : 0.f);
        __syncthreads();
        const int n = nch - cb < 64 ? nch - cb : 64;
        const float* pc = base + cb * cs;
        if (lane < dh) {
#pragma unroll 16
            for (int i = 0; i < n; ++i) o0 += pc[i * cs + lane] * scl[i];
        }
        if (lane + 64 < dh) {
#pragma unroll 16
            for (int i = 0; i < n; ++i) o1 += pc[i * cs + lane + 64] * scl[i];
        }
        __syncthreads();
    }
    if (lane < dh) out[lane] = o0;
    if (lane + 64 < dh) out[lane + 64] = o1;
}

// ---------------------------------------------------------------- output projection per weight slot
// Work group (four waves) = (weight slot, up to 8 tokens that use it, 64 column units of 16 bytes):
// slot = W_o of routed expert e (the tokens that chose it), W_oR of group g (variant gqe) or the
// shared head's W_os (every token).  Each token's slot vector (its head output, times the
// raw router probability for weighted_concat; the renormalised mix sum_r w_r o_r for W_oR) times the
// slot's d_h x d block, each weight row read once for the group of tokens: the waves take the
// 12-row batches of the block round-robin, and their partial sums meet in LDS in wave order.  Writes
// the token's float32 partial row of that slot; dec_ysum_kernel adds a token's slots in a fixed
// order.
template <typename T>
__global__ void __launch_bounds__(256) dec_oproj_kernel(DecArgs a) {
    constexpr int E = 16 / (int)sizeof(T);
    constexpr int NWV = 4;  // waves
    __shared__ __align__(16) float vs[kTok][128 + kOprojRows];
    __shared__ __align__(16) float red[NWV][kTok][64 * E];  // the waves' partial sums
    __shared__ int list[kTok];
    __shared__ int wcount[NWV];
    const int sm = blockIdx.x, tg = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = a.G, dh = a.dh, d = a.d;
    const int kr = a.dense ? a.n : a.k;
    const bool rslot = !a.dense && a.variant == GQE_VARIANT_GQE;
    const int nr = G * kr;
    int kind, g = 0, e = 0;  // 0 routed expert, 1 renormalised slot, 2 shared head
    if (sm < a.N) {
        kind = 0;
        e = sm;
        g = e / a.n;
    } else if (rslot && sm < a.N + G) {
        kind = 1;
        g = sm - a.N;
    } else {
        kind = 2;
    }
    const int cu = blockIdx.z * 64 + lane;  // column unit
    const bool cact = cu * E < d;
    const T* W = kind == 0 ? (const T*)a.wo + (int64_t)e * dh * d
                           : (kind == 1 ? (const T*)a.wor + (int64_t)g * dh * d : (const T*)a.wos);
    const T* wp = W + (cact ? cu * E : 0);
    // weight rows in batches of kOprojRows, batch b taken by wave b % 4, a wave's next batch in
    // flight while one is used; its first is issued before the token selection (rows past d_h
    // repeat the last; they meet zero slot values)
    constexpr int RB = kOprojRows;
    const int nb = (dh + RB - 1) / RB;
    u32x4_t wv[2][RB];
    auto issue = [&](int buf, int j0) {
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const int j = j0 + i < dh ? j0 + i : dh - 1;
            wv[buf][i] = load16(wp + (int64_t)j * d);
        }
    };
    if (w < nb) issue(0, w * RB);
    const int ntok = token_group(a, kind == 0 && !a.dense, e, g, kind == 0 ? e % a.n : 0, tg, list, wcount);
    if (ntok <= 0) return;
    constexpr int VW = 128 + kOprojRows;  // slot vector row (zero past d_h)
    static_assert(VW % 4 == 0, "float4 units");
    // the slot vectors in float4 units (d_h is a multiple of 4), lane i taking units i, i + 64, ...;
    // every load of a lane is issued before the first is used (the renormalised slot: once per
    // choice rank), so the staging costs one memory round trip instead of one per element
    constexpr int VU = VW / 4, NI = (kTok * VU + 64 * NWV - 1) / (64 * NWV);
    const bool wc = !a.dense && a.variant == GQE_VARIANT_WEIGHTED_CONCAT;
    f32x4_t vv[NI];
    const float* orow[NI];  // the unit's source in the token's head outputs (null: zero)
    int64_t selr[NI];       // the token's routing entries
    int rk[NI];
#pragma unroll
    for (int n = 0; n < NI; ++n) {
        const int i = tid + 64 * NWV * n, t = i / VU, j = (i - t * VU) * 4;
        vv[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        orow[n] = nullptr;
        selr[n] = 0;
        rk[n] = 0;
        if (t < ntok && j < dh) {
            const int tk = list[t];
            const int b = tk & 0xffffff;
            rk[n] = tk >> 24;
            selr[n] = ((int64_t)b * G + g) * a.k;
            orow[n] = a.od + (int64_t)b * a.H * dh + j;
        }
    }
    if (kind == 1) {
        for (int q = 0; q < a.k; ++q) {
            f32x4_t ov[NI];
            float wq[NI];
#pragma unroll
            for (int n = 0; n < NI; ++n) {
                ov[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                wq[n] = 0.f;
                if (orow[n]) {
                    ov[n] = *reinterpret_cast<const f32x4_t*>(orow[n] + (g * a.k + q) * dh);
                    wq[n] = a.wsel[selr[n] + q];
                }
            }
#pragma unroll
            for (int n = 0; n < NI; ++n) vv[n] += wq[n] * ov[n];
        }
    } else {
        float cf[NI];
#pragma unroll
        for (int n = 0; n < NI; ++n) {
            cf[n] = 1.f;
            if (orow[n]) {
                vv[n] = *reinterpret_cast<const f32x4_t*>(orow[n] + (kind == 0 ? (g * kr + rk[n]) * dh : nr * dh));
                if (kind == 0 && wc) cf[n] = a.psel[selr[n] + rk[n]];
            }
        }
#pragma unroll
        for (int n = 0; n < NI; ++n)
            if (kind == 0 && wc) vv[n] *= cf[n];
    }
#pragma unroll
    for (int n = 0; n < NI; ++n) {
        const int i = tid + 64 * NWV * n, t = i / VU, j = (i - t * VU) * 4;
        if (t < kTok) *reinterpret_cast<f32x4_t*>(&vs[t][j]) = vv[n];  // zero past d_h and the tokens
    }
    __syncthreads();
    float acc[kTok][E];
#pragma unroll
    for (int t = 0; t < kTok; ++t)
#pragma unroll
        for (int q = 0; q < E; ++q) acc[t][q] = 0.f;
    auto use = [&](const u32x4_t (&wb)[RB], int j0) {
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            float f[E];
            widen16(wb[i], f);
#pragma unroll
            for (int t = 0; t < kTok; ++t) {
                const float x = vs[t][j0 + i];
#pragma unroll
                for (int q = 0; q < E; ++q) acc[t][q] += x * f[q];
            }
        }
    };
    for (int b = w; b < nb; b += 2 * NWV) {
        if (b + NWV < nb) issue(1, (b + NWV) * RB);
        use(wv[0], b * RB);
        if (b + 2 * NWV < nb) issue(0, (b + 2 * NWV) * RB);
        if (b + NWV < nb) use(wv[1], (b + NWV) * RB);
    }
    // partial sums through LDS; wave w then adds the four partials (in wave order) of tokens
    // 2 w and 2 w + 1 and writes them
#pragma unroll
    for (int t = 0; t < kTok; ++t)
#pragma unroll
        for (int q = 0; q < E; q += 4)
            *reinterpret_cast<f32x4_t*>(&red[w][t][lane * E + q]) =
                f32x4_t{acc[t][q], acc[t][q + 1], acc[t][q + 2], acc[t][q + 3]};
    __syncthreads();
    static_assert(kTok == 2 * NWV, "two tokens per wave");
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int t = 2 * w + h;
        if (t >= ntok || !cact) continue;
        const int tk = list[t];
        const int b = tk & 0xffffff, r = tk >> 24;
        const int ls = kind == 0 ? g * kr + r : (kind == 1 ? nr + g : nr + (rslot ? G : 0));
        float* dst = a.yp + ((int64_t)b * a.NS + ls) * d + cu * E;
#pragma unroll
        for (int q = 0; q < E; q += 4) {
            f32x4_t v = *reinterpret_cast<const f32x4_t*>(&red[0][t][lane * E + q]);
#pragma unroll
            for (int p = 1; p < NWV; ++p) v += *reinterpret_cast<const f32x4_t*>(&red[p][t][lane * E + q]);
            *reinterpret_cast<f32x4_t*>(dst + q) = v;
        }
    }
}

// y[b, :] = sum of the token's slot rows, in slot order (deterministic).
template <typename T>
__global__ void __launch_bounds__(256) dec_ysum_kernel(DecArgs a) {
    const int b = blockIdx.y;
    const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= a.d) return;
    T* y = (T*)a.y + (int64_t)b * a.d + c;
    if (!pos_ok(a.pos[b], a.s_max)) {
        for (int z = 0; z < 4; ++z) y[z] = from_f32<T>(__builtin_nanf(""));
        return;
    }
    const int kr = a.dense ? a.n : a.k;
    const int nslot = a.G * kr + ((!a.dense && a.variant == GQE_VARIANT_GQE) ? a.G : 0) + a.s;
    const float* src = a.yp + (int64_t)b * a.NS * a.d + c;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int sl = 0; sl < nslot; ++sl) acc += *reinterpret_cast<const f32x4_t*>(src + (int64_t)sl * a.d);
    for (int z = 0; z < 4; ++z) y[z] = from_f32<T>(acc[z]);
}

}  // namespace

int decode_units(const GqeDims& D) {
    const int u = D.dh * (D.dtype == GQE_DTYPE_BF16 ? 2 : 4) / 16;
    int up = 1;
    while (up < u) up <<= 1;
    return up;
}

int decode_chunk(const GqeDims& D) { return 256 / decode_units(D) * kKeysPerThread; }

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

hipError_t launch_decode(const GqeDims& D, const DecodePlan& P, const gqe_weights_t& w, const double* rope,
                         const void* x, void* y, const int32_t* pos, void* kc, void* vc, char* ws, hipStream_t st,
                         KernelMarks* km) {
    DecArgs a{};
    a.rope = D.rope > 0.f ? rope : nullptr;
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
    a.yp = (float*)(ws + P.yp);
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
    a.NS = P.NS;
    a.up = decode_units(D);
    a.qscale = (float)(1.4426950408889634 / std::sqrt((double)D.dh));
    const bool bf = D.dtype == GQE_DTYPE_BF16;
    const unsigned tgroups = (unsigned)ceil_div(P.B, kTok);
    hipError_t e;
    // projections of the new tokens (K/V into the cache)
    if (km) km->begin(KT_DEC_PROJ);
    // weight rows per thread and chunk, all loaded at once: 24 (a chunk of 768 rows) with 8 or more
    // units per d_h row, fewer with fewer units so that the staged chunk stays within kDC rows
    const dim3 gp((unsigned)(2 * D.G + D.s + D.N), tgroups);
#define GQE_DEC_PROJ(R)                                             \
    if (bf) dec_proj_kernel<bf16_t, R><<<gp, 256, 0, st>>>(a);     \
    else dec_proj_kernel<float, R><<<gp, 256, 0, st>>>(a);
    if (a.up >= 8) { GQE_DEC_PROJ(24) }
    else if (a.up == 4) { GQE_DEC_PROJ(16) }
    else if (a.up == 2) { GQE_DEC_PROJ(8) }
    else { GQE_DEC_PROJ(4) }
#undef GQE_DEC_PROJ
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (km) km->mark(KT_DEC_PROJ);
    // attention over the cache chunks, then the merge
    if (km) km->begin(KT_DEC_ATTN);
    const dim3 ga((unsigned)P.NC, (unsigned)D.G, (unsigned)P.B);
#define GQE_DEC_ATTN(MHV)                                            \
    if (bf) dec_attn_kernel<bf16_t, MHV><<<ga, 256, 0, st>>>(a);    \
    else dec_attn_kernel<float, MHV><<<ga, 256, 0, st>>>(a);
    if (P.MH <= 1) { GQE_DEC_ATTN(1) }
    else if (P.MH <= 2) { GQE_DEC_ATTN(2) }
    else if (P.MH <= 4) { GQE_DEC_ATTN(4) }
    else { GQE_DEC_ATTN(8) }
#undef GQE_DEC_ATTN
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (km) km->mark(KT_DEC_ATTN);
    if (km) km->begin(KT_DEC_MERGE);
    dec_merge_kernel<<<dim3((unsigned)D.H, (unsigned)P.B), 64, 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (km) km->mark(KT_DEC_MERGE);
    // output construction + output projection: per weight slot, then the per-token sum
    if (km) km->begin(KT_DEC_COMBINE);
    const int E = bf ? 8 : 4;
    const unsigned nsm = (unsigned)(D.N + ((!D.dense && D.variant == GQE_VARIANT_GQE) ? D.G : 0) + D.s);
    const dim3 go(nsm, tgroups, (unsigned)ceil_div(D.d / E, 64));
    if (bf) dec_oproj_kernel<bf16_t><<<go, 256, 0, st>>>(a);
    else dec_oproj_kernel<float><<<go, 256, 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 gy((unsigned)ceil_div(D.d / 4, 256), (unsigned)P.B);
    if (bf) dec_ysum_kernel<bf16_t><<<gy, 256, 0, st>>>(a);
    else dec_ysum_kernel<float><<<gy, 256, 0, st>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (km) km->mark(KT_DEC_COMBINE);
    return hipSuccess;
}
