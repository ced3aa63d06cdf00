// Router of the GQE layer (gfx950): logits, in-group softmax, top-k, renormalised weights and the
// per-expert statistics of the Switch-style balance loss.
//
// GQE README "Algorithm Overview": softmax over the experts inside each GQA group, then top-k;
// a Switch-style load-balancing auxiliary loss.  Tutorial "Mixture of experts (MoE)": the router
// scores are x @ router_w; the chosen experts are mixed by renormalised router weights.
//
// Precision: the routing decision is an integer result decided by floating point, so the logits
// are accumulated in float64 (fp64 FMA is full rate on gfx950); the selection compares float64
// logits (softmax is monotone, so top-k of the logits is top-k of the probabilities).  Equal
// logits resolve to the lower local index.
#include "gqe_common.h"
#include "gqe_internal.h"

namespace {

constexpr int kTok = 64;     // tokens per block (one per lane)
constexpr int kEChunk = 16;  // experts accumulated per pass over x

template <typename Tin>
__device__ __forceinline__ void load8(const Tin* p, double* v);
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, double* v) {
    const u32x4_t q = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = (double)__uint_as_float(q[i] << 16);
        v[2 * i + 1] = (double)__uint_as_float(q[i] & 0xffff0000u);
    }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, double* v) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = (double)a[i];
        v[4 + i] = (double)b[i];
    }
}

// Block: 256 threads = 4 waves; 64 tokens (lane = token); wave w accumulates the w-th quarter of
// the hidden dimension, the four partial sums are added in a fixed order.
template <typename Tin, bool kVec>
__global__ void __launch_bounds__(256) router_kernel(
    const Tin* __restrict__ x, const double* __restrict__ wr, const double* __restrict__ br,
    int64_t T, int d, int N, int G, int k, int32_t* __restrict__ idx, float* __restrict__ wsel,
    float* __restrict__ psel, int32_t* __restrict__ ridx, float* __restrict__ rw,
    int32_t* __restrict__ part_cnt, double* __restrict__ part_psum) {
    __shared__ double red[4][kTok][kEChunk + 1];
    __shared__ double lg[kTok][65];
    __shared__ int cnt[64];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t0 = (int64_t)blockIdx.x * kTok;
    const int64_t t = t0 + lane;
    const bool valid = t < T;
    const int n = N / G;
    if (threadIdx.x < 64) cnt[threadIdx.x] = 0;

    const int dq = kVec ? d / 4 : (d + 3) / 4;
    const int i0 = min(d, wv * dq), i1 = min(d, i0 + dq);
    const Tin* xr = x + (valid ? t : (int64_t)0) * d;

    for (int e0 = 0; e0 < N; e0 += kEChunk) {
        double acc[kEChunk];
#pragma unroll
        for (int j = 0; j < kEChunk; ++j) acc[j] = 0.0;
        if (kVec) {
            for (int i = i0; i < i1; i += 8) {
                double xv[8];
                load8<Tin>(xr + i, xv);
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const double* wrow = wr + (size_t)(i + u) * N + e0;
#pragma unroll
                    for (int j = 0; j < kEChunk; ++j)
                        if (e0 + j < N) acc[j] = __builtin_fma(xv[u], wrow[j], acc[j]);
                }
            }
        } else {
            for (int i = i0; i < i1; ++i) {
                const double xv = (double)to_f32(xr[i]);
                const double* wrow = wr + (size_t)i * N + e0;
#pragma unroll
                for (int j = 0; j < kEChunk; ++j)
                    if (e0 + j < N) acc[j] = __builtin_fma(xv, wrow[j], acc[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < kEChunk; ++j) red[wv][lane][j] = acc[j];
        __syncthreads();
        for (int q = threadIdx.x; q < kTok * kEChunk; q += 256) {
            const int tok = q / kEChunk, j = q % kEChunk;
            if (e0 + j < N)
                lg[tok][e0 + j] = ((red[0][tok][j] + red[1][tok][j]) + red[2][tok][j]) + red[3][tok][j] +
                                  (br ? br[e0 + j] : 0.0);
        }
        __syncthreads();
    }

    // one (token, group) pair per thread: softmax, top-k, renormalised weights
    for (int q = threadIdx.x; q < kTok * G; q += 256) {
        const int tok = q / G, g = q % G;
        const int64_t tt = t0 + tok;
        if (tt >= T) continue;
        const double* l = &lg[tok][g * n];
        double m = l[0];
        for (int j = 1; j < n; ++j) m = fmax(m, l[j]);
        double den = 0.0;
        for (int j = 0; j < n; ++j) den += exp(l[j] - m);
        uint64_t taken = 0;
        double ps = 0.0;
        for (int r = 0; r < k; ++r) {
            int best = -1;
            for (int j = 0; j < n; ++j)
                if (!((taken >> j) & 1) && (best < 0 || l[j] > l[best])) best = j;
            taken |= (uint64_t)1 << best;
            ps += exp(l[best] - m) / den;
        }
        taken = 0;
        const int64_t o = (tt * G + g) * k;
        for (int r = 0; r < k; ++r) {
            int best = -1;
            for (int j = 0; j < n; ++j)
                if (!((taken >> j) & 1) && (best < 0 || l[j] > l[best])) best = j;
            taken |= (uint64_t)1 << best;
            const double p = exp(l[best] - m) / den;
            const int e = g * n + best;
            idx[o + r] = e;
            wsel[o + r] = (float)(p / ps);
            psel[o + r] = (float)p;
            if (ridx) ridx[o + r] = e;
            if (rw) rw[o + r] = (float)(p / ps);
            atomicAdd(&cnt[e], 1);
        }
        // keep the probabilities for the statistics (only this thread touches group g of tok)
        for (int j = 0; j < n; ++j) {
            const double pj = exp(l[j] - m) / den;
            lg[tok][g * n + j] = pj;
        }
    }
    __syncthreads();
    if (threadIdx.x < N) {
        const int e = threadIdx.x;
        double s = 0.0;
        for (int tok = 0; tok < kTok; ++tok)
            if (t0 + tok < T) s += lg[tok][e];
        part_psum[(int64_t)blockIdx.x * N + e] = s;
        part_cnt[(int64_t)blockIdx.x * N + e] = cnt[e];
    }
}

// Sums the per-block partials in block order (deterministic) and forms the balance loss.
__global__ void __launch_bounds__(256) stats_finalize_kernel(const int32_t* __restrict__ part_cnt,
                                                             const double* __restrict__ part_psum,
                                                             int64_t nblk, int64_t T, int N, int G,
                                                             int k, char* __restrict__ stats) {
    __shared__ double fp[64];
    int64_t* counts = reinterpret_cast<int64_t*>(stats);
    double* mean = reinterpret_cast<double*>(stats + 8 * N);
    double* aux = reinterpret_cast<double*>(stats + 16 * N);
    const int e = threadIdx.x;
    if (e < N) {
        int64_t c = 0;
        double s = 0.0;
        for (int64_t b = 0; b < nblk; ++b) {
            c += part_cnt[b * N + e];
            s += part_psum[b * N + e];
        }
        counts[e] = c;
        const double P = s / (double)T;
        mean[e] = P;
        fp[e] = ((double)c / ((double)T * (double)k)) * P;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int n = N / G;
        double tot = 0.0;
        for (int g = 0; g < G; ++g) {
            double Lg = 0.0;
            for (int j = 0; j < n; ++j) Lg += fp[g * n + j];
            tot += (double)n * Lg;
        }
        *aux = tot / (double)G;
    }
}

}  // namespace

hipError_t launch_router(const GqeDims& D, const WorkPlan& P, const void* x, const void* packed,
                         const PackedLayout& pl, char* ws, int32_t* route_idx, float* route_w,
                         hipStream_t st) {
    const char* pk = (const char*)packed;
    const double* wr = (const double*)(pk + pl.wr64);
    const double* br = (const double*)(pk + pl.br64);
    int32_t* idx = (int32_t*)(ws + P.idx);
    float* wsel = (float*)(ws + P.wsel);
    float* psel = (float*)(ws + P.psel);
    int32_t* pc = (int32_t*)(ws + P.part_cnt);
    double* pp = (double*)(ws + P.part_psum);
    const dim3 grid((unsigned)P.nblk_router);
    const bool vec = D.d % 32 == 0;
    if (D.dtype == GQE_DTYPE_BF16) {
        if (vec)
            router_kernel<bf16_t, true><<<grid, 256, 0, st>>>((const bf16_t*)x, wr, br, P.T, D.d, D.N, D.G, D.k,
                                                               idx, wsel, psel, route_idx, route_w, pc, pp);
        else
            router_kernel<bf16_t, false><<<grid, 256, 0, st>>>((const bf16_t*)x, wr, br, P.T, D.d, D.N, D.G, D.k,
                                                                idx, wsel, psel, route_idx, route_w, pc, pp);
    } else {
        if (vec)
            router_kernel<float, true><<<grid, 256, 0, st>>>((const float*)x, wr, br, P.T, D.d, D.N, D.G, D.k,
                                                              idx, wsel, psel, route_idx, route_w, pc, pp);
        else
            router_kernel<float, false><<<grid, 256, 0, st>>>((const float*)x, wr, br, P.T, D.d, D.N, D.G, D.k,
                                                               idx, wsel, psel, route_idx, route_w, pc, pp);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    stats_finalize_kernel<<<1, 256, 0, st>>>(pc, pp, P.nblk_router, P.T, D.N, D.G, D.k, ws + P.stats);
    return hipGetLastError();
}
