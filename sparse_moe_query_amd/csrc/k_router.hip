// Router of the GQE layer (gfx950): logits, in-group softmax, top-k, renormalised weights and the
// per-expert statistics of the Switch-style balance loss.
//
// GQE README "Algorithm Overview": softmax over the experts inside each GQA group, then top-k;
// a Switch-style load-balancing auxiliary loss.  Tutorial "Mixture of experts (MoE)": the router
// scores are x @ router_w; the chosen experts are mixed by renormalised router weights.
//
// The routing decision is an integer result decided by floating point, so the logits are summed
// in float64; top-k compares the float64 logits (softmax is monotone) and equal logits resolve to
// the lower local index.
//
// Fast path (d % 64 == 0, N <= 16): v_mfma_f64_16x16x4_f64 (full-rate fp64 on gfx950).  A block
// owns 64 tokens; wave w of 8 (two per SIMD, so one wave's conversions overlap the other's
// products) sums the w-th eighth of the hidden dimension for all of them, its x and weight loads
// issued three 32-wide chunks at a time ahead of the products.  Each lane
// loads eight consecutive hidden values of one token with one 16-byte load; the k index of the
// MFMA is permuted accordingly (k-step s of lane group q covers hidden index 8q + s), and the
// router weights are pre-permuted into exactly that lane order ([octet of 8 hidden indices]
// [column][8], by gqe_pack_weights), so the B operands are 64 contiguous bytes per lane.  The
// eight partial sums are added in a fixed order (103 KB of LDS: one block per CU).
// Generic path (any d, N <= 64): one token per lane, float64 FMAs with the weights as wave-uniform
// scalar operands.
#include "gqe_common.h"
#include "gqe_internal.h"
#include "gqe_stats.h"

namespace {

constexpr int kTok = 64;  // tokens per block

typedef double f64x4_t __attribute__((ext_vector_type(4)));
// Read-only, wave-uniform weights: the constant address space lets them come through the scalar
// cache as SGPR operands.
typedef const __attribute__((address_space(4))) double* const_f64_ptr;

struct RouterArgs {
    const void* x;
    const double* wr;    // generic: [d][Np] zero padded; fast: lane-ordered blocks
    const double* br;    // [N]
    int64_t T;
    int d, N, G, k, n, Np;  // Np = N rounded up to 16
    int32_t* idx;
    float* wsel;
    float* psel;
    float* probs;  // [T][N] every expert's in-group probability, or null
    int32_t* ridx;
    float* rw;
    int32_t* part_cnt;
    double* part_psum;
};

template <typename Tin>
__device__ __forceinline__ void widen8(const Tin* p, double* v);
template <>
__device__ __forceinline__ void widen8<bf16_t>(const bf16_t* p, double* v) {
    const u32x4_t q = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = (double)__uint_as_float(q[i] << 16);
        v[2 * i + 1] = (double)__uint_as_float(q[i] & 0xffff0000u);
    }
}
template <>
__device__ __forceinline__ void widen8<float>(const float* p, double* v) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = (double)a[i];
        v[4 + i] = (double)b[i];
    }
}

// Softmax, top-k and weights for the block's tokens; logits in lg[tok][e] (bias included).
// The selection compares the float64 logits; the probabilities are formed from the float64
// differences l - max with the float32 exponential (relative error ~1e-7), and overwrite the
// logits of the same (token, group).  Per-block statistics follow.
// The decision of one (token tt, group g) on the group's n logits l (overwritten with the
// probabilities); counts the choice in cnt when given.
__device__ void select_one(const RouterArgs& a, double* l, int64_t tt, int g, int* cnt) {
    const int n = a.n, k = a.k;
    double m = l[0];
    for (int j = 1; j < n; ++j) m = fmax(m, l[j]);
    uint64_t taken = 0, sel = 0;  // sel: 4 bits per rank (n <= 16)
    for (int r = 0; r < k; ++r) {
        int best = -1;
        for (int j = 0; j < n; ++j)
            if (!((taken >> j) & 1) && (best < 0 || l[j] > l[best])) best = j;
        taken |= (uint64_t)1 << best;
        sel |= (uint64_t)best << (4 * r);
    }
    float den = 0.f;
    for (int j = 0; j < n; ++j) den += expf((float)(l[j] - m));
    const float inv = 1.0f / den;
    for (int j = 0; j < n; ++j) l[j] = (double)(expf((float)(l[j] - m)) * inv);  // probabilities
    if (a.probs)
        for (int j = 0; j < n; ++j) a.probs[tt * a.N + g * n + j] = (float)l[j];
    double ps = 0.0;
    for (int r = 0; r < k; ++r) ps += l[(sel >> (4 * r)) & 15];
    const int64_t o = (tt * a.G + g) * k;
    for (int r = 0; r < k; ++r) {
        const int j = (int)((sel >> (4 * r)) & 15);
        const int e = g * n + j;
        const double p = l[j];
        a.idx[o + r] = e;
        a.wsel[o + r] = (float)(p / ps);
        a.psel[o + r] = (float)p;
        if (a.ridx) a.ridx[o + r] = e;
        if (a.rw) a.rw[o + r] = (float)(p / ps);
        if (cnt) atomicAdd(&cnt[e], 1);
    }
}

// Softmax, top-k and weights for the block's tokens; logits in lg[tok][e] (bias included).
// The selection compares the float64 logits; the probabilities are formed from the float64
// differences l - max with the float32 exponential (relative error ~1e-7), and overwrite the
// logits of the same (token, group).  Per-block statistics follow.
__device__ void select_and_stats(const RouterArgs& a, double (*lg)[65], int* cnt, int64_t t0, int nthreads, int blk) {
    const int G = a.G;
    for (int q = threadIdx.x; q < kTok * G; q += nthreads) {
        const int tok = q / G, g = q % G;
        const int64_t tt = t0 + tok;
        if (tt >= a.T) continue;
        select_one(a, &lg[tok][g * a.n], tt, g, cnt);
    }
    __syncthreads();
    // per-block probability sums of every expert, in a fixed order: thread (expert e, token
    // group j) sums tokens j, j + kJ, ...; the kJ group sums are then added in order
    constexpr int kJ = 8;  // token groups
    __shared__ double gs[kJ][64];
    for (int q = threadIdx.x; q < kJ * a.N; q += nthreads) {
        const int e = q % a.N, j = q / a.N;
        double s = 0.0;
        for (int tok = j; tok < kTok; tok += kJ)
            if (t0 + tok < a.T) s += lg[tok][e];
        gs[j][e] = s;
    }
    __syncthreads();
    if (threadIdx.x < a.N) {
        const int e = threadIdx.x;
        double s = 0.0;
        for (int j = 0; j < kJ; ++j) s += gs[j][e];
        a.part_psum[(int64_t)blk * a.N + e] = s;
        a.part_cnt[(int64_t)blk * a.N + e] = cnt[e];
    }
}

template <typename Tin>
__global__ void __launch_bounds__(512) router_mfma_kernel(RouterArgs a) {
    constexpr int kW = 8;  // waves; wave w sums the w-th eighth of the hidden dimension
    __shared__ double red[kW][kTok][17];
    __shared__ double lg[kTok][65];
    __shared__ int cnt[64];
    const int blk = (int)blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t0 = (int64_t)blk * kTok;
    if (threadIdx.x < 64) cnt[threadIdx.x] = 0;

    const int dq = a.d / kW;            // multiple of 8 (d % 64 == 0)
    const int nchunk = (dq + 31) / 32;  // 32-wide hidden chunks of this wave's share
    f64x4_t acc[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[tb] = f64x4_t{0.0, 0.0, 0.0, 0.0};
    const Tin* xb = reinterpret_cast<const Tin*>(a.x);
    // Chunks go in batches of kBatch whose x and weight loads are all issued before the first
    // product of the batch (one memory latency per batch instead of one per chunk).
    constexpr int kBatch = 3;
    constexpr int XW = sizeof(Tin) * 2;  // 32-bit words of a lane's eight hidden values
    for (int c0 = 0; c0 < nchunk; c0 += kBatch) {
        uint32_t xr[kBatch][4][XW];
        f64x4_t wr[kBatch][2];
#pragma unroll
        for (int cc = 0; cc < kBatch; ++cc) {
            const int c = c0 + cc;
            const int i0 = wv * dq + 32 * c;  // first hidden index of the chunk
            const bool in = c < nchunk && 8 * (lane >> 4) < dq - 32 * c;
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                int64_t t = t0 + 16 * tb + (lane & 15);
                if (t >= a.T) t = a.T - 1;
                if (in) {
                    const uint32_t* src = reinterpret_cast<const uint32_t*>(xb + t * a.d + i0 + 8 * (lane >> 4));
#pragma unroll
                    for (int q = 0; q < XW; q += 4) {
                        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src + q);
                        xr[cc][tb][q] = v[0];
                        xr[cc][tb][q + 1] = v[1];
                        xr[cc][tb][q + 2] = v[2];
                        xr[cc][tb][q + 3] = v[3];
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < XW; ++q) xr[cc][tb][q] = 0u;
                }
            }
            // lane-ordered weights [octet][column][8]: this lane's octet of hidden indices is
            // i0/8 + (lane >> 4) (clamped: past the end x is zero), its column lane & 15
            const int oct = min(i0 / 8 + (lane >> 4), a.d / 8 - 1);
            const f64x4_t* wp = reinterpret_cast<const f64x4_t*>(a.wr + ((int64_t)oct * 16 + (lane & 15)) * 8);
            wr[cc][0] = wp[0];
            wr[cc][1] = wp[1];
        }
#pragma unroll
        for (int cc = 0; cc < kBatch; ++cc) {
            if (c0 + cc >= nchunk) break;
            const double wv8[8] = {wr[cc][0][0], wr[cc][0][1], wr[cc][0][2], wr[cc][0][3],
                                   wr[cc][1][0], wr[cc][1][1], wr[cc][1][2], wr[cc][1][3]};
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                double xv[8];
                widen8<Tin>(reinterpret_cast<const Tin*>(xr[cc][tb]), xv);
#pragma unroll
                for (int s = 0; s < 8; ++s)
                    acc[tb] = __builtin_amdgcn_mfma_f64_16x16x4f64(xv[s], wv8[s], acc[tb], 0, 0, 0);
            }
        }
    }
    // C layout of v_mfma_f64_16x16x4: lane holds rows (lane >> 4) + 4i, column lane & 15
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wv][16 * tb + (lane >> 4) + 4 * i][lane & 15] = acc[tb][i];
    __syncthreads();
    for (int q = threadIdx.x; q < kTok * a.N; q += 64 * kW) {
        const int tok = q / a.N, e = q % a.N;
        double v = red[0][tok][e];
#pragma unroll
        for (int w = 1; w < kW; ++w) v += red[w][tok][e];
        lg[tok][e] = v + a.br[e];
    }
    __syncthreads();
    select_and_stats(a, lg, cnt, t0, 64 * kW, blk);
}

template <typename Tin>
__global__ void __launch_bounds__(256) router_valu_kernel(RouterArgs a) {
    __shared__ double red[4][kTok][17];
    __shared__ double lg[kTok][65];
    __shared__ int cnt[64];
    const int blk = (int)blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t0 = (int64_t)blk * kTok;
    const int64_t t = t0 + lane;
    const bool valid = t < a.T;
    if (threadIdx.x < 64) cnt[threadIdx.x] = 0;
    const int dq = (a.d + 3) / 4;
    const int i0 = min(a.d, wv * dq), i1 = min(a.d, i0 + dq);
    const Tin* xr = reinterpret_cast<const Tin*>(a.x) + (valid ? t : (int64_t)0) * a.d;
    for (int e0 = 0; e0 < a.Np; e0 += 16) {
        double acc[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = 0.0;
        for (int i = i0; i < i1; ++i) {
            const double xv = (double)to_f32(xr[i]);
            const_f64_ptr wrow = (const_f64_ptr)(a.wr + (int64_t)i * a.Np + e0);
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[j] = __builtin_fma(xv, wrow[j], acc[j]);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) red[wv][lane][j] = acc[j];
        __syncthreads();
        for (int q = threadIdx.x; q < kTok * 16; q += 256) {
            const int tok = q / 16, j = q % 16;
            if (e0 + j < a.N)
                lg[tok][e0 + j] = ((red[0][tok][j] + red[1][tok][j]) + red[2][tok][j]) + red[3][tok][j] + a.br[e0 + j];
        }
        __syncthreads();
    }
    select_and_stats(a, lg, cnt, t0, 256, blk);
}

// One token per block (few tokens, e.g. a decode step): thread (expert column e, hidden slice)
// sums its slice of x . W_r[:, e] in float64; the slices are added in a fixed order, then the
// same decision as the blocked kernels.  No balance statistics.  fast: the weights are in the
// lane-ordered layout of router_mfma_kernel ([octet][column][8], 16 columns), else [d][Np].
template <typename Tin>
__global__ void __launch_bounds__(256) router_token_kernel(RouterArgs a, int fast) {
    __shared__ double part[16][65];
    __shared__ double lg[65];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x;
    const int np = a.Np, nsl = 256 / np;  // Np in {16, 32, 48, 64}: 16 .. 5 slices
    const int e = tid % np, sl = tid / np;
    if (sl < nsl) {
        const Tin* xr = reinterpret_cast<const Tin*>(a.x) + t * a.d;
        double acc = 0.0;
        if (e < a.N) {
            if (fast) {
                // d % 64 == 0: octets sl, sl + nsl, ... of eight hidden values, one 16-byte load of
                // x and the 64 contiguous bytes of the lane-ordered weights each
                const int noct = a.d / 8;
#pragma unroll 4
                for (int oc = sl; oc < noct; oc += nsl) {
                    double xv[8];
                    widen8<Tin>(xr + 8 * oc, xv);
                    const f64x4_t* wp = reinterpret_cast<const f64x4_t*>(a.wr + ((int64_t)oc * 16 + e) * 8);
                    const f64x4_t w0 = wp[0], w1 = wp[1];
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc = __builtin_fma(xv[q], w0[q], acc);
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc = __builtin_fma(xv[4 + q], w1[q], acc);
                }
            } else {
                const int len = (a.d + nsl - 1) / nsl;
                const int i0 = sl * len, i1 = min(a.d, i0 + len);
#pragma unroll 8
                for (int i = i0; i < i1; ++i) acc = __builtin_fma((double)to_f32(xr[i]), a.wr[(int64_t)i * np + e], acc);
            }
        }
        part[sl][e] = acc;
    }
    __syncthreads();
    if (tid < a.N) {
        double v = part[0][tid];
        for (int q = 1; q < nsl; ++q) v += part[q][tid];
        lg[tid] = v + a.br[tid];
    }
    __syncthreads();
    if (tid < a.G) select_one(a, &lg[tid * a.n], t, tid, nullptr);
}

// Sums the per-block partials in a fixed order (deterministic) and forms the balance loss.
// Thread (slice j, expert e) sums blocks j, j + J, ...; the J slice sums are then added in order.
__global__ void __launch_bounds__(256) stats_finalize_kernel(const int32_t* __restrict__ part_cnt,
                                                             const double* __restrict__ part_psum,
                                                             int64_t nblk, int64_t T, int N, int G,
                                                             int k, char* __restrict__ stats) {
    __shared__ double ps[256];
    __shared__ int64_t pc[256];
    __shared__ double fp[64];
    stats_finalize_block(part_cnt, part_psum, nblk, T, N, G, k, stats, ps, pc, fp);
}

}  // namespace

bool router_uses_mfma(const GqeDims& D) { return D.d % 64 == 0 && D.N <= 16; }

hipError_t launch_router_tokens(const GqeDims& D, int64_t T, const void* x, const void* packed,
                                const PackedLayout& pl, int32_t* idx, float* wsel, float* psel, int32_t* route_idx,
                                float* route_w, hipStream_t st, KernelMarks* km) {
    const char* pk = (const char*)packed;
    RouterArgs a{};
    a.x = x;
    a.wr = (const double*)(pk + pl.wr64);
    a.br = (const double*)(pk + pl.br64);
    a.T = T;
    a.d = D.d;
    a.N = D.N;
    a.G = D.G;
    a.k = D.k;
    a.n = D.n;
    a.Np = (int)round_up(D.N, 16);
    a.idx = idx;
    a.wsel = wsel;
    a.psel = psel;
    a.ridx = route_idx;
    a.rw = route_w;
    const int fast = router_uses_mfma(D) ? 1 : 0;
    if (km) km->begin(KT_ROUTER);
    if (D.dtype == GQE_DTYPE_BF16) router_token_kernel<bf16_t><<<dim3((unsigned)T), 256, 0, st>>>(a, fast);
    else router_token_kernel<float><<<dim3((unsigned)T), 256, 0, st>>>(a, fast);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (km) km->mark(KT_ROUTER);
    return hipSuccess;
}

hipError_t launch_router(const GqeDims& D, const WorkPlan& P, const void* x, const void* packed,
                         const PackedLayout& pl, char* ws, int32_t* route_idx, float* route_w,
                         hipStream_t st, KernelMarks* km, bool finalize) {
    const char* pk = (const char*)packed;
    RouterArgs a{};
    a.x = x;
    a.wr = (const double*)(pk + pl.wr64);
    a.br = (const double*)(pk + pl.br64);
    a.T = P.T;
    a.d = D.d;
    a.N = D.N;
    a.G = D.G;
    a.k = D.k;
    a.n = D.n;
    a.Np = (int)round_up(D.N, 16);
    a.idx = (int32_t*)(ws + P.idx);
    a.wsel = (float*)(ws + P.wsel);
    a.psel = (float*)(ws + P.psel);
    a.probs = (float*)(ws + P.probs);
    a.ridx = route_idx;
    a.rw = route_w;
    a.part_cnt = (int32_t*)(ws + P.part_cnt);
    a.part_psum = (double*)(ws + P.part_psum);
    const dim3 grid((unsigned)P.nblk_router);
    const bool bf = D.dtype == GQE_DTYPE_BF16;
    if (km) km->begin(KT_ROUTER);
    if (router_uses_mfma(D)) {
        if (bf) router_mfma_kernel<bf16_t><<<grid, 512, 0, st>>>(a);
        else router_mfma_kernel<float><<<grid, 512, 0, st>>>(a);
    } else {
        if (bf) router_valu_kernel<bf16_t><<<grid, 256, 0, st>>>(a);
        else router_valu_kernel<float><<<grid, 256, 0, st>>>(a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (km) km->mark(KT_ROUTER);
    if (!finalize) return hipSuccess;  // the projection kernel's last work group finalizes
    if (km) km->begin(KT_ROUTER_STATS);
    stats_finalize_kernel<<<1, 256, 0, st>>>(a.part_cnt, a.part_psum, P.nblk_router, P.T, D.N, D.G, D.k,
                                             ws + P.stats);
    if (km) km->mark(KT_ROUTER_STATS);
    return hipGetLastError();
}
