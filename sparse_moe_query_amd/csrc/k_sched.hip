// Device builder of the attention work schedule (one work group per forward).
//
// The matrix-core attention runs one job per work group: an item (batch, group, block of
// positions) or a chunk of consecutive key tiles of a long item, dispatched longest first, with
// a merge record per split item (k_attn.hip).  The tables follow the canonical order defined in
// gqe_internal.h; the host only chooses the chunk cap (a simulation of the dispatch,
// attn_sched.cpp), so that gqe_forward allocates nothing and copies nothing: every forward
// rebuilds the tables in its workspace on its stream, ahead of the router.
//
// Steps (1024 threads):
//   1  per item of one sequence: its chunk count nc; exclusive scans give the first template of
//      every item, the first partial slot (chunks of the split items before it) and its merge
//      number (split items before it)
//   2  per template: its item and length; a histogram of the lengths in LDS
//   3  the histogram scanned from the longest length down: the first rank of every length
//   4  one wave walks the templates in order, 64 at a time; lanes of equal length take
//      consecutive ranks (ballot + masked popcount), so equal lengths keep template order
//   5  per (template, sequence): its job record at B rank + b; per (split item, sequence): its
//      merge record
#include "gqe_common.h"
#include "gqe_internal.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxLen = 8192;      // histogram entries in LDS: template lengths 1 .. kMaxLen - 1
constexpr int kLdsTpl = 16384;     // template lengths kept in LDS for the ranking wave

struct SchedArgs {
    AttnJob* jobs;
    AttnMerge* merges;
    int32_t* tstart;   // [items + 1] first template of every item
    int32_t* sstart;   // [items + 1] chunks of the split items before it (slots / B)
    int32_t* mstart;   // [items + 1] split items before it (merges / B)
    int32_t* tf;       // [tpl] item of every template
    int16_t* tlen;     // [tpl] length of every template
    int32_t* rank;     // [tpl] dispatch rank of every template
    int64_t B, S;
    int G, k, s, skv, C, items, tpl, maxlen;
};

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(x, o);
        if (lane >= o) x += t;
    }
    return x;
}

// Exclusive scan of NV interleaved int sequences of length n (ld(i, v) reads element i, st(i, v)
// writes its exclusive prefix); returns the totals in tot.
template <int NV, class Ld, class St>
__device__ void block_scan(int n, Ld ld, St st, int* lds_tot, int (&tot)[NV]) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int q = 0; q < NV; ++q) tot[q] = 0;
    for (int base = 0; base < n; base += kThreads) {
        const int i = base + tid;
        int v[NV], inc[NV];
        ld(i, v);
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            if (i >= n) v[q] = 0;
            inc[q] = wave_incl_scan(v[q], lane);
        }
        if (lane == 63)
#pragma unroll
            for (int q = 0; q < NV; ++q) lds_tot[w * NV + q] = inc[q];
        __syncthreads();
        int pre[NV], bt[NV];
#pragma unroll
        for (int q = 0; q < NV; ++q) pre[q] = bt[q] = 0;
        for (int x = 0; x < kWaves; ++x)
#pragma unroll
            for (int q = 0; q < NV; ++q) {
                const int t = lds_tot[x * NV + q];
                if (x < w) pre[q] += t;
                bt[q] += t;
            }
        if (i < n) {
            int out[NV];
#pragma unroll
            for (int q = 0; q < NV; ++q) out[q] = tot[q] + pre[q] + inc[q] - v[q];
            st(i, out);
        }
#pragma unroll
        for (int q = 0; q < NV; ++q) tot[q] += bt[q];
        __syncthreads();
    }
}

__global__ void __launch_bounds__(kThreads) attn_sched_kernel(SchedArgs a) {
    __shared__ int goff[65];        // first item of every group (+ the total)
    __shared__ int lds_tot[kWaves * 3];
    __shared__ int cursor[kMaxLen];  // histogram, then the next free rank, per length
    __shared__ int16_t tlen_l[kLdsTpl];
    const int tid = threadIdx.x, lane = tid & 63;
    const int G = a.G;
    if (tid == 0) {
        int acc = 0;
        for (int g = 0; g < G; ++g) {
            goff[g] = acc;
            acc += attn_items_of_group(a.S, attn_item_nh(g, a.k, a.s, a.skv));
        }
        goff[G] = acc;
    }
    for (int i = tid; i <= a.maxlen; i += kThreads) cursor[i] = 0;
    __syncthreads();
    // item f -> group, item of the group, geometry, chunk count
    auto item = [&](int f, int& g, int& nh, int& p0, int& np, int& kt, int& nc) {
        int lo = 0, hi = G - 1;  // the last group with goff[g] <= f
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (goff[mid] <= f) lo = mid;
            else hi = mid - 1;
        }
        g = lo;
        nh = attn_item_nh(g, a.k, a.s, a.skv);
        kt = attn_item_tiles(a.S, nh, f - goff[g], &p0, &np);
        nc = attn_chunks_of(kt, a.C);
    };

    // ---- 1: per-item prefixes
    {
        int tot[3];
        block_scan<3>(
            a.items,
            [&](int f, int (&v)[3]) {
                if (f < a.items) {
                    int g, nh, p0, np, kt, nc;
                    item(f, g, nh, p0, np, kt, nc);
                    v[0] = nc;
                    v[1] = nc > 1 ? nc : 0;
                    v[2] = nc > 1 ? 1 : 0;
                }
            },
            [&](int f, int (&o)[3]) {
                a.tstart[f] = o[0];
                a.sstart[f] = o[1];
                a.mstart[f] = o[2];
            },
            lds_tot, tot);
        if (tid == 0) {
            a.tstart[a.items] = tot[0];
            a.sstart[a.items] = tot[1];
            a.mstart[a.items] = tot[2];
        }
    }
    __threadfence_block();
    __syncthreads();

    // ---- 2: templates of every item, their lengths, the length histogram
    const bool lds_len = a.tpl <= kLdsTpl;
    for (int f = tid; f < a.items; f += kThreads) {
        int g, nh, p0, np, kt, nc;
        item(f, g, nh, p0, np, kt, nc);
        const int t0 = a.tstart[f];
        for (int c = 0; c < nc; ++c) {
            int k0, k1;
            attn_chunk_range(kt, nc, c, &k0, &k1);
            const int len = k1 - k0;
            a.tf[t0 + c] = f;
            a.tlen[t0 + c] = (int16_t)len;
            if (lds_len) tlen_l[t0 + c] = (int16_t)len;
            atomicAdd(&cursor[len], 1);
        }
    }
    __threadfence_block();
    __syncthreads();

    // ---- 3: first rank of every length, longest first (lengths 1 .. maxlen)
    {
        const int L = a.maxlen;
        int tot[1];
        block_scan<1>(
            L, [&](int j, int (&v)[1]) { if (j < L) v[0] = cursor[L - j]; },
            [&](int j, int (&o)[1]) { cursor[L - j] = o[0]; }, lds_tot, tot);
    }
    __syncthreads();

    // ---- 4: ranks in template order (one wave; LDS accesses of a wave are in order)
    if (tid < 64) {
        const int16_t* tl = lds_len ? tlen_l : a.tlen;
        for (int base = 0; base < a.tpl; base += 64) {
            const int t = base + lane;
            const bool valid = t < a.tpl;
            const int len = valid ? tl[t] : 0;
            uint64_t rem = __builtin_amdgcn_ballot_w64(valid);
            while (rem) {
                const int src = __builtin_ctzll(rem);
                const int l0 = __shfl(len, src);
                const uint64_t m = __builtin_amdgcn_ballot_w64(valid && len == l0);
                const int cur = cursor[l0];
                if (valid && len == l0) {
                    const uint64_t below = lane ? (m & ((~0ull) >> (64 - lane))) : 0ull;
                    a.rank[t] = cur + __builtin_popcountll(below);
                }
                if (lane == src) cursor[l0] = cur + __builtin_popcountll(m);
                rem &= ~m;
            }
        }
    }
    __threadfence_block();
    __syncthreads();

    // ---- 5: job records (template t, sequence b) -> position B rank + b; merge records
    const int64_t B = a.B;
    const int64_t nj = B * a.tpl;
    for (int64_t j = tid; j < nj; j += kThreads) {
        const int t = (int)(j / B);
        const int b = (int)(j - (int64_t)t * B);
        const int f = a.tf[t];
        int g, nh, p0, np, kt, nc;
        item(f, g, nh, p0, np, kt, nc);
        const int c = t - a.tstart[f];
        int k0, k1;
        attn_chunk_range(kt, nc, c, &k0, &k1);
        const int part = nc > 1 ? (int)(B * a.sstart[f] + (int64_t)b * nc + c) : -1;
        a.jobs[B * a.rank[t] + b] = AttnJob{b, g, nh, p0, np, k0, k1, part};
    }
    const int64_t nm = B * a.items;
    for (int64_t j = tid; j < nm; j += kThreads) {
        const int f = (int)(j / B);
        const int b = (int)(j - (int64_t)f * B);
        int g, nh, p0, np, kt, nc;
        item(f, g, nh, p0, np, kt, nc);
        if (nc <= 1) continue;
        a.merges[B * a.mstart[f] + b] = AttnMerge{b, g, nh, p0, np, (int)(B * a.sstart[f] + (int64_t)b * nc), nc, 0};
    }
}

}  // namespace

size_t attn_sched_scratch_bytes(const AttnCounts& ac) {
    return (size_t)(3 * (ac.items + 1) + ac.tpl) * 4 + (size_t)ac.tpl * 4 + (size_t)ac.tpl * 2 + 64;
}

hipError_t launch_attn_sched(const GqeDims& D, const WorkPlan& P, char* ws, hipStream_t st) {
    const AttnCounts& ac = P.ac;
    if (ac.njobs <= 0 || ac.maxlen >= kMaxLen || D.G > 64) return hipErrorInvalidValue;
    SchedArgs a{};
    a.jobs = (AttnJob*)(ws + P.sched_jobs);
    a.merges = (AttnMerge*)(ws + P.sched_merges);
    int32_t* sc = (int32_t*)(ws + P.sched_scratch);
    a.tstart = sc;
    a.sstart = a.tstart + (ac.items + 1);
    a.mstart = a.sstart + (ac.items + 1);
    a.tf = a.mstart + (ac.items + 1);
    a.rank = a.tf + ac.tpl;
    a.tlen = (int16_t*)(a.rank + ac.tpl);
    a.B = P.B;
    a.S = P.S;
    a.G = D.G;
    a.k = D.k;
    a.s = D.s;
    a.skv = D.skv;
    a.C = ac.chunk;
    a.items = ac.items;
    a.tpl = ac.tpl;
    a.maxlen = ac.maxlen;
    attn_sched_kernel<<<1, kThreads, 0, st>>>(a);
    return hipGetLastError();
}
