// Device builder of the attention work schedule: run by one work group of any size, either as a
// kernel of its own (k_sched.hip) or as the first work group of the router launch (k_router.hip),
// where it overlaps the routing of the other work groups.
//
// The tables follow the canonical order defined in gqe_internal.h (the host only chooses the chunk
// cap, by a simulation of the dispatch in attn_sched.cpp), so gqe_forward allocates nothing and
// copies nothing: every forward rebuilds the tables in its workspace on its stream.
//
// Steps:
//   1  per item of one sequence: its chunk count nc; exclusive scans give the first template of
//      every item, its first partial slot (chunks of the split items before it) and its merge
//      number (split items before it)
//   2  per template: its item, and the sort key (longest first, then template number)
//   3  bitonic sort of the keys (in LDS when they fit, else in the workspace)
//   4  rank of every template = its position in the sorted keys
//   5  per (template, sequence): its job record at B rank + b; per (split item, sequence): its
//      merge record
#pragma once

#include "gqe_common.h"
#include "gqe_internal.h"

struct SchedArgs {
    AttnJob* jobs;
    AttnMerge* merges;
    int32_t* tstart;   // [items + 1] first template of every item
    int32_t* sstart;   // [items + 1] chunks of the split items before it (slots / B)
    int32_t* mstart;   // [items + 1] split items before it (merges / B)
    int32_t* tf;       // [tpl] item of every template
    int32_t* rank;     // [tpl] dispatch rank of every template
    uint64_t* gkeys;   // [npow2] sort keys when they do not fit in LDS
    int64_t B, S;
    int G, k, s, skv, C, items, tpl, maxlen, npow2;
};

// Scratch bytes of the builder in the workspace (int32 prefix arrays, item and rank of every
// template, sort keys).
__host__ __device__ inline int sched_npow2(int tpl) {
    int n = 2;
    while (n < tpl) n <<= 1;
    return n;
}

namespace sched_dev {

constexpr int kHeader = 512;  // LDS bytes for the group offsets and the scan's wave totals

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(x, o);
        if (lane >= o) x += t;
    }
    return x;
}

// Exclusive scan of NV interleaved int sequences of length n by a work group of NT threads
// (ld(i, v) reads element i, st(i, v) writes its exclusive prefix); returns the totals.
template <int NT, int NV, class Ld, class St>
__device__ void block_scan(int n, Ld ld, St st, int* lds_tot, int (&tot)[NV]) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
    for (int q = 0; q < NV; ++q) tot[q] = 0;
    for (int base = 0; base < n; base += NT) {
        const int i = base + tid;
        int v[NV], inc[NV];
#pragma unroll
        for (int q = 0; q < NV; ++q) v[q] = 0;
        if (i < n) ld(i, v);
#pragma unroll
        for (int q = 0; q < NV; ++q) inc[q] = wave_incl_scan(v[q], lane);
        if (lane == 63)
#pragma unroll
            for (int q = 0; q < NV; ++q) lds_tot[w * NV + q] = inc[q];
        __syncthreads();
        int pre[NV], bt[NV];
#pragma unroll
        for (int q = 0; q < NV; ++q) pre[q] = bt[q] = 0;
        for (int x = 0; x < NW; ++x)
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

}  // namespace sched_dev

// The whole builder, by one work group of NT threads; lds: at least kHeader + 8 bytes of LDS
// (keys live there when kHeader + 8 npow2 <= lds_bytes).
template <int NT>
__device__ void attn_sched_block(const SchedArgs& a, unsigned char* lds, int lds_bytes) {
    using namespace sched_dev;
    int* goff = reinterpret_cast<int*>(lds);            // [65]
    int* lds_tot = reinterpret_cast<int*>(lds) + 68;    // [NT / 64 * 3]
    const bool keys_lds = kHeader + 8 * a.npow2 <= lds_bytes;
    uint64_t* keys = keys_lds ? reinterpret_cast<uint64_t*>(lds + kHeader) : a.gkeys;
    const int tid = threadIdx.x;
    const int G = a.G;
    if (tid == 0) {
        int acc = 0;
        for (int g = 0; g < G; ++g) {
            goff[g] = acc;
            acc += attn_items_of_group(a.S, attn_item_nh(g, a.k, a.s, a.skv));
        }
        goff[G] = acc;
    }
    __syncthreads();
    // item f -> group, geometry, chunk count
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
        block_scan<NT, 3>(
            a.items,
            [&](int f, int (&v)[3]) {
                int g, nh, p0, np, kt, nc;
                item(f, g, nh, p0, np, kt, nc);
                v[0] = nc;
                v[1] = nc > 1 ? nc : 0;
                v[2] = nc > 1 ? 1 : 0;
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

    // ---- 2: the templates of every item and their sort keys (longest first, then number)
    for (int f = tid; f < a.items; f += NT) {
        int g, nh, p0, np, kt, nc;
        item(f, g, nh, p0, np, kt, nc);
        const int t0 = a.tstart[f];
        for (int c = 0; c < nc; ++c) {
            int k0, k1;
            attn_chunk_range(kt, nc, c, &k0, &k1);
            a.tf[t0 + c] = f;
            keys[t0 + c] = ((uint64_t)(uint32_t)(a.maxlen - (k1 - k0)) << 32) | (uint32_t)(t0 + c);
        }
    }
    for (int t = a.tpl + tid; t < a.npow2; t += NT) keys[t] = ~0ull;
    __threadfence_block();
    __syncthreads();

    // ---- 3: bitonic sort, ascending
    const int n = a.npow2;
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < (n >> 1); i += NT) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const uint64_t x = keys[lo], y = keys[hi];
                const bool up = (lo & size) == 0;
                if ((x > y) == up) {
                    keys[lo] = y;
                    keys[hi] = x;
                }
            }
            __threadfence_block();
            __syncthreads();
        }
    }

    // ---- 4: ranks
    for (int p = tid; p < a.tpl; p += NT) a.rank[(uint32_t)keys[p]] = p;
    __threadfence_block();
    __syncthreads();

    // ---- 5: job records (template t, sequence b) -> position B rank + b; merge records
    const int64_t B = a.B;
    const int64_t nj = B * a.tpl;
    for (int64_t j = tid; j < nj; j += NT) {
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
    for (int64_t j = tid; j < nm; j += NT) {
        const int f = (int)(j / B);
        const int b = (int)(j - (int64_t)f * B);
        int g, nh, p0, np, kt, nc;
        item(f, g, nh, p0, np, kt, nc);
        if (nc <= 1) continue;
        a.merges[B * a.mstart[f] + b] = AttnMerge{b, g, nh, p0, np, (int)(B * a.sstart[f] + (int64_t)b * nc), nc, 0};
    }
}

// Host: the builder's arguments for the forward of plan P (workspace ws).
SchedArgs make_sched_args(const GqeDims& D, const WorkPlan& P, char* ws);
