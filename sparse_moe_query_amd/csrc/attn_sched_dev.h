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
//   2  per template: its item, and the sort key (longest first)
//   3  a stable radix sort of the template numbers by key (equal keys keep template order)
//   4  per (sorted position p, sequence b): the job record of the template at p goes to B p + b;
//      per (split item, sequence): its merge record
// The per-item and per-template arrays live in LDS when they fit (the usual case), else in the
// workspace.
#pragma once

#include "gqe_common.h"
#include "gqe_internal.h"

struct SchedArgs {
    AttnJob* jobs;
    AttnMerge* merges;
    int32_t* gscratch;  // the same arrays as in LDS, when they do not fit there
    int64_t B, S;
    int G, k, s, skv, C, items, tpl;
    int nbits;         // bits of the longest template length (the sort key is maxlen - length)
    int maxlen;
};

// Bytes of the builder's arrays: tstart, sstart, mstart [items + 1], then tf, key, idx, tmp and
// pre [tpl] (int32 each).
__host__ __device__ inline size_t sched_array_bytes(int items, int tpl) {
    return ((size_t)3 * (items + 1) + (size_t)5 * tpl) * 4;
}

namespace sched_dev {

// LDS bytes for the group offsets (ints [0, 65)) and the scan's wave totals (ints [68, 68 + 4 NT/64),
// up to 1024 threads)
constexpr int kHeader = 1024;

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

// The builder on arrays at `arr` (LDS or workspace; the two instantiations keep the accesses in
// their own address space).
template <int NT>
__device__ __forceinline__ void build(const SchedArgs& a, int* goff, int* lds_tot, int32_t* arr) {
    const int tid = threadIdx.x;
    const int G = a.G;
    int32_t* tstart = arr;
    int32_t* sstart = tstart + (a.items + 1);
    int32_t* mstart = sstart + (a.items + 1);
    int32_t* tf = mstart + (a.items + 1);
    int32_t* key = tf + a.tpl;
    int32_t* idx = key + a.tpl;
    int32_t* tmp = idx + a.tpl;
    int32_t* pre = tmp + a.tpl;
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
                tstart[f] = o[0];
                sstart[f] = o[1];
                mstart[f] = o[2];
            },
            lds_tot, tot);
        if (tid == 0) {
            tstart[a.items] = tot[0];
            sstart[a.items] = tot[1];
            mstart[a.items] = tot[2];
        }
    }
    __threadfence_block();
    __syncthreads();

    // ---- 2: the templates of every item: their item and sort key (longest first)
    for (int f = tid; f < a.items; f += NT) {
        int g, nh, p0, np, kt, nc;
        item(f, g, nh, p0, np, kt, nc);
        const int t0 = tstart[f];
        for (int c = 0; c < nc; ++c) {
            int k0, k1;
            attn_chunk_range(kt, nc, c, &k0, &k1);
            tf[t0 + c] = f;
            key[t0 + c] = a.maxlen - (k1 - k0);
            idx[t0 + c] = t0 + c;
        }
    }
    __threadfence_block();
    __syncthreads();

    // ---- 3: stable LSD radix sort of the template numbers by key, two bits per pass (a stable
    // four-way split: a block scan of the digit flags, then a scatter)
    for (int shift = 0; shift < a.nbits; shift += 2) {
        int tot[4];
        block_scan<NT, 4>(
            a.tpl,
            [&](int i, int (&v)[4]) {
                const int dgt = (key[idx[i]] >> shift) & 3;
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = dgt == q ? 1 : 0;
            },
            [&](int i, int (&o)[4]) {
                const int dgt = (key[idx[i]] >> shift) & 3;
                pre[i] = dgt == 0 ? o[0] : dgt == 1 ? o[1] : dgt == 2 ? o[2] : o[3];
            },
            lds_tot, tot);
        const int s1 = tot[0], s2 = s1 + tot[1], s3 = s2 + tot[2];
        for (int i = tid; i < a.tpl; i += NT) {
            const int t = idx[i];
            const int dgt = (key[t] >> shift) & 3;
            tmp[(dgt == 0 ? 0 : dgt == 1 ? s1 : dgt == 2 ? s2 : s3) + pre[i]] = t;
        }
        __threadfence_block();
        __syncthreads();
        int32_t* x = idx;
        idx = tmp;
        tmp = x;
    }

    // ---- 4: job records (sorted position p, sequence b) -> B p + b; merge records
    const int B = (int)a.B;   // B tpl < 2^31 (checked on the host)
    const int nj = B * a.tpl;
    for (int j = tid; j < nj; j += NT) {
        const int p = j / B;
        const int b = j - p * B;
        const int t = idx[p];
        const int f = tf[t];
        int g, nh, p0, np, kt, nc;
        item(f, g, nh, p0, np, kt, nc);
        const int c = t - tstart[f];
        int k0, k1;
        attn_chunk_range(kt, nc, c, &k0, &k1);
        const int part = nc > 1 ? B * sstart[f] + b * nc + c : -1;
        a.jobs[j] = AttnJob{b, g, nh, p0, np, k0, k1, part};
    }
    const int nm = B * a.items;
    for (int j = tid; j < nm; j += NT) {
        const int f = j / B;
        const int b = j - f * B;
        int g, nh, p0, np, kt, nc;
        item(f, g, nh, p0, np, kt, nc);
        if (nc <= 1) continue;
        a.merges[B * mstart[f] + b] = AttnMerge{b, g, nh, p0, np, B * sstart[f] + b * nc, nc, 0};
    }
}

}  // namespace sched_dev

// The whole builder, by one work group of NT threads; lds: LDS scratch of lds_bytes (the
// arrays live there when kHeader + their bytes fit).
template <int NT>
__device__ __forceinline__ void attn_sched_block(const SchedArgs& a, unsigned char* lds, int lds_bytes) {
    using namespace sched_dev;
    int* goff = reinterpret_cast<int*>(lds);            // [65]
    static_assert(68 + 4 * (NT / 64) <= kHeader / 4, "scan totals must fit the header");
    int* lds_tot = reinterpret_cast<int*>(lds) + 68;    // [NT / 64 * 4]
    if (threadIdx.x < 64) {
        // lane g: the items of group g; the wave's exclusive scan gives the first item of each
        const int g = threadIdx.x;
        const int cnt = g < a.G ? attn_items_of_group(a.S, attn_item_nh(g, a.k, a.s, a.skv)) : 0;
        const int inc = sched_dev::wave_incl_scan(cnt, g);
        if (g < a.G) goff[g] = inc - cnt;
        if (g == a.G - 1) goff[a.G] = inc;
    }
    __syncthreads();
    if ((size_t)kHeader + sched_array_bytes(a.items, a.tpl) <= (size_t)lds_bytes)
        build<NT>(a, goff, lds_tot, reinterpret_cast<int32_t*>(lds + kHeader));
    else
        build<NT>(a, goff, lds_tot, a.gscratch);
}

// Host: the builder's arguments for the forward of plan P (workspace ws).
SchedArgs make_sched_args(const GqeDims& D, const WorkPlan& P, char* ws);
