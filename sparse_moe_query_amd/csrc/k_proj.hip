// Projections of the GQE layer on gfx950 matrix cores (bf16 in, fp32 accumulate, bf16 out).
//
// GQE README "Algorithm Overview": the K/V heads stay dense and unchanged (every token, every
// group), the always-on shared query head is dense, and only the selected query-head experts are
// computed.  All of them read the same token rows, so one kernel does them all:
//
//   work item = (tile of 256 tokens, 4 head blocks); head block = d_h output columns of one of
//               K_g, V_g, the shared query head, or routed expert e.  Eight waves: wave w computes
//               head block w & 3 on half w >> 2 of the head block's rows
//   pipeline   per 64-wide slice of the hidden dimension, the x tile (256 x 64) and the four head
//              blocks' weights (4 d_h x 64, pre-transposed by gqe_pack_weights) go straight from
//              global memory into LDS (global_load_lds_dwordx4 into XOR-swizzled 16-byte chunks,
//              so fragment reads are bank-conflict free); two LDS stages, the next slice in
//              flight while the current one multiplies.  The x tile is shared by the eight waves
//              and each head block's weights by two, so a 256-token tile halves the global reads
//              per product of a 128-token one
//   rows       a dense head block's rows are the tile's tokens, 128 per wave.  A routed expert's
//              rows are the tile's tokens routed to it: tile-local bucketing scans the routing
//              decisions with a ballot (histogram = popcount, exclusive prefix = masked popcount)
//              into a contiguous row list, split between the head block's two waves in whole
//              16-row blocks.  A wave multiplies only the 16-row blocks that hold rows (no
//              capacity, no dropped tokens; an expert with no rows in the tile does no products)
//   products   v_mfma_f32_16x16x32_bf16 computing C^T = W^T x^T; each lane ends with four
//              consecutive head-dim values of one token (K/Q rows are stored as 8-byte vectors,
//              V goes to V^T [dim][key], keys slotted by vt_pos)
//   epilogue   queries are stored multiplied by log2(e)/sqrt(d_h) (the attention scale, folded in
//              before the single rounding to bf16); every key's norm is stored for the attention
//              kernel's range test
#include "attn_sched_dev.h"
#include "gqe_common.h"
#include "gqe_internal.h"
#include "gqe_stats.h"

namespace {

constexpr int kBM = 256;   // tokens per tile
constexpr int kKC = 64;    // hidden-dim slice per LDS stage (8 chunks of 16 bytes per row)
constexpr int kWaves = 8;  // wave w: head block w & 3 of the item, row half w >> 2

struct ProjArgs {
    const bf16_t* x;
    const bf16_t* wproj;   // [HB][DH][d]
    const int32_t* idx;    // [T][G][k]
    bf16_t* Q;             // [B][H][S][DH]
    bf16_t* K;             // [B][G][S_pad][DH]
    bf16_t* Vt;            // [B][G][DH][S_pad]
    float* kn;             // [B][G][S_pad] key norms
    float* knt;            // [B][G][S_pad / 64] largest key norm per 64-key tile (when knt_here)
    float qscale;          // log2(e) / sqrt(d_h): queries are stored pre-scaled
    const double* rope;    // rotary embedding frequencies (cycles per position), or null when off
    int64_t T, S, S_pad;
    int d, G, k, n, H, s, dense, HB, njobs, ntiles;
    int knt_here;          // S % 64 == 0: every 64-key tile is one half of a 128-token tile
    // router statistics finalize, run by the last work group after its own tile (when stats_here)
    int stats_here, N;
    const int32_t* part_cnt;
    const double* part_psum;
    char* stats;
    int64_t nblk_router;
    // when set, work group 0 builds the attention work schedule and work group L + 1 runs job L
    int sched_here;
    SchedArgs sched;
};

// Element offset of (row, 16-byte chunk c) in an LDS stage of [rows][64] bf16 whose chunks are
// XOR-swizzled by the row: rows 2m and 2m+1 fall in different halves of the 256-byte bank row and
// the XOR spreads eight such pairs, so the 16 rows one fragment read serves per LDS cycle hit
// distinct bank groups.
__device__ __forceinline__ int swz64(int row, int c) { return (row * 8 + (c ^ ((row >> 1) & 7))) * 8; }

// Compile-time loop: f(integral_constant<int, I>) for I = B .. E - 1, so array indices derived from
// I are constants whatever the unroller decides (the accumulators stay in registers).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// One 64-wide slice of the hidden dimension for one wave: C^T += W^T x^T over the first NRB row
// blocks xrow[] of the x stage and the wave's d_h weight rows.  The x fragments are read two row
// blocks ahead of their products into a three-entry ring (the scheduling barriers pin that order:
// left alone, the compiler reads each fragment right before its products), and the row-block count
// is a template argument, so the body is straight-line code whose LDS waits count exactly the
// reads in flight (with a run-time count every conditional read made the compiler wait for all).
template <int DH, int NRB>
__device__ __forceinline__ void mma_slice(f32x4_t (&acc)[8][DH / 16], const uint16_t* xb, const uint16_t* wb,
                                          const int (&xrow)[8], int wrow, int lane) {
    constexpr int CB = DH / 16;
#pragma unroll
    for (int ks = 0; ks < kKC / 32; ++ks) {
        const int c = 4 * ks + (lane >> 4);
        bf16x8_t wf[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
            wf[cb] = *reinterpret_cast<const bf16x8_t*>(wb + swz64(wrow + 16 * cb + (lane & 15), c));
        auto xfrag = [&](int rb) { return *reinterpret_cast<const bf16x8_t*>(xb + swz64(xrow[rb], c)); };
        bf16x8_t xq[3];
        xq[0] = xfrag(0);
        if constexpr (NRB > 1) xq[1] = xfrag(1);
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, NRB>([&](auto rbc) {
            constexpr int rb = decltype(rbc)::value;
            if constexpr (rb + 2 < NRB) xq[(rb + 2) % 3] = xfrag(rb + 2);
            static_for<0, CB>([&](auto cbc) {
                constexpr int cb = decltype(cbc)::value;
                acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[cb], xq[rb % 3], acc[rb][cb], 0, 0, 0);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    }
}

template <int DH>
__global__ void __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2))) proj_kernel(ProjArgs a) {
    constexpr int CB = DH / 16;
    constexpr int NT = kWaves * 64;
    constexpr int LX = kBM * kKC * 2 / 1024 / kWaves;       // 1 KB x segments per wave per stage
    constexpr int LW = 4 * DH * kKC * 2 / 1024 / kWaves;    // 1 KB weight segments per wave per stage
    static_assert(LX * 1024 * kWaves == kBM * kKC * 2 && LW * 1024 * kWaves == 4 * DH * kKC * 2, "whole segments");
    // one LDS buffer: two x stages and two weight stages (or, in the schedule-building work
    // group, the builder's arrays)
    __shared__ __align__(1024) uint16_t lds_all[2 * kBM * kKC + 2 * 4 * DH * kKC];
    if (a.sched_here && blockIdx.x == 0) {
        attn_sched_block<NT>(a.sched, reinterpret_cast<unsigned char*>(lds_all), (int)sizeof(lds_all));
        return;
    }
    uint16_t (*xs)[kBM * kKC] = reinterpret_cast<uint16_t (*)[kBM * kKC]>(lds_all);
    uint16_t (*wls)[4 * DH * kKC] = reinterpret_cast<uint16_t (*)[4 * DH * kKC]>(lds_all + 2 * kBM * kKC);
    // per head block: its row list (row | rank << 8) and row count; they live in x stage 1 until
    // the first slice is loaded into it (each lane keeps the entries it needs in registers)
    uint16_t (*rows)[kBM] = reinterpret_cast<uint16_t (*)[kBM]>(&xs[1][0]);
    int* rcount = reinterpret_cast<int*>(&xs[1][4 * kBM]);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = w >> 2;
    // XCD-aware order: the items of one token tile run on one XCD so its x tile stays in L2
    const int L = (int)blockIdx.x - a.sched_here;
    int tile, job;
    if (a.ntiles % 8 == 0) {
        const int xcd = L % 8, i = L / 8;
        tile = (i / a.njobs) * 8 + xcd;
        job = i % a.njobs;
    } else {
        tile = L / a.njobs;
        job = L % a.njobs;
    }
    tile = __builtin_amdgcn_readfirstlane(tile);  // keep the tile's addresses in scalar registers
    job = __builtin_amdgcn_readfirstlane(job);
    const int64_t t0 = (int64_t)tile * kBM;
    const int GD = a.G;
    // head block kinds: [0,G) K_g, [G,2G) V_g, 2G shared query (if s), then expert e. Jobs take
    // them in the order K, V, experts, shared query: the dense shared block comes last, alone
    // in the last job when 4 j + 1 blocks leave one over, instead of sharing a job (and a SIMD's
    // two waves) with routed blocks that hold about half as many rows
    auto hb_at = [&](int p) { return (a.s && p >= 2 * GD) ? (p == a.HB - 1 ? 2 * GD : p + 1) : p; };
    const int p0 = job * 4;
    // a job holding only the last head block (not a K block, whose epilogue keeps per-half key
    // norms) spreads it over all eight waves, 32 rows each, instead of leaving six of them idle
    const bool single = p0 + 1 == a.HB && hb_at(p0) >= GD;
    const int slot = single ? 0 : (w & 3);
    const bool active = p0 + slot < a.HB;
    const int hb = active ? hb_at(p0 + slot) : a.HB;
    const int ebase = 2 * GD + a.s;
    const bool is_v = active && hb >= GD && hb < 2 * GD;
    const bool is_expert = active && hb >= ebase;
    const int e = hb - ebase;
    const int g_of = is_expert ? e / a.n : (hb < GD ? hb : hb - GD);
    const bool routed = is_expert && !a.dense;

    // ---- stage loader: each wave moves LX segments of the x tile (rows past the last token
    // repeat it) and LW segments of the weights (a head block past the last one reads block 0);
    // per-lane byte offsets are loop invariant, the slice index moves the (scalar) bases
    uint32_t xoff[LX], woff[LW];
#pragma unroll
    for (int i = 0; i < LX; ++i) {
        const int q = (w + kWaves * i) * 64 + lane;
        const int r = q >> 3, c = (q & 7) ^ ((r >> 1) & 7);
        const int64_t rem = a.T - 1 - t0;
        xoff[i] = (uint32_t)(((r < rem ? r : rem) * a.d + 8 * c) * 2);
    }
#pragma unroll
    for (int i = 0; i < LW; ++i) {
        const int q = (w + kWaves * i) * 64 + lane;
        const int r = q >> 3, c = (q & 7) ^ ((r >> 1) & 7);
        const int pw = p0 + r / DH;
        const int h = pw < a.HB ? hb_at(pw) : 0;
        woff[i] = (uint32_t)(((h * DH + r % DH) * a.d + 8 * c) * 2);
    }
    const bf16_t* xbase = a.x + t0 * a.d;
    auto issue = [&](int kc, int stage) {
#pragma unroll
        for (int i = 0; i < LX; ++i) dma16(xbase + kc * kKC, xoff[i], &xs[stage][(w + kWaves * i) * 512]);
#pragma unroll
        for (int i = 0; i < LW; ++i) dma16(a.wproj + kc * kKC, woff[i], &wls[stage][(w + kWaves * i) * 512]);
    };
    // ---- row lists, built before the first copies are issued so that their index loads wait for
    // nothing else: the first wave of each routed head block buckets the tile's decisions; the
    // tile's four index entries per lane are loaded together, one choice rank at a time
    if (routed && (single ? w == 0 : half == 0)) {
        constexpr int NP = kBM / 64;
        int rank[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) rank[p] = -1;
        for (int r = 0; r < a.k; ++r) {
            int32_t id[NP];
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int64_t t = t0 + p * 64 + lane;
                const int64_t tc = t < a.T ? t : a.T - 1;  // in bounds; masked below
                id[p] = a.idx[(tc * a.G + g_of) * a.k + r];
                if (t >= a.T) id[p] = -1;
            }
#pragma unroll
            for (int p = 0; p < NP; ++p)
                if (id[p] == e) rank[p] = r;
        }
        int base = 0;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const uint64_t m = __builtin_amdgcn_ballot_w64(rank[p] >= 0);
            const int pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
            if (rank[p] >= 0) rows[slot][base + pre] = (uint16_t)((p * 64 + lane) | (rank[p] << 8));
            base += __builtin_popcountll(m);
        }
        // padding entries (past the list) point at row 0 so every LDS read stays in the tile
        for (int i = base + lane; i < kBM; i += 64) rows[slot][i] = 0;
        if (lane == 0) rcount[slot] = base;
    }
    issue(0, 0);
    __syncthreads();  // row lists visible
    int nrows;
    int myrow[8], xrow[8];  // row | rank << 8, and the row alone, of the lane's row in each row block
    if (routed) {
        // the head block's list split in whole 16-row blocks: half 0 takes the first
        // 16 * ceil(cnt / 32) entries (at most 128), half 1 the rest; in a single-block job
        // wave w takes entries 32 w .. 32 w + 31
        const int cnt = rcount[slot];
        const int split = min(cnt, 16 * ((cnt + 31) / 32));
        const int first = single ? 32 * w : (half ? split : 0);
        nrows = single ? max(0, min(32, cnt - first)) : (half ? cnt - split : split);
#pragma unroll
        for (int rb = 0; rb < 8; ++rb) {
            const int i = first + 16 * rb + (lane & 15);
            myrow[rb] = rows[slot][i < kBM ? i : 0];
        }
    } else {
        const int r0 = single ? 32 * w : 128 * half, rmax = single ? 32 : 128;
        const int64_t rem = a.T - t0 - r0;
        nrows = active ? (int)(rem < 0 ? 0 : (rem < rmax ? rem : rmax)) : 0;
        const int rank = is_expert ? e % a.n : 0;  // all-active GQA: expert j of a group is head j
#pragma unroll
        for (int rb = 0; rb < 8; ++rb) myrow[rb] = ((r0 + 16 * rb + (lane & 15)) & 0xff) | (rank << 8);
    }
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) xrow[rb] = myrow[rb] & 0xff;
    nrows = __builtin_amdgcn_readfirstlane(nrows);
    const int nrb = (nrows + 15) / 16;

    f32x4_t acc[8][CB];
#pragma unroll
    for (int rb = 0; rb < 8; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = a.d / kKC;
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    __syncthreads();  // stage 0 visible; the row lists are read, stage 1 is free

    // ---- epilogue: acc[rb][cb] lane holds row block rb's row of this lane, head dims
    // 16 cb + 4 (lane >> 4) + 0..3
    auto epilogue = [&]() {
        const uint32_t S = (uint32_t)a.S;  // the host limits a call to 2^28 tokens
        float kmx[2] = {0.f, 0.f};  // K blocks: largest squared norm of each 64-token quarter
        // rotary embedding of query and key blocks: this lane's pairs are head dims
        // 16 cb + 4 (lane >> 4) + {0, 1} and {2, 3}, i.e. pairs 8 cb + 2 (lane >> 4) + {0, 1}
        const bool rot = a.rope != nullptr && !is_v;
        double rev[DH / 16][2];
#pragma unroll
        for (int cb = 0; cb < DH / 16; ++cb)
#pragma unroll
            for (int p = 0; p < 2; ++p) rev[cb][p] = rot ? a.rope[8 * cb + 2 * (lane >> 4) + p] : 0.0;
#pragma unroll
        for (int rb = 0; rb < 8; ++rb) {
            if (rb >= nrb) continue;
            const int li = 16 * rb + (lane & 15);
            const bool ok = li < nrows;
            const int row = myrow[rb] & 0xff, rank = myrow[rb] >> 8;
            const uint32_t t = (uint32_t)(t0 + row);
            const uint32_t b = t / S, sp = t - b * S;
            if (hb < GD) {
                // key: also its norm (the four lane groups hold complementary dims)
                float ss = 0.f;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) ss += acc[rb][cb][i] * acc[rb][cb][i];
                ss += __shfl_xor(ss, 16);
                ss += __shfl_xor(ss, 32);
                if (!ok) continue;
                if (rot)
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) rope_quad(acc[rb][cb], sp, rev[cb][0], rev[cb][1]);
                kmx[rb >> 2] = __builtin_fmaxf(kmx[rb >> 2], ss);
                if ((lane >> 4) == 0) a.kn[((int64_t)b * a.G + hb) * a.S_pad + sp] = sqrtf(ss);
                bf16_t* dst = a.K + (((int64_t)b * a.G + hb) * a.S_pad + sp) * DH;
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) {
                    const f32x4_t v = acc[rb][cb];
                    u32x2_t pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                    *reinterpret_cast<u32x2_t*>(dst + 16 * cb + 4 * (lane >> 4)) = pk;
                }
                continue;
            }
            if (!ok) continue;
            if (is_v) {
                // V^T [dim][key]: this lane's token is one key of four consecutive dim rows
                const int g = hb - GD;
                uint16_t* dst = reinterpret_cast<uint16_t*>(a.Vt) + ((int64_t)b * a.G + g) * DH * a.S_pad + vt_pos(sp);
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int i = 0; i < 4; i += 2) {
                        const uint32_t pk = pack_bf16x2(acc[rb][cb][i], acc[rb][cb][i + 1]);
                        dst[(int64_t)(16 * cb + 4 * (lane >> 4) + i) * a.S_pad] = (uint16_t)(pk & 0xffffu);
                        dst[(int64_t)(16 * cb + 4 * (lane >> 4) + i + 1) * a.S_pad] = (uint16_t)(pk >> 16);
                    }
                continue;
            }
            bf16_t* dst;
            if (!is_expert) dst = a.Q + (((int64_t)b * a.H + a.G * a.k) * S + sp) * DH;  // shared head
            else dst = a.Q + (((int64_t)b * a.H + g_of * a.k + rank) * S + sp) * DH;
            const float qs = a.qscale;
            if (rot)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) rope_quad(acc[rb][cb], sp, rev[cb][0], rev[cb][1]);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const f32x4_t v = acc[rb][cb] * qs;
                u32x2_t pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                *reinterpret_cast<u32x2_t*>(dst + 16 * cb + 4 * (lane >> 4)) = pk;
            }
        }
        if (hb < GD && a.knt_here) {
            // S % 64 == 0: the two 64-token quarters of this wave's half are whole 64-key tiles
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float m = kmx[h];
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o));
                const int64_t t = t0 + 128 * half + 64 * h;
                if (lane == 0 && t < a.T) {
                    const uint32_t b = (uint32_t)t / S, sp = (uint32_t)t - b * S;
                    a.knt[((int64_t)b * a.G + hb) * (a.S_pad / 64) + sp / 64] = sqrtf(m);
                }
            }
        }
    };

    // ---- main loop: the same barriers for every wave; the loop is specialised on the wave's
    // row-block count (one copy per count, chosen once)
    auto run = [&](auto nrbc) {
        constexpr int NRB = decltype(nrbc)::value;
        for (int kc = 0; kc < nk; ++kc) {
            const int stage = kc & 1;
            if (kc + 1 < nk) issue(kc + 1, stage ^ 1);
            if constexpr (NRB > 0) mma_slice<DH, NRB>(acc, xs[stage], wls[stage], xrow, slot * DH, lane);
            __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
            __syncthreads();
        }
    };
    switch (nrb) {
        case 0: run(std::integral_constant<int, 0>{}); break;
        case 1: run(std::integral_constant<int, 1>{}); break;
        case 2: run(std::integral_constant<int, 2>{}); break;
        case 3: run(std::integral_constant<int, 3>{}); break;
        case 4: run(std::integral_constant<int, 4>{}); break;
        case 5: run(std::integral_constant<int, 5>{}); break;
        case 6: run(std::integral_constant<int, 6>{}); break;
        case 7: run(std::integral_constant<int, 7>{}); break;
        default: run(std::integral_constant<int, 8>{}); break;
    }
    if (active) epilogue();
    if (a.stats_here && blockIdx.x == gridDim.x - 1) {
        // the x stages are free now: LDS scratch of the statistics finalize
        __syncthreads();
        double* ps = reinterpret_cast<double*>(&xs[0][0]);
        int64_t* pc = reinterpret_cast<int64_t*>(&xs[0][0] + 1024);
        double* fp = reinterpret_cast<double*>(&xs[1][0]);
        stats_finalize_block(a.part_cnt, a.part_psum, a.nblk_router, a.T, a.N, a.G, a.k, a.stats, ps, pc, fp);
    }
}

}  // namespace

hipError_t launch_proj_mfma(const GqeDims& D, const WorkPlan& P, const void* x, const void* packed,
                            const PackedLayout& pl, char* ws, hipStream_t st, KernelMarks* km, bool build_sched) {
    ProjArgs a{};
    a.x = (const bf16_t*)x;
    a.wproj = (const bf16_t*)((const char*)packed + pl.wproj);
    a.idx = (const int32_t*)(ws + P.idx);
    a.Q = (bf16_t*)(ws + P.q);
    a.K = (bf16_t*)(ws + P.kk);
    a.Vt = (bf16_t*)(ws + P.vt);
    a.kn = (float*)(ws + P.kn);
    a.knt = (float*)(ws + P.knt);
    a.knt_here = (P.S % 64 == 0) ? 1 : 0;
    a.stats_here = D.dense ? 0 : 1;
    a.N = D.N;
    a.part_cnt = (const int32_t*)(ws + P.part_cnt);
    a.part_psum = (const double*)(ws + P.part_psum);
    a.stats = ws + P.stats;
    a.nblk_router = P.nblk_router;
    a.qscale = (float)(1.4426950408889634 / std::sqrt((double)D.dh));
    a.rope = D.rope > 0.f ? (const double*)((const char*)packed + pl.rope) : nullptr;
    a.T = P.T;
    a.S = P.S;
    a.S_pad = P.S_pad;
    a.d = D.d;
    a.G = D.G;
    a.k = D.k;
    a.n = D.n;
    a.H = D.H;
    a.s = D.s;
    a.dense = D.dense;
    a.HB = pl.hb_total;
    a.njobs = (a.HB + 3) / 4;
    a.ntiles = (int)ceil_div(P.T, kBM);
    if (D.d % kKC != 0) return hipErrorInvalidValue;
    a.sched_here = build_sched ? 1 : 0;
    if (build_sched) a.sched = make_sched_args(D, P, ws);
    const unsigned grid = (unsigned)((int64_t)a.ntiles * a.njobs + a.sched_here);
    if (km) km->begin(KT_PROJ);
    switch (D.dh) {
        case 32: proj_kernel<32><<<grid, kWaves * 64, 0, st>>>(a); break;
        case 48: proj_kernel<48><<<grid, kWaves * 64, 0, st>>>(a); break;
        case 64: proj_kernel<64><<<grid, kWaves * 64, 0, st>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    if (km) km->mark(KT_PROJ);
    return hipGetLastError();
}
