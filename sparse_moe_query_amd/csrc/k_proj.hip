// Projections of the GQE layer on gfx950 matrix cores (bf16 in, fp32 accumulate, bf16 out).
//
// GQE README "Algorithm Overview": the K/V heads stay dense and unchanged (every token, every
// group), the always-on shared query head is dense, and only the selected query-head experts are
// computed.  All of them read the same token rows, so one kernel does them all:
//
//   work item = (tile of 128 tokens, 4 head blocks); head block = d_h output columns of one of
//               K_g, V_g, the shared query head, or routed expert e; one wave per head block
//   pipeline   per 64-wide slice of the hidden dimension, the x tile (128 x 64) and the four head
//              blocks' weights (4 d_h x 64, pre-transposed by gqe_pack_weights) go straight from
//              global memory into LDS (global_load_lds_dwordx4 into XOR-swizzled 16-byte chunks,
//              so fragment reads are bank-conflict free); two LDS stages, the next slice in
//              flight while the current one multiplies; the x tile is shared by the four waves
//   routed     tile-local token-to-expert bucketing: for its expert e the wave scans the tile's
//              routing decisions with a ballot (histogram = popcount, exclusive prefix = masked
//              popcount) and gathers the matching rows into a contiguous LDS slice; only those
//              rows are multiplied (no capacity, no dropped tokens; empty slices do no work)
//   products   v_mfma_f32_16x16x32_bf16 computing C^T = W^T x^T, one straight-line body for every
//              wave; each lane ends with four consecutive head-dim values of one token (K/Q rows
//              are stored as 8-byte vectors, V goes to V^T [dim][key], keys slotted by vt_pos)
//   epilogue   queries are stored multiplied by log2(e)/sqrt(d_h) (the attention scale, folded in
//              before the single rounding to bf16); every key's norm is stored for the attention
//              kernel's range test
#include "gqe_common.h"
#include "gqe_internal.h"
#include "gqe_stats.h"

namespace {

constexpr int kBM = 128;   // tokens per tile
constexpr int kKC = 64;    // hidden-dim slice per LDS stage (8 chunks of 16 bytes per row)

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
};

// Element offset of (row, 16-byte chunk c) in an LDS stage of [rows][64] bf16 whose chunks are
// XOR-swizzled by the row: rows 2m and 2m+1 fall in different halves of the 256-byte bank row and
// the XOR spreads eight such pairs, so the 16 rows one fragment read serves per LDS cycle hit
// distinct bank groups.
__device__ __forceinline__ int swz64(int row, int c) { return (row * 8 + (c ^ ((row >> 1) & 7))) * 8; }

// One 64-wide slice of the hidden dimension for one wave: C^T += W^T x^T over the eight row
// blocks myrow[] of the x stage and the wave's d_h weight rows.  Every wave runs this same
// straight-line body (routed slices too, on their gathered rows; padding rows are not stored),
// so the accumulators stay in place across the loop.
template <int DH>
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
#pragma unroll
        for (int rb = 0; rb < 8; ++rb) {
            const bf16x8_t xf = *reinterpret_cast<const bf16x8_t*>(xb + swz64(xrow[rb], c));
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
                acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[cb], xf, acc[rb][cb], 0, 0, 0);
        }
    }
}

template <int DH>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) proj_kernel(ProjArgs a) {
    constexpr int CB = DH / 16;
    constexpr int LX = kBM * kKC * 2 / 1024 / 4;       // 1 KB x segments per wave per stage
    constexpr int LW = 4 * DH * kKC * 2 / 1024 / 4;    // 1 KB weight segments per wave per stage
    __shared__ __align__(1024) uint16_t xs[2][kBM * kKC];
    __shared__ __align__(1024) uint16_t wls[2][4 * DH * kKC];
    // per wave: gathered tile rows (| rank << 8); lives in x stage 1 until the first slice is
    // loaded into it (each lane keeps the entries it needs in registers)
    uint16_t (*rows)[kBM] = reinterpret_cast<uint16_t (*)[kBM]>(&xs[1][0]);

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // XCD-aware order: the items of one token tile run on one XCD so its x tile stays in L2
    const int L = blockIdx.x;
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
    const int hb = job * 4 + w;
    const bool active = hb < a.HB;
    const int GD = a.G;
    // head block kinds: [0,G) K_g, [G,2G) V_g, 2G shared query (if s), then expert e
    const int ebase = 2 * GD + a.s;
    const bool is_v = active && hb >= GD && hb < 2 * GD;
    const bool is_expert = active && hb >= ebase;
    const int e = hb - ebase;
    const int g_of = is_expert ? e / a.n : (hb < GD ? hb : hb - GD);

    // ---- stage loader: each wave moves LX segments of the x tile (rows past the last token
    // repeat it) and LW segments of the weights (a head block past the last one reads block 0)
    // per-lane byte offsets are loop invariant; the slice index moves the (scalar) bases
    const int hb0 = job * 4;
    uint32_t xoff[LX], woff[LW];
#pragma unroll
    for (int i = 0; i < LX; ++i) {
        const int q = (w + 4 * i) * 64 + lane;
        const int r = q >> 3, c = (q & 7) ^ ((r >> 1) & 7);
        const int64_t rem = a.T - 1 - t0;
        xoff[i] = (uint32_t)(((r < rem ? r : rem) * a.d + 8 * c) * 2);
    }
#pragma unroll
    for (int i = 0; i < LW; ++i) {
        const int q = (w + 4 * i) * 64 + lane;
        const int r = q >> 3, c = (q & 7) ^ ((r >> 1) & 7);
        int h = hb0 + r / DH;
        if (h >= a.HB) h = 0;
        woff[i] = (uint32_t)(((h * DH + r % DH) * a.d + 8 * c) * 2);
    }
    const bf16_t* xbase = a.x + t0 * a.d;
    auto issue = [&](int kc, int stage) {
#pragma unroll
        for (int i = 0; i < LX; ++i) dma16(xbase + kc * kKC, xoff[i], &xs[stage][(w + 4 * i) * 512]);
#pragma unroll
        for (int i = 0; i < LW; ++i) dma16(a.wproj + kc * kKC, woff[i], &wls[stage][(w + 4 * i) * 512]);
    };
    issue(0, 0);

    // ---- rows of this wave (tile-local bucketing for a routed expert)
    int nrows;
    if (is_expert && !a.dense) {
        // padding entries (past the slice) point at row 0 so every LDS read stays in the tile
        rows[w][lane] = 0;
        rows[w][lane + 64] = 0;
        int base = 0;
        for (int half = 0; half < kBM / 64; ++half) {
            const int row = half * 64 + lane;
            const int64_t t = t0 + row;
            int rank = -1;
            if (t < a.T) {
                const int32_t* id = a.idx + (t * a.G + g_of) * a.k;
                for (int r = 0; r < a.k; ++r)
                    if (id[r] == e) rank = r;
            }
            const uint64_t m = __builtin_amdgcn_ballot_w64(rank >= 0);
            const int pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
            if (rank >= 0) rows[w][base + pre] = (uint16_t)(row | (rank << 8));
            base += __builtin_popcountll(m);
        }
        nrows = base;
    } else {
        const int64_t rem = a.T - t0;
        nrows = active ? (int)(rem < kBM ? rem : kBM) : 0;
        const int rank = is_expert ? e % a.n : 0;  // all-active GQA: expert j of a group is head j
        for (int i = lane; i < kBM; i += 64) rows[w][i] = (uint16_t)(i | (rank << 8));
    }
    nrows = __builtin_amdgcn_readfirstlane(nrows);
    const int nrb = (nrows + 15) / 16;

    f32x4_t acc[8][CB];
#pragma unroll
    for (int rb = 0; rb < 8; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = a.d / kKC;
    // my gathered entry for each row block (lane's row = rows[16 rb + lane % 16]); rows[] is
    // written and read by its own wave only, the barrier below frees stage 1 for the loads
    int myrow[8], xrow[8];  // row | rank << 8, and the row alone
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) {
        myrow[rb] = rows[w][16 * rb + (lane & 15)];
        xrow[rb] = myrow[rb] & 0xff;
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    __syncthreads();  // stage 0 visible, stage 1 free

    // ---- epilogue: acc[rb][cb] lane holds row 16 rb + (lane & 15) of the slice, head dims
    // 16 cb + 4 (lane >> 4) + 0..3
    auto epilogue = [&](f32x4_t (&acc)[8][DH / 16], const int (&myrow)[8], int nrows, int nrb) {
        const uint32_t S = (uint32_t)a.S;  // the host limits a call to 2^28 tokens
        float kmx[2] = {0.f, 0.f};  // K blocks: largest squared norm of each 64-token half
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
            // S % 64 == 0: the two 64-token halves of the tile are whole 64-key tiles
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float m = kmx[h];
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o));
                const int64_t t = t0 + 64 * h;
                if (lane == 0 && t < a.T) {
                    const uint32_t b = (uint32_t)t / S, sp = (uint32_t)t - b * S;
                    a.knt[((int64_t)b * a.G + hb) * (a.S_pad / 64) + sp / 64] = sqrtf(m);
                }
            }
        }
    };

    for (int kc = 0; kc < nk; ++kc) {
        const int stage = kc & 1;
        if (kc + 1 < nk) issue(kc + 1, stage ^ 1);
        mma_slice<DH>(acc, xs[stage], wls[stage], xrow, w * DH, lane);
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
        __syncthreads();
    }
    if (active) epilogue(acc, myrow, nrows, nrb);
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
                            const PackedLayout& pl, char* ws, hipStream_t st, KernelMarks* km) {
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
    const unsigned grid = (unsigned)((int64_t)a.ntiles * a.njobs);
    if (km) km->begin(KT_PROJ);
    switch (D.dh) {
        case 32: proj_kernel<32><<<grid, 256, 0, st>>>(a); break;
        case 48: proj_kernel<48><<<grid, 256, 0, st>>>(a); break;
        case 64: proj_kernel<64><<<grid, 256, 0, st>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    if (km) km->mark(KT_PROJ);
    return hipGetLastError();
}
