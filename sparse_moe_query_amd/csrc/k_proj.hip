// Projections of the GQE layer on gfx950 matrix cores (bf16 in, fp32 accumulate, bf16 out).
//
// GQE README "Algorithm Overview": the K/V heads stay dense and unchanged (every token, every
// group), the always-on shared query head is dense, and only the selected query-head experts are
// computed.  All of them read the same token rows, so one kernel does them all:
//
//   work item = (tile of 128 tokens, 4 head blocks); head block = d_h output columns of one of
//               K_g, V_g, the shared query head, or routed expert e
//   x tile     staged once in LDS per 32-wide slice of the hidden dimension, shared by the four
//              waves (one wave per head block)
//   routed     tile-local token-to-expert bucketing: for its expert e the wave scans the tile's
//              routing decisions with a ballot (histogram = popcount, exclusive prefix = masked
//              popcount) and gathers the matching rows into a contiguous LDS slice; only those
//              rows are multiplied (no capacity, no dropped tokens; empty slices do no work)
//   products   v_mfma_f32_16x16x32_bf16; K/Q blocks compute C^T = W^T x^T so each lane stores four
//              consecutive head-dim values; V blocks compute C = x W so each lane stores four
//              consecutive keys of V^T (slotted by vt_pos, see k_attn)
//   epilogue   queries are stored multiplied by log2(e)/sqrt(d_h) (the attention scale, folded in
//              before the single rounding to bf16); every key's norm is stored for the attention
//              kernel's range test
#include "gqe_common.h"
#include "gqe_internal.h"

namespace {

constexpr int kBM = 128;   // tokens per tile
constexpr int kKC = 32;    // hidden-dim slice per LDS stage
constexpr int kXP = kKC + 8;  // LDS pitch of the x tile (elements)

struct ProjArgs {
    const bf16_t* x;
    const bf16_t* wproj;   // [HB][DH][d]
    const int32_t* idx;    // [T][G][k]
    bf16_t* Q;             // [B][H][S][DH]
    bf16_t* K;             // [B][G][S_pad][DH]
    bf16_t* Vt;            // [B][G][DH][S_pad]
    float* kn;             // [B][G][S_pad] key norms
    float qscale;          // log2(e) / sqrt(d_h): queries are stored pre-scaled
    int64_t T, S, S_pad;
    int d, G, k, n, H, s, dense, HB, njobs, ntiles;
};

template <int DH>
__global__ void __launch_bounds__(256, 2) proj_kernel(ProjArgs a) {
    constexpr int CB = DH / 16;
    __shared__ __align__(16) uint16_t xs[2][kBM * kXP];
    __shared__ uint16_t rows[4][kBM];   // per wave: gathered tile rows (| rank << 8)
    __shared__ int nrows_s[4];

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
    if (lane == 0) nrows_s[w] = nrows;
    nrows = __builtin_amdgcn_readfirstlane(nrows);
    const int nrb = (nrows + 15) / 16;

    // ---- x tile loader: 128 rows x 32 columns = 512 chunks of 16 bytes, 2 per thread
    u32x4_t xr[2];
    auto gload = [&](int kc) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int ch = tid + 256 * u;
            const int r = ch >> 2, c = ch & 3;
            int64_t t = t0 + r;
            if (t >= a.T) t = a.T - 1;
            xr[u] = *reinterpret_cast<const u32x4_t*>(a.x + t * a.d + (int64_t)kc * kKC + 8 * c);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int ch = tid + 256 * u;
            const int r = ch >> 2, c = ch & 3;
            *reinterpret_cast<u32x4_t*>(&xs[buf][r * kXP + 8 * c]) = xr[u];
        }
    };

    f32x4_t acc[8][CB];
#pragma unroll
    for (int rb = 0; rb < 8; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const bf16_t* wb = a.wproj + (int64_t)(active ? hb : 0) * DH * a.d;
    const int nk = a.d / kKC;
    gload(0);
    __syncthreads();  // rows[] visible
    lstore(0);
    __syncthreads();
    // my gathered row indices for the 8 row blocks (lane's row = rows[16 rb + lane%16])
    int myrow[8];
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) myrow[rb] = rows[w][(16 * rb + (lane & 15)) & (kBM - 1)] & 0xff;

    bf16x8_t wf[CB];
    auto wload = [&](int kc) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
            wf[cb] = *reinterpret_cast<const bf16x8_t*>(wb + (int64_t)(16 * cb + (lane & 15)) * a.d + (int64_t)kc * kKC + 8 * (lane >> 4));
    };
    if (active) wload(0);
    for (int kc = 0; kc < nk; ++kc) {
        const int buf = kc & 1;
        if (kc + 1 < nk) gload(kc + 1);
        bf16x8_t wcur[CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) wcur[cb] = wf[cb];
        if (active && kc + 1 < nk) wload(kc + 1);
        if (active) {
            const uint16_t* xb = xs[buf];
#pragma unroll
            for (int rb = 0; rb < 8; ++rb) {
                if (rb < nrb) {
                    const bf16x8_t xf = *reinterpret_cast<const bf16x8_t*>(xb + myrow[rb] * kXP + 8 * (lane >> 4));
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) {
                        if (is_v)
                            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xf, wcur[cb], acc[rb][cb], 0, 0, 0);
                        else
                            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wcur[cb], xf, acc[rb][cb], 0, 0, 0);
                    }
                }
            }
        }
        if (kc + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }
    if (!active) return;

    // ---- epilogue
    const int64_t S = a.S;
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) {
        if (rb >= nrb) continue;
        if (!is_v) {
            // C^T tile: lane holds token column (lane & 15), head dims 16cb + 4(lane>>4) + 0..3
            const int li = 16 * rb + (lane & 15);
            const bool ok = li < nrows;
            const int packed = rows[w][li & (kBM - 1)];
            const int row = packed & 0xff, rank = packed >> 8;
            const int64_t t = t0 + row;
            const int64_t b = t / S, sp = t % S;
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
            bf16_t* dst;
            if (!is_expert) dst = a.Q + (((int64_t)b * a.H + a.G * a.k) * S + sp) * DH;  // shared head
            else dst = a.Q + (((int64_t)b * a.H + g_of * a.k + rank) * S + sp) * DH;
            const float qs = a.qscale;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const f32x4_t v = acc[rb][cb] * qs;
                u32x2_t pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                *reinterpret_cast<u32x2_t*>(dst + 16 * cb + 4 * (lane >> 4)) = pk;
            }
        } else {
            // C tile: lane holds head dim 16cb + (lane & 15), tokens 16rb + 4(lane>>4) + 0..3
            const int g = hb - GD;
            const int r0 = 16 * rb + 4 * (lane >> 4);
            const int64_t t = t0 + r0;
            const int64_t b = t / S, sp = t % S;
            const bool vec = (sp % 4 == 0) && (sp + 3 < S) && (t + 3 < a.T);
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const int dim = 16 * cb + (lane & 15);
                const f32x4_t v = acc[rb][cb];
                if (vec) {
                    bf16_t* dst = a.Vt + (((int64_t)b * a.G + g) * DH + dim) * a.S_pad + vt_pos(sp);
                    u32x2_t pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                    *reinterpret_cast<u32x2_t*>(dst) = pk;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t ti = t + i;
                        if (ti >= a.T) break;
                        const int64_t bi = ti / S, si = ti % S;
                        a.Vt[(((int64_t)bi * a.G + g) * DH + dim) * a.S_pad + vt_pos(si)] = from_f32<bf16_t>(v[i]);
                    }
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_proj_mfma(const GqeDims& D, const WorkPlan& P, const void* x, const void* packed,
                            const PackedLayout& pl, char* ws, hipStream_t st) {
    ProjArgs a{};
    a.x = (const bf16_t*)x;
    a.wproj = (const bf16_t*)((const char*)packed + pl.wproj);
    a.idx = (const int32_t*)(ws + P.idx);
    a.Q = (bf16_t*)(ws + P.q);
    a.K = (bf16_t*)(ws + P.kk);
    a.Vt = (bf16_t*)(ws + P.vt);
    a.kn = (float*)(ws + P.kn);
    a.qscale = (float)(1.4426950408889634 / std::sqrt((double)D.dh));
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
    const unsigned grid = (unsigned)((int64_t)a.ntiles * a.njobs);
    switch (D.dh) {
        case 32: proj_kernel<32><<<grid, 256, 0, st>>>(a); break;
        case 48: proj_kernel<48><<<grid, 256, 0, st>>>(a); break;
        case 64: proj_kernel<64><<<grid, 256, 0, st>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
