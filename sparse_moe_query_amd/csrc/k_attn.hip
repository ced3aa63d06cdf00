// Causal flash attention of the GQE layer on gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// GQE README "Algorithm Overview": the routed query heads of a group and the always-on shared
// head attend to the group's dense, unchanged KV head.  A work item is (batch b, group g, block of
// positions); its 256 query columns are all (position, head) pairs of the group's active heads, so
// every K/V tile staged in LDS serves the k routed heads (+ the shared head for its group) at once.
//
// Per wave: 64 query columns (two 32-column tiles).
//   S^T = K Q^T       v_mfma_f32_32x32x16_bf16 (d_h = 48 needs no padding: 3 k-steps of 16)
//   online softmax    per lane: one query column, 16 keys per 32-key subtile; the row maximum
//                     of a tile is the lane maximum combined with lane l^32 (v_permlane32_swap);
//                     the running maximum is only raised when it grows by more than 2^8 (lazy
//                     rescale), so the O rescale is rare
//   P -> B operand    probabilities are packed to bf16 and two v_permlane16_swap per register pair
//                     turn the 32x32 accumulator layout into the 16x16x32 B-operand layout; V^T is
//                     stored with keys slotted (vt_pos) so that one 16-byte LDS read gives each
//                     lane the eight keys its probabilities hold
//   O^T += V^T P^T    v_mfma_f32_16x16x32_bf16, d_h in 16-row blocks
//
// Work order: items sorted by causal key range, longest first (an in-kernel closed-form rank:
// every item has the same number of query columns, so its cost is its key range).
#include "gqe_common.h"
#include "gqe_internal.h"

namespace {

constexpr int kWaves = 4;
constexpr int kQW = 64;                // query columns per wave
constexpr int kCols = kWaves * kQW;    // query columns per work item
constexpr int kBN = GQE_KV_TILE;       // keys per LDS tile
constexpr float kLazy = 8.0f;          // raise the running max only when it grows by > 2^8

struct AttnArgs {
    const bf16_t* Q;
    const bf16_t* K;
    const bf16_t* Vt;
    bf16_t* O;
    int64_t S, S_pad;
    int B, G, H, k, skv, s;
    float scale_log2;  // log2(e) / sqrt(d_h)
    // schedule: up to two classes of groups (heads per group NH, positions per item P)
    int ncls;
    int nh[2], P[2], m[2], J[2], ngr[2];
    int single_group[2];  // class made of the shared head's group only
};

struct Item {
    int b, g, p0, np, nh;
};

__device__ __forceinline__ int64_t count_ge(const AttnArgs& a, int64_t e) {
    // number of items whose key range end E >= e (1 <= e <= S)
    int64_t n = 0;
    for (int c = 0; c < a.ncls; ++c) n += (int64_t)a.m[c] * (a.J[c] - (e - 1) / a.P[c]);
    return n;
}

__device__ Item decode_item(const AttnArgs& a, int64_t r) {
    int64_t lo = 1, hi = a.S;
    while (lo < hi) {
        const int64_t mid = (lo + hi + 1) / 2;
        if (count_ge(a, mid) > r) lo = mid;
        else hi = mid - 1;
    }
    const int64_t E = lo;
    int64_t o = r - (E == a.S ? 0 : count_ge(a, E + 1));
    Item it{0, 0, 0, 0, 1};
    for (int c = 0; c < a.ncls; ++c) {
        const bool has = (E == a.S) || (E % a.P[c] == 0);
        if (!has) continue;
        if (o < a.m[c]) {
            const int j = (E == a.S) ? a.J[c] - 1 : (int)(E / a.P[c]) - 1;
            const int pair = (int)o;
            if (a.single_group[c]) {
                it.b = pair;
                it.g = a.skv;
            } else {
                it.b = pair / a.ngr[c];
                const int gi = pair % a.ngr[c];
                it.g = (a.s && a.ncls == 2 && gi >= a.skv) ? gi + 1 : gi;
            }
            it.nh = a.nh[c];
            it.p0 = j * a.P[c];
            it.np = a.P[c];
            return it;
        }
        o -= a.m[c];
    }
    return it;  // unreachable for r < total
}

__device__ __forceinline__ float fmax3(float a, float b, float c) {
    return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}

template <int DH>
__global__ void __launch_bounds__(256, 2) attn_fwd_kernel(AttnArgs a) {
    constexpr int KS = DH / 16;        // k-steps of the 32x32x16 QK^T product
    constexpr int DB = DH / 16;        // 16-row blocks of d_h in the PV product
    constexpr int KP = DH + 8;         // LDS row pitch of K (elements)
    constexpr int VP = kBN + 8;        // LDS row pitch of V^T (elements)
    constexpr int KCH = kBN * DH / 8;  // 16-byte chunks per K tile
    constexpr int VCH = DH * kBN / 8;  // 16-byte chunks per V^T tile
    constexpr int LCH = (KCH + 255) / 256;
    __shared__ __align__(16) uint16_t ks_lds[2][kBN * KP];
    __shared__ __align__(16) uint16_t vs_lds[2][DH * VP];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Item it = decode_item(a, blockIdx.x);
    const int NH = it.nh;
    const int64_t S = a.S;
    const int64_t last_pos = min((int64_t)it.p0 + it.np, S) - 1;  // last query position of the item
    const int ntiles = (int)(last_pos / kBN) + 1;

    const bf16_t* Kg = a.K + ((int64_t)it.b * a.G + it.g) * a.S_pad * DH;
    const bf16_t* Vg = a.Vt + ((int64_t)it.b * a.G + it.g) * (int64_t)DH * a.S_pad;

    // ---------------------------------------------------------------- query columns of the lane
    int64_t posq[2];
    bool qvalid[2];
    int vhead[2];
    bf16x8_t qf[2][KS];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int c = w * kQW + qt * 32 + (lane & 31);
        const int p = c / NH, h = c % NH;
        const int64_t pos = (int64_t)it.p0 + p;
        qvalid[qt] = (p < it.np) && (pos < S);
        posq[qt] = qvalid[qt] ? pos : S - 1;
        vhead[qt] = h < a.k ? it.g * a.k + h : a.G * a.k;
        const bf16_t* qr = a.Q + (((int64_t)it.b * a.H + vhead[qt]) * S + posq[qt]) * DH + 8 * (lane >> 5);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) qf[qt][kk] = *reinterpret_cast<const bf16x8_t*>(qr + 16 * kk);
    }
    // key range of this wave
    const int cfirst = w * kQW, clast = w * kQW + kQW - 1;
    const int64_t wfirst = min((int64_t)it.p0 + cfirst / NH, S - 1);
    const int64_t wlast = min(min((int64_t)it.p0 + min(clast / NH, it.np - 1), S - 1), last_pos);
    const int wtiles = (int)(wlast / kBN) + 1;

    f32x4_t oacc[2][2][DB];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[qt][hf][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float mrun[2] = {-INFINITY, -INFINITY};
    float lsum[2] = {0.f, 0.f};

    // ---------------------------------------------------------------- tile loader
    u32x4_t kreg[LCH], vreg[LCH];
    auto gload = [&](int kt) {
#pragma unroll
        for (int u = 0; u < LCH; ++u) {
            const int ch = tid + 256 * u;
            if (ch < KCH) {
                const int r = ch / (DH / 8), c8 = ch % (DH / 8);
                kreg[u] = *reinterpret_cast<const u32x4_t*>(Kg + ((int64_t)kt * kBN + r) * DH + 8 * c8);
            }
            if (ch < VCH) {
                const int r = ch / (kBN / 8), c8 = ch % (kBN / 8);
                vreg[u] = *reinterpret_cast<const u32x4_t*>(Vg + (int64_t)r * a.S_pad + (int64_t)kt * kBN + 8 * c8);
                if ((int64_t)(kt + 1) * kBN > S) {
                    // keys past the sequence end hold no data: zero them (their P is 0)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int q = (8 * c8 + e) & 31;
                        const int sl = q >> 2;
                        const int key = (((sl & 3) << 1) | (sl >> 2)) * 4 + (q & 3);
                        const int64_t kidx = (int64_t)kt * kBN + ((8 * c8 + e) & ~31) + key;
                        if (kidx >= S) {
                            const uint32_t msk = (e & 1) ? 0x0000ffffu : 0xffff0000u;
                            vreg[u][e >> 1] &= msk;
                        }
                    }
                }
            }
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int u = 0; u < LCH; ++u) {
            const int ch = tid + 256 * u;
            if (ch < KCH) {
                const int r = ch / (DH / 8), c8 = ch % (DH / 8);
                *reinterpret_cast<u32x4_t*>(&ks_lds[buf][r * KP + 8 * c8]) = kreg[u];
            }
            if (ch < VCH) {
                const int r = ch / (kBN / 8), c8 = ch % (kBN / 8);
                *reinterpret_cast<u32x4_t*>(&vs_lds[buf][r * VP + 8 * c8]) = vreg[u];
            }
        }
    };

    gload(0);
    lstore(0);
    __syncthreads();

    for (int kt = 0; kt < ntiles; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < ntiles) gload(kt + 1);
        if (kt < wtiles) {
            const uint16_t* kb = ks_lds[buf];
            const uint16_t* vb = vs_lds[buf];
            // S^T tiles: [key subtile][query tile]
            f32x16_t sacc[2][2];
#pragma unroll
            for (int kst = 0; kst < 2; ++kst) {
                bf16x8_t kf[KS];
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
                    kf[kk] = *reinterpret_cast<const bf16x8_t*>(kb + (32 * kst + (lane & 31)) * KP + 16 * kk + 8 * (lane >> 5));
#pragma unroll
                for (int qt = 0; qt < 2; ++qt) {
                    f32x16_t acc = {};
#pragma unroll
                    for (int kk = 0; kk < KS; ++kk)
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[qt][kk], acc, 0, 0, 0);
                    sacc[kst][qt] = acc;
                }
            }
            const bool diag = (int64_t)kt * kBN + kBN - 1 > wfirst;
            uint32_t pb[2][2][8];  // packed bf16 probabilities [qt][kst][reg]
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                if (diag) {
#pragma unroll
                    for (int kst = 0; kst < 2; ++kst)
#pragma unroll
                        for (int j = 0; j < 16; ++j) {
                            const int64_t kidx = (int64_t)kt * kBN + 32 * kst + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
                            if (kidx > posq[qt]) sacc[kst][qt][j] = -INFINITY;
                        }
                }
                float mx = -INFINITY;
#pragma unroll
                for (int kst = 0; kst < 2; ++kst)
#pragma unroll
                    for (int j = 0; j < 16; j += 2) mx = fmax3(mx, sacc[kst][qt][j], sacc[kst][qt][j + 1]);
                {
                    const uint32_t mb = __float_as_uint(mx);
                    auto sw = __builtin_amdgcn_permlane32_swap(mb, mb, false, false);
                    mx = __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
                }
                const float cand = mx * a.scale_log2;
                const bool need = cand > mrun[qt] + kLazy;
                if (__builtin_amdgcn_ballot_w64(need)) {
                    const float mnew = need ? cand : mrun[qt];
                    const float alpha = need ? __builtin_amdgcn_exp2f(mrun[qt] - mnew) : 1.0f;
                    mrun[qt] = mnew;
                    lsum[qt] *= alpha;
                    const float aa = __shfl(alpha, lane & 15);
                    const float ab = __shfl(alpha, 16 + (lane & 15));
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        oacc[qt][0][db] *= aa;
                        oacc[qt][1][db] *= ab;
                    }
                }
                const float nm = -mrun[qt];
                float ls = 0.f;
#pragma unroll
                for (int kst = 0; kst < 2; ++kst) {
                    float pv[16];
#pragma unroll
                    for (int j = 0; j < 16; ++j) {
                        pv[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kst][qt][j], a.scale_log2, nm));
                        ls += pv[j];
                    }
                    uint32_t X[4], Y[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        X[i] = pack_bf16x2(pv[2 * i], pv[2 * i + 1]);
                        Y[i] = pack_bf16x2(pv[8 + 2 * i], pv[9 + 2 * i]);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        auto r = __builtin_amdgcn_permlane16_swap(X[i], Y[i], false, false);
                        pb[qt][kst][i] = r[0];      // query block 32qt + 0..15
                        pb[qt][kst][4 + i] = r[1];  // query block 32qt + 16..31
                    }
                }
                lsum[qt] += ls;
            }
            // O^T += V^T P^T
#pragma unroll
            for (int kst = 0; kst < 2; ++kst) {
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const bf16x8_t vf = *reinterpret_cast<const bf16x8_t*>(vb + (16 * db + (lane & 15)) * VP + 32 * kst + 8 * (lane >> 4));
#pragma unroll
                    for (int qt = 0; qt < 2; ++qt) {
                        u32x4_t ba = {pb[qt][kst][0], pb[qt][kst][1], pb[qt][kst][2], pb[qt][kst][3]};
                        u32x4_t bb = {pb[qt][kst][4], pb[qt][kst][5], pb[qt][kst][6], pb[qt][kst][7]};
                        oacc[qt][0][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, __builtin_bit_cast(bf16x8_t, ba), oacc[qt][0][db], 0, 0, 0);
                        oacc[qt][1][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, __builtin_bit_cast(bf16x8_t, bb), oacc[qt][1][db], 0, 0, 0);
                    }
                }
            }
        }
        if (kt + 1 < ntiles) lstore(buf ^ 1);
        __syncthreads();
    }

    // ---------------------------------------------------------------- normalise and store
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const uint32_t lb = __float_as_uint(lsum[qt]);
        auto sw = __builtin_amdgcn_permlane32_swap(lb, lb, false, false);
        const float ltot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const float inv = 1.0f / ltot;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int src = 16 * hf + (lane & 15);  // S-layout lane holding this O column
            const float sc = __shfl(inv, src);
            const int c = w * kQW + qt * 32 + 16 * hf + (lane & 15);
            const int p = c / NH, h = c % NH;
            const int64_t pos = (int64_t)it.p0 + p;
            if (p >= it.np || pos >= S) continue;
            const int v = h < a.k ? it.g * a.k + h : a.G * a.k;
            bf16_t* orow = a.O + (((int64_t)it.b * S + pos) * a.H + v) * DH + 4 * (lane >> 4);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const f32x4_t o = oacc[qt][hf][db] * sc;
                u32x2_t pk = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
                *reinterpret_cast<u32x2_t*>(orow + 16 * db) = pk;
            }
        }
    }
}

}  // namespace

hipError_t launch_attn_mfma(const GqeDims& D, const WorkPlan& P, char* ws, hipStream_t st) {
    AttnArgs a{};
    a.Q = (const bf16_t*)(ws + P.q);
    a.K = (const bf16_t*)(ws + P.kk);
    a.Vt = (const bf16_t*)(ws + P.vt);
    a.O = (bf16_t*)(ws + P.o);
    a.S = P.S;
    a.S_pad = P.S_pad;
    a.B = (int)P.B;
    a.G = D.G;
    a.H = D.H;
    a.k = D.k;
    a.skv = D.skv;
    a.s = D.s;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D.dh));
    int64_t total = 0;
    auto add_class = [&](int nh, int ngroups, bool single) {
        const int c = a.ncls++;
        a.nh[c] = nh;
        a.P[c] = kCols / nh;
        a.ngr[c] = ngroups;
        a.m[c] = (int)P.B * ngroups;
        a.J[c] = (int)ceil_div(P.S, a.P[c]);
        a.single_group[c] = single ? 1 : 0;
        total += (int64_t)a.m[c] * a.J[c];
    };
    if (D.s) {
        add_class(D.k + 1, 1, true);
        if (D.G > 1) add_class(D.k, D.G - 1, false);
    } else {
        add_class(D.k, D.G, false);
    }
    if (total <= 0 || total > 0x7fffffff) return hipErrorInvalidValue;
    switch (D.dh) {
        case 32: attn_fwd_kernel<32><<<(unsigned)total, 256, 0, st>>>(a); break;
        case 48: attn_fwd_kernel<48><<<(unsigned)total, 256, 0, st>>>(a); break;
        case 64: attn_fwd_kernel<64><<<(unsigned)total, 256, 0, st>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
