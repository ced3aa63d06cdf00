// Causal flash attention of the GQE layer on gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// GQE README "Algorithm Overview": the routed query heads of a group and the always-on shared
// head attend to the group's dense, unchanged KV head.  A work item is (batch b, group g, block of
// positions); its 256 query columns are all (position, head) pairs of the group's active heads, so
// every K/V tile staged in LDS serves the k routed heads (+ the shared head for its group) at once.
//
// Per wave: 64 query columns (two 32-column tiles), 64-key tiles.
//   S^T = K Q^T     v_mfma_f32_32x32x16_bf16 (d_h = 48 needs no padding: 3 k-steps of 16).  The
//                   queries arrive pre-scaled by log2(e)/sqrt(d_h), so S is in log2 units.
//   softmax         per lane: one query column, 16 keys per 32-key subtile.  Fast tiles: when the
//                   Cauchy-Schwarz bound max|q| * max|k| <= 64 holds for the wave and tile (the
//                   key norms come from the projection) and the running offset is 0, P = exp2(S)
//                   directly (no maximum, no subtraction: one exp2 and half a convert per score).
//                   Otherwise the standard online softmax runs (lane maximum combined with lane
//                   l^32 by v_permlane32_swap; the offset is raised lazily, only when it grows by
//                   more than 2^8, so O is rarely rescaled).
//   P -> B operand  bf16-packed and re-laid by two v_permlane16_swap per register pair into the
//                   16x16x32 B layout; V^T is stored with keys slotted (vt_pos) so that one 16-byte
//                   LDS read gives each lane the eight keys its probabilities hold.
//   O^T += V^T P^T  v_mfma_f32_16x16x32_bf16 over d_h in 16-row blocks plus one block whose first
//                   row is all ones: the matrix core also forms the row sums, from the same
//                   bf16 P that multiplies V.
// Long causal ranges are split into KV chunks (separate work items); each chunk stores its
// unnormalised O, row sum and offset, and the chunk that finishes last (per-item atomic counter,
// no waiting) merges them.  Work order: items by causal range, longest first.
#include "gqe_common.h"
#include "gqe_internal.h"

namespace {

constexpr int kWaves = 4;
constexpr int kQW = 64;                // query columns per wave
constexpr int kCols = kWaves * kQW;    // query columns per work item
constexpr int kBN = GQE_KV_TILE;       // keys per LDS tile
constexpr float kLazy = 8.0f;          // raise the running offset only when it grows by > 2^8
constexpr float kFastBound = 64.0f;    // |S| <= 64 (log2 units) keeps exp2 in range without offset

struct AttnArgs {
    const bf16_t* Q;
    const bf16_t* K;
    const bf16_t* Vt;
    const float* kn;      // per-key norms [B][G][S_pad]
    bf16_t* O;
    float* part;          // split-KV partials
    int* counters;        // split-KV arrival counters, one per item
    int64_t S, S_pad;
    int B, G, H, k, skv, s;
    int kch;              // tiles per KV chunk
    int ncmax;            // chunks of the longest item (grid = items * ncmax)
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

__global__ void zero_ints_kernel(int* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o));
    return v;
}

template <int DH>
__global__ void __launch_bounds__(256, 2) attn_fwd_kernel(AttnArgs a) {
    constexpr int KS = DH / 16;        // k-steps of the 32x32x16 QK^T product
    constexpr int DB = DH / 16;        // 16-row blocks of d_h in the PV product
    constexpr int DBX = DB + 1;        // plus the row-sum block
    constexpr int KP = DH + 8;         // LDS row pitch of K (elements)
    constexpr int VP = kBN + 8;        // LDS row pitch of V^T (elements)
    constexpr int KCH = kBN * DH / 8;  // 16-byte chunks per K tile
    constexpr int VCH = DH * kBN / 8;  // 16-byte chunks per V^T tile
    constexpr int LCH = (KCH + 255) / 256;
    constexpr int NREG = 2 * 2 * DBX * 4;  // partial O floats per lane
    __shared__ __align__(16) uint16_t ks_lds[2][kBN * KP];
    __shared__ __align__(16) uint16_t vs_lds[2][(DH + 16) * VP];
    __shared__ int last_flag;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t rank = blockIdx.x / a.ncmax;
    const int chunk = blockIdx.x % a.ncmax;
    const Item it = decode_item(a, rank);
    const int NH = it.nh;
    const int64_t S = a.S;
    const int64_t last_pos = min((int64_t)it.p0 + it.np, S) - 1;  // last query position of the item
    const int ntiles_item = (int)(last_pos / kBN) + 1;
    const int nchunks = (ntiles_item + a.kch - 1) / a.kch;
    if (chunk >= nchunks) return;  // uniform for the whole block
    const int kt_begin = chunk * a.kch;
    const int kt_end = min(ntiles_item, kt_begin + a.kch);

    const bf16_t* Kg = a.K + ((int64_t)it.b * a.G + it.g) * a.S_pad * DH;
    const bf16_t* Vg = a.Vt + ((int64_t)it.b * a.G + it.g) * (int64_t)DH * a.S_pad;
    const float* kng = a.kn + ((int64_t)it.b * a.G + it.g) * a.S_pad;

    // ---------------------------------------------------------------- query columns of the lane
    int64_t posq[2];
    bf16x8_t qf[2][KS];
    float qsq[2];  // sum of squares of the lane's half of the query column's dims
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int c = w * kQW + qt * 32 + (lane & 31);
        const int p = c / NH, h = c % NH;
        const int64_t pos = (int64_t)it.p0 + p;
        const bool valid = (p < it.np) && (pos < S);
        posq[qt] = valid ? pos : S - 1;
        const int vh = h < a.k ? it.g * a.k + h : a.G * a.k;
        const bf16_t* qr = a.Q + (((int64_t)it.b * a.H + vh) * S + posq[qt]) * DH + 8 * (lane >> 5);
        float ss = 0.f;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            qf[qt][kk] = *reinterpret_cast<const bf16x8_t*>(qr + 16 * kk);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = (float)qf[qt][kk][e];
                ss += v * v;
            }
        }
        qsq[qt] = ss;
    }
    // |q|^2 = (this half) + (other half) <= 2 max(half): a bound on every query norm of the wave
    const float qmax_w = sqrtf(wave_max(__builtin_fmaxf(qsq[0], qsq[1]) * 2.0f));
    // key range of this wave
    const int cfirst = w * kQW, clast = w * kQW + kQW - 1;
    const int64_t wfirst = min((int64_t)it.p0 + cfirst / NH, S - 1);
    const int64_t wlast = min(min((int64_t)it.p0 + min(clast / NH, it.np - 1), S - 1), last_pos);
    const int wtiles = (int)(wlast / kBN) + 1;

    f32x4_t oacc[2][2][DBX];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int db = 0; db < DBX; ++db) oacc[qt][hf][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float mrun[2] = {-INFINITY, -INFINITY};
    bool offset_zero = true;  // wave-uniform: every lane's offset is 0 or unset

    // row-sum block of V^T: first row ones, the rest zeros (both buffers, written once)
    for (int i = tid; i < 2 * 16 * kBN; i += 256) {
        const int buf = i / (16 * kBN), r = (i / kBN) % 16, c = i % kBN;
        vs_lds[buf][(DH + r) * VP + c] = r == 0 ? (uint16_t)0x3f80 : (uint16_t)0;
    }

    // ---------------------------------------------------------------- tile loader
    u32x4_t kreg[LCH], vreg[LCH];
    float kn_next = 0.f;  // norm of key kt*64 + lane of the tile being prefetched
    auto gload = [&](int kt) {
        const int64_t kl = (int64_t)kt * kBN + lane;
        kn_next = kl < S ? kng[kl] : 0.f;
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

    gload(kt_begin);
    lstore(0);
    // largest key norm of the current tile (wave-uniform); the next tile's is formed while this
    // tile computes, so neither the load nor the cross-lane maximum sits on the critical path
    float kmax_cur = wave_max(kn_next);
    __syncthreads();

    for (int kt = kt_begin; kt < kt_end; ++kt) {
        const int buf = (kt - kt_begin) & 1;
        if (kt + 1 < kt_end) gload(kt + 1);
        if (kt < wtiles) {
            const uint16_t* kb = ks_lds[buf];
            const uint16_t* vb = vs_lds[buf];
            const bool fast = offset_zero && (qmax_w * kmax_cur * 1.02f <= kFastBound);
            // K fragments of both 32-key subtiles (shared by the two query tiles)
            bf16x8_t kf[2][KS];
#pragma unroll
            for (int kst = 0; kst < 2; ++kst)
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
                    kf[kst][kk] = *reinterpret_cast<const bf16x8_t*>(kb + (32 * kst + (lane & 31)) * KP + 16 * kk + 8 * (lane >> 5));
            const bool diag = (int64_t)kt * kBN + kBN - 1 > wfirst;
            uint32_t pb[2][2][8];  // packed bf16 probabilities [qt][kst][reg]
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                // S^T tiles of this query tile: [key subtile]
                f32x16_t sacc[2];
#pragma unroll
                for (int kst = 0; kst < 2; ++kst) {
                    f32x16_t acc = {};
#pragma unroll
                    for (int kk = 0; kk < KS; ++kk)
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kst][kk], qf[qt][kk], acc, 0, 0, 0);
                    sacc[kst] = acc;
                }
                if (diag) {
#pragma unroll
                    for (int kst = 0; kst < 2; ++kst)
#pragma unroll
                        for (int j = 0; j < 16; ++j) {
                            const int64_t kidx = (int64_t)kt * kBN + 32 * kst + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
                            if (kidx > posq[qt]) sacc[kst][j] = -INFINITY;
                        }
                }
                float nm = 0.f;
                if (fast) {
                    mrun[qt] = 0.f;  // from unset (nothing accumulated) or already 0
                } else {
                    float mx = -INFINITY;
#pragma unroll
                    for (int kst = 0; kst < 2; ++kst)
#pragma unroll
                        for (int j = 0; j < 16; j += 2) mx = fmax3(mx, sacc[kst][j], sacc[kst][j + 1]);
                    {
                        const uint32_t mb = __float_as_uint(mx);
                        auto sw = __builtin_amdgcn_permlane32_swap(mb, mb, false, false);
                        mx = __builtin_fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
                    }
                    const bool need = mx > mrun[qt] + kLazy;
                    if (__builtin_amdgcn_ballot_w64(need)) {
                        const float mnew = need ? mx : mrun[qt];
                        const float alpha = (need && mrun[qt] != -INFINITY) ? __builtin_amdgcn_exp2f(mrun[qt] - mnew)
                                                                             : (need ? 0.f : 1.f);
                        mrun[qt] = mnew;
                        const float aa = __shfl(alpha, lane & 15);
                        const float ab = __shfl(alpha, 16 + (lane & 15));
#pragma unroll
                        for (int db = 0; db < DBX; ++db) {
                            oacc[qt][0][db] *= aa;
                            oacc[qt][1][db] *= ab;
                        }
                    }
                    nm = mrun[qt] == -INFINITY ? 0.f : -mrun[qt];
                }
#pragma unroll
                for (int kst = 0; kst < 2; ++kst) {
                    float pv[16];
                    if (fast) {
#pragma unroll
                        for (int j = 0; j < 16; ++j) pv[j] = __builtin_amdgcn_exp2f(sacc[kst][j]);
                    } else {
#pragma unroll
                        for (int j = 0; j < 16; ++j) pv[j] = __builtin_amdgcn_exp2f(sacc[kst][j] + nm);
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
            }
            if (!fast) offset_zero = !__builtin_amdgcn_ballot_w64(mrun[0] != 0.f && mrun[0] != -INFINITY) &&
                                     !__builtin_amdgcn_ballot_w64(mrun[1] != 0.f && mrun[1] != -INFINITY);
            // O^T += V^T P^T (last block: row sums)
#pragma unroll
            for (int kst = 0; kst < 2; ++kst) {
#pragma unroll
                for (int db = 0; db < DBX; ++db) {
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
        if (kt + 1 < kt_end) {
            lstore(buf ^ 1);
            kmax_cur = wave_max(kn_next);
        }
        __syncthreads();
    }

    // offsets in the O layout: lane holds column (lane & 15) of block (qt, hf); the S layout lane
    // holding that column is 16 hf + (lane & 15)
    float mo[2][2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) mo[qt][hf] = __shfl(mrun[qt], 16 * hf + (lane & 15));

    if (nchunks > 1) {
        // ---------------------------------------------------------- split-KV: store, count, merge
        const int64_t slot_base = rank * (int64_t)a.ncmax;
        float* mine = a.part + ((slot_base + chunk) * 256 + w * 64 + lane) * (NREG + 4);
        int r = 0;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
                for (int db = 0; db < DBX; ++db)
#pragma unroll
                    for (int i = 0; i < 4; ++i) mine[r++] = oacc[qt][hf][db][i];
                mine[NREG + 2 * qt + hf] = mo[qt][hf];
            }
        __threadfence();
        __syncthreads();
        if (tid == 0) {
            const int prev = atomicAdd(&a.counters[rank], 1);
            last_flag = (prev == nchunks - 1) ? 1 : 0;
        }
        __syncthreads();
        if (!last_flag) return;
        __threadfence();
        // merge every chunk's partial into oacc (max offset, rescale, add)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                float M = -INFINITY;
                for (int c = 0; c < nchunks; ++c) {
                    const float* pc = a.part + ((slot_base + c) * 256 + w * 64 + lane) * (NREG + 4);
                    M = __builtin_fmaxf(M, pc[NREG + 2 * qt + hf]);
                }
                if (M == -INFINITY) M = 0.f;
#pragma unroll
                for (int db = 0; db < DBX; ++db) oacc[qt][hf][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                for (int c = 0; c < nchunks; ++c) {
                    const float* pc = a.part + ((slot_base + c) * 256 + w * 64 + lane) * (NREG + 4);
                    const float mc = pc[NREG + 2 * qt + hf];
                    const float sc = mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc - M);
                    const int base = (qt * 2 + hf) * DBX * 4;
#pragma unroll
                    for (int db = 0; db < DBX; ++db)
#pragma unroll
                        for (int i = 0; i < 4; ++i) oacc[qt][hf][db][i] += sc * pc[base + db * 4 + i];
                }
            }
        if (tid == 0) a.counters[rank] = 0;  // ready for the next forward
    }

    // ---------------------------------------------------------------- normalise and store
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            // row sum: row 0 of the last block, held by the lane of this column in lane group 0
            const float lsum = __shfl(oacc[qt][hf][DB][0], lane & 15);
            const float sc = 1.0f / lsum;
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

// Workspace needs of the attention kernel for one forward (split-KV partials and counters).
void attn_plan(const GqeDims& D, int64_t B, int64_t S, int64_t* items, int* ncmax, int* kch) {
    int64_t total = 0, tiles = 0;
    auto cls = [&](int nh, int ngroups) {
        const int P = kCols / nh;
        const int64_t J = ceil_div(S, P);
        total += B * ngroups * J;
        for (int64_t j = 0; j < J; ++j) {
            const int64_t E = std::min<int64_t>((j + 1) * P, S);
            tiles += B * ngroups * ceil_div(E, kBN);
        }
    };
    if (D.s) {
        cls(D.k + 1, 1);
        if (D.G > 1) cls(D.k, D.G - 1);
    } else {
        cls(D.k, D.G);
    }
    // chunk length: at least 32 tiles, else about a quarter of the average load of one of the 512
    // concurrent work items (2 per CU), so that the longest item no longer dominates
    const int64_t slots = 512;
    const int64_t c = std::max<int64_t>(32, tiles / (slots * 4) * 2);
    const int64_t longest = ceil_div(S, kBN);
    *kch = (int)std::min<int64_t>(c, longest);
    *ncmax = (int)ceil_div(longest, *kch);
    *items = total;
}

size_t attn_partial_bytes(const GqeDims& D, int64_t items, int ncmax) {
    if (ncmax <= 1) return 0;
    const int DBX = D.dh / 16 + 1;
    return (size_t)items * ncmax * 256 * (2 * 2 * DBX * 4 + 4) * sizeof(float);
}

hipError_t launch_attn_mfma(const GqeDims& D, const WorkPlan& P, char* ws, hipStream_t st) {
    AttnArgs a{};
    a.Q = (const bf16_t*)(ws + P.q);
    a.K = (const bf16_t*)(ws + P.kk);
    a.Vt = (const bf16_t*)(ws + P.vt);
    a.kn = (const float*)(ws + P.kn);
    a.O = (bf16_t*)(ws + P.o);
    a.part = (float*)(ws + P.attn_part);
    a.counters = (int*)(ws + P.attn_cnt);
    a.S = P.S;
    a.S_pad = P.S_pad;
    a.B = (int)P.B;
    a.G = D.G;
    a.H = D.H;
    a.k = D.k;
    a.skv = D.skv;
    a.s = D.s;
    a.kch = P.attn_kch;
    a.ncmax = P.attn_ncmax;
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
    const int64_t grid = total * a.ncmax;
    if (total != P.attn_items || grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidValue;
    if (a.ncmax > 1) {
        zero_ints_kernel<<<(unsigned)ceil_div(total, 256), 256, 0, st>>>(a.counters, total);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    switch (D.dh) {
        case 32: attn_fwd_kernel<32><<<(unsigned)grid, 256, 0, st>>>(a); break;
        case 48: attn_fwd_kernel<48><<<(unsigned)grid, 256, 0, st>>>(a); break;
        case 64: attn_fwd_kernel<64><<<(unsigned)grid, 256, 0, st>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
