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
//   P -> A operand  bf16-packed straight from the score registers: each lane holds, per 16-key
//                   chunk, the eight keys that V^T's slotting (vt_pos) puts in one 16-byte read.
//   O += P [V|1|0]  v_mfma_f32_32x32x16_bf16 over 32-wide column blocks of V (d_h = 48: two blocks,
//                   the second's spare columns carry a column of ones), so the matrix core also
//                   forms the row sums, from the same bf16 P that multiplies V.
// Work order: items by causal range, longest first (LPT over the concurrent work-group slots).
#include <type_traits>

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
    const float* knt;     // per-tile maximum key norm [B][G][S_pad / 64]
    bf16_t* O;
    int64_t S, S_pad;
    int B, G, H, k, skv, s;
    // schedule: up to two classes of groups (heads per group NH, positions per item P)
    int ncls;
    int nh[2], P[2], m[2], J[2], ngr[2];
    int single_group[2];  // class made of the shared head's group only
};

struct Item {
    int b, g, p0, np, nh;
};

__device__ __forceinline__ int count_ge(const AttnArgs& a, int e) {
    // number of items whose key range end E >= e (1 <= e <= S); 32-bit: items and S fit easily
    int n = 0;
    for (int c = 0; c < a.ncls; ++c) n += a.m[c] * (a.J[c] - (int)((uint32_t)(e - 1) / (uint32_t)a.P[c]));
    return n;
}

__device__ Item decode_item(const AttnArgs& a, int r) {
    const int S = (int)a.S;
    int lo = 1, hi = S;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (count_ge(a, mid) > r) lo = mid;
        else hi = mid - 1;
    }
    const int E = lo;
    int o = r - (E == S ? 0 : count_ge(a, E + 1));
    Item it{0, 0, 0, 0, 1};
    for (int c = 0; c < a.ncls; ++c) {
        const bool has = (E == S) || ((uint32_t)E % (uint32_t)a.P[c] == 0);
        if (!has) continue;
        if (o < a.m[c]) {
            const int j = (E == S) ? a.J[c] - 1 : (int)((uint32_t)E / (uint32_t)a.P[c]) - 1;
            const int pair = o;
            if (a.single_group[c]) {
                it.b = pair;
                it.g = a.skv;
            } else {
                it.b = (int)((uint32_t)pair / (uint32_t)a.ngr[c]);
                const int gi = pair - it.b * a.ngr[c];
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

// Per forward, before the attention kernel: the largest key norm of every 64-key tile (keys past
// the sequence end excluded), and zero V^T at the padding keys [S, S_pad) so that P = 0 there
// meets finite values.
__global__ void __launch_bounds__(256) attn_prep_kernel(const float* __restrict__ kn, float* __restrict__ knt,
                                                       bf16_t* __restrict__ Vt, int64_t BG, int64_t S,
                                                       int64_t S_pad, int dh) {
    const int64_t ntile = S_pad / 64;
    const int64_t pad = S_pad - S;
    const int64_t n1 = BG * ntile, n2 = BG * dh * pad;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n1 + n2;
         i += (int64_t)gridDim.x * blockDim.x) {
        if (i < n1) {
            const int64_t bg = i / ntile, t = i % ntile;
            const f32x4_t* p = reinterpret_cast<const f32x4_t*>(kn + bg * S_pad + t * 64);
            float m = 0.f;
#pragma unroll 4
            for (int q = 0; q < 16; ++q) {
                const f32x4_t v = p[q];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (t * 64 + 4 * q + e < S) m = fmaxf(m, v[e]);
            }
            knt[i] = m;
        } else {
            const int64_t j = i - n1;
            const int64_t row = j / pad, s = S + j % pad;  // row = bg * dh + head dim
            Vt[row * S_pad + vt_pos(s)] = bf16_t{0};
        }
    }
}

// LDS layout of a key row: pitch in 16-byte chunks and XOR swizzle of the chunk order, chosen per
// head dim so that a fragment read (sixteen lanes per LDS cycle, sixteen consecutive rows, same
// logical chunk) touches sixteen distinct 16-byte bank groups of the 256-byte bank row.
template <int DH>
__host__ __device__ constexpr int kpitch() { return DH == 48 ? 7 : DH / 8; }  // 48: odd pitch
template <int DH>
__device__ __forceinline__ int kswz(int r) {
    if constexpr (DH == 64) return (r >> 1) & 7;
    else if constexpr (DH == 32) return (r >> 2) & 3;
    else return 0;
}
// V^T rows (128 bytes): rows 2m and 2m+1 sit in different halves of the bank row, the XOR spreads
// eight such pairs
__device__ __forceinline__ int vswz(int n) { return (n >> 1) & 7; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o));
    return v;
}

// softmax of one query tile's S^T (32 keys x 32 columns per kst, lane = column) -> P packed to
// bf16 as A operands of the 32x32x16 P.V product: pa[2 kst + u] holds, for the lane's column, the
// eight keys of 16-key chunk u of subtile kst that the score layout left in this lane (register
// order = the key order of V^T's slotting).  FAST: P = exp2(S) (the range test holds and the offset
// is 0).  diag: keys past the lane's position are masked.  Rescales the tile's O accumulators when
// the offset rises (alpha of each accumulator row fetched from the lane that owns that column).
template <int NCB, bool FAST>
__device__ __forceinline__ void softmax_tile(f32x16_t (&sacc)[2], float& mrun, f32x16_t (&oacc)[NCB],
                                             bf16x8_t (&pa)[4], bool diag, int key0, int pos, int lane) {
    if (diag) {
        // key index of register j: key0 + 32 kst + 8 (j / 4) + 4 (lane / 32) + j % 4
        const int lim = pos - key0 - 4 * (lane >> 5);
#pragma unroll
        for (int kst = 0; kst < 2; ++kst)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (32 * kst + 8 * (j >> 2) + (j & 3) > lim) sacc[kst][j] = -INFINITY;
    }
    float nm = 0.f;
    if (!FAST) {
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
        const bool need = mx > mrun + kLazy;
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float mnew = need ? mx : mrun;
            const float alpha = (need && mrun != -INFINITY) ? __builtin_amdgcn_exp2f(mrun - mnew) : (need ? 0.f : 1.f);
            mrun = mnew;
            // accumulator register j of this lane is query row 8 (j / 4) + 4 (lane / 32) + j % 4,
            // whose alpha lives in the lane of that column
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float aj = __shfl(alpha, 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3));
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) oacc[cb][j] *= aj;
            }
        }
        nm = mrun == -INFINITY ? 0.f : -mrun;
    } else {
        mrun = 0.f;  // from unset (nothing accumulated) or already 0
    }
#pragma unroll
    for (int kst = 0; kst < 2; ++kst) {
        float pv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) pv[j] = __builtin_amdgcn_exp2f(FAST ? sacc[kst][j] : sacc[kst][j] + nm);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const u32x4_t pk = {pack_bf16x2(pv[8 * u + 0], pv[8 * u + 1]), pack_bf16x2(pv[8 * u + 2], pv[8 * u + 3]),
                                pack_bf16x2(pv[8 * u + 4], pv[8 * u + 5]), pack_bf16x2(pv[8 * u + 6], pv[8 * u + 7])};
            pa[2 * kst + u] = __builtin_bit_cast(bf16x8_t, pk);
        }
    }
}

template <int DH>
__global__ void __launch_bounds__(256, 2) attn_fwd_kernel(AttnArgs a) {
    constexpr int KS = DH / 16;        // k-steps of the 32x32x16 QK^T product
    constexpr int NCB = DH / 32 + 1;   // 32-wide column blocks of [V | 1 | 0] in the P.V product
    constexpr int KC8 = DH / 8;        // 16-byte chunks per key row
    constexpr int KP = kpitch<DH>();   // LDS pitch of a key row in chunks (>= KC8)
    constexpr int TILE_K = kBN * KP * 8;  // elements of a K tile in LDS (chunk-swizzled)
    constexpr int TILE_V = DH * kBN;   // elements of a V^T tile (unpadded, chunk-swizzled)
    constexpr int SEGK = TILE_K * 2 / 1024;  // 1 KB segments per tile (one wave-wide load each)
    constexpr int SEGV = TILE_V * 2 / 1024;
    constexpr int LK = (SEGK + 3) / 4;       // direct loads per wave per tile (same for every wave)
    constexpr int LV = (SEGV + 3) / 4;
    constexpr int NSTAGE = 3;
    constexpr int XR = NCB * 32 - DH;        // rows of the last block past d_h: row DH is ones
    __shared__ __align__(1024) uint16_t ks_lds[NSTAGE][TILE_K];
    __shared__ __align__(1024) uint16_t vs_lds[NSTAGE][TILE_V];
    __shared__ __align__(1024) uint16_t one_lds[XR * kBN];  // rows DH.. of [V | 1 | 0]^T

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const Item it = decode_item(a, (int)blockIdx.x);
    const int NH = it.nh;
    const int S = (int)a.S;  // the host limits a call to 2^28 tokens
    const int last_pos = min(it.p0 + it.np, S) - 1;  // last query position of the item
    const int kt_end = last_pos / kBN + 1;

    const bf16_t* Kg = a.K + ((int64_t)it.b * a.G + it.g) * a.S_pad * DH;
    const bf16_t* Vg = a.Vt + ((int64_t)it.b * a.G + it.g) * (int64_t)DH * a.S_pad;

    // ---------------------------------------------------------------- query columns of the lane
    bf16x8_t qf[2][KS];
    int posq[2];
    float mrun[2] = {-INFINITY, -INFINITY};
    float qsq[2];  // sum of squares of the lane's half of the query column's dims
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int c = w * kQW + qt * 32 + (lane & 31);
        const int p = c / NH, h = c % NH;
        const int pos = it.p0 + p;
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
    const int wfirst = min(it.p0 + cfirst / NH, S - 1);
    const int wlast = min(min(it.p0 + min(clast / NH, it.np - 1), S - 1), last_pos);
    const int wtiles = wlast / kBN + 1;

    // O accumulators: [qt][column block], 32 query rows x 32 columns of [V | 1 | 0] each
    f32x16_t oacc[2][NCB];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) oacc[qt][cb] = f32x16_t{};
    bool offset_zero = true;  // wave-uniform: every lane's offset is 0 or unset

    // rows DH.. of the [V | 1 | 0]^T operand: row DH all ones, the rest zero
    for (int i = tid; i < XR * kBN; i += 256) one_lds[i] = (i < kBN) ? (uint16_t)0x3f80 : (uint16_t)0;

    // Tiles go straight from global memory into LDS (global_load_lds_dwordx4: each wave-wide load
    // fills one contiguous 1 KB segment, lane i its 16 bytes at 16 i).  Every lane therefore loads
    // the global chunk that belongs at its LDS position; the chunk order inside a row is XOR
    // swizzled (and d_h = 48 key rows are padded to an odd pitch) so that fragment reads of
    // sixteen consecutive rows hit distinct banks.
    // Three stages: while tile kt computes, tile kt+1 has landed or is landing and tile kt+2 is in
    // flight.  Every wave issues the same number of loads per tile (segments past the end are
    // re-issued, same bytes), so the wait is a compile-time vmcnt.
    auto issue = [&](int kt, int stage) {
        const int64_t key0 = (int64_t)kt * kBN;
#pragma unroll
        for (int i = 0; i < LK; ++i) {
            const int seg = min(w + 4 * i, SEGK - 1);
            const int q = seg * 64 + lane;          // chunk position in the tile
            const int r = q / KP, cpos = q % KP;    // key row, swizzled chunk slot
            const int c = cpos < KC8 ? cpos ^ kswz<DH>(r) : 0;  // pad slot: any chunk of the row
            dma16(Kg + (key0 + r) * DH + 8 * c, &ks_lds[stage][seg * 512]);
        }
#pragma unroll
        for (int i = 0; i < LV; ++i) {
            const int seg = min(w + 4 * i, SEGV - 1);
            const int q = seg * 64 + lane;
            const int r = q / 8, cpos = q % 8;      // V^T row (head dim), swizzled chunk slot
            const int c = cpos ^ vswz(r);
            dma16(Vg + (int64_t)r * a.S_pad + key0 + 8 * c, &vs_lds[stage][seg * 512]);
        }
    };
    // per-tile maximum key norm: a wave-uniform scalar load (not on the vector-memory counter)
    typedef const __attribute__((address_space(4))) float* const_f32_ptr;
    const_f32_ptr kntg = (const_f32_ptr)(a.knt + ((int64_t)it.b * a.G + it.g) * (a.S_pad / kBN));
    constexpr int NLOAD = LK + LV;  // vector-memory operations issued per tile per wave

    // [V | 1 | 0]^T fragment rows of this lane: row n = 32 cb + (lane & 31)
    const int hsel = lane >> 5;
    auto body = [&](auto fast_t, bool diag, int kt) {
        constexpr bool FAST = decltype(fast_t)::value;
        const int stage = kt % NSTAGE;
        const uint16_t* kb = ks_lds[stage];
        const uint16_t* vb = vs_lds[stage];
        // K fragments of both 32-key subtiles (shared by the two query tiles)
        bf16x8_t kf[2][KS];
#pragma unroll
        for (int kst = 0; kst < 2; ++kst)
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const int r = 32 * kst + (lane & 31), c = 2 * kk + hsel;
                kf[kst][kk] = *reinterpret_cast<const bf16x8_t*>(kb + (r * KP + (c ^ kswz<DH>(r))) * 8);
            }
        bf16x8_t pa[2][4];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            f32x16_t sacc[2];
#pragma unroll
            for (int kst = 0; kst < 2; ++kst) {
                f32x16_t acc = {};
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kst][kk], qf[qt][kk], acc, 0, 0, 0);
                sacc[kst] = acc;
            }
            softmax_tile<NCB, FAST>(sacc, mrun[qt], oacc[qt], pa[qt], diag, kt * kBN, posq[qt], lane);
        }
        // O += P [V | 1 | 0]: per 16-key chunk, one fragment of each column block serves both
        // query tiles
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
            const int c = 2 * ch + hsel;  // 16-byte chunk of the slotted key order
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const int n = 32 * cb + (lane & 31);
                const uint16_t* src = n < DH ? vb + (n * 8 + (c ^ vswz(n))) * 8
                                             : one_lds + ((n - DH) * 8 + (c ^ vswz(n))) * 8;
                const bf16x8_t vf = *reinterpret_cast<const bf16x8_t*>(src);
#pragma unroll
                for (int qt = 0; qt < 2; ++qt)
                    oacc[qt][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[qt][ch], vf, oacc[qt][cb], 0, 0, 0);
            }
        }
    };

    issue(0, 0);
    if (kt_end > 1) {
        issue(1, 1);
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(NLOAD));
    } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    }
    __syncthreads();

    for (int kt = 0; kt < kt_end; ++kt) {
        const bool ahead = kt + 2 < kt_end;
        if (ahead) issue(kt + 2, (kt + 2) % NSTAGE);
        const float kmax_cur = kntg[kt];
        if (kt < wtiles) {
            const bool fast = offset_zero && (qmax_w * kmax_cur * 1.02f <= kFastBound);
            const bool diag = kt * kBN + kBN - 1 > wfirst;
            if (fast) {
                body(std::true_type{}, diag, kt);
            } else {
                body(std::false_type{}, diag, kt);
                offset_zero = !__builtin_amdgcn_ballot_w64(mrun[0] != 0.f && mrun[0] != -INFINITY) &&
                              !__builtin_amdgcn_ballot_w64(mrun[1] != 0.f && mrun[1] != -INFINITY);
            }
        }
        if (kt + 1 < kt_end) {
            // tile kt+1 must have landed: only this step's loads (tile kt+2) may still be in flight
            if (ahead) __builtin_amdgcn_s_waitcnt(vmcnt_wait(NLOAD));
            else __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
        }
        __syncthreads();
    }

    // ---------------------------------------------------------------- normalise and store
    // accumulator register j of this lane: query row 8 (j / 4) + 4 (lane / 32) + j % 4 of the
    // tile, column 32 cb + (lane & 31); the row sum is column DH, held by lane DH % 32 (+32)
    constexpr int CBS = DH / 32, CS = DH % 32;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int row = 8 * (j >> 2) + 4 * hsel + (j & 3);
            const float lsum = __shfl(oacc[qt][CBS][j], CS + 32 * hsel);
            const float sc = 1.0f / lsum;
            const int c = w * kQW + qt * 32 + row;
            const int p = c / NH, h = c % NH;
            const int pos = it.p0 + p;
            if (p >= it.np || pos >= S) continue;
            const int v = h < a.k ? it.g * a.k + h : a.G * a.k;
            bf16_t* orow = a.O + (((int64_t)it.b * S + pos) * a.H + v) * DH;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const int n = 32 * cb + (lane & 31);
                if (n < DH) orow[n] = from_f32<bf16_t>(oacc[qt][cb][j] * sc);
            }
        }
    }
}

}  // namespace

hipError_t launch_attn_mfma(const GqeDims& D, const WorkPlan& P, char* ws, hipStream_t st, KernelMarks* km, bool prep) {
    AttnArgs a{};
    a.Q = (const bf16_t*)(ws + P.q);
    a.K = (const bf16_t*)(ws + P.kk);
    a.Vt = (const bf16_t*)(ws + P.vt);
    a.kn = (const float*)(ws + P.kn);
    a.O = (bf16_t*)(ws + P.o);
    a.S = P.S;
    a.S_pad = P.S_pad;
    a.B = (int)P.B;
    a.G = D.G;
    a.H = D.H;
    a.k = D.k;
    a.skv = D.skv;
    a.s = D.s;
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
    const int64_t grid = total;
    if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidValue;
    a.knt = (const float*)(ws + P.knt);
    if (prep) {
        const int64_t BG = P.B * D.G;
        const int64_t work = BG * (P.S_pad / 64) + BG * D.dh * (P.S_pad - P.S);
        const unsigned pg = (unsigned)std::min<int64_t>(ceil_div(work, 256), 1024);
        if (km) km->begin(KT_ATTN_PREP);
        attn_prep_kernel<<<pg, 256, 0, st>>>(a.kn, (float*)(ws + P.knt), (bf16_t*)(ws + P.vt), BG, P.S, P.S_pad,
                                             D.dh);
        if (km) km->mark(KT_ATTN_PREP);
    }
    {
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (km) km->begin(KT_ATTN);
    switch (D.dh) {
        case 32: attn_fwd_kernel<32><<<(unsigned)grid, 256, 0, st>>>(a); break;
        case 48: attn_fwd_kernel<48><<<(unsigned)grid, 256, 0, st>>>(a); break;
        case 64: attn_fwd_kernel<64><<<(unsigned)grid, 256, 0, st>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    if (km) km->mark(KT_ATTN);
    return hipGetLastError();
}
