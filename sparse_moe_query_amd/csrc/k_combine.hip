// Output construction + output projection of the GQE layer on gfx950 matrix cores.
//
// GQE README "Parameters"/"Ablations" and the explainer's "Output Construction": the output is
// built from the selected experts' head outputs (hard concatenation: each selected expert uses
// its own d_h x d slice of the output projection), a renormalised weighted-sum slot per group
// (variant gqe), and the always-on shared head.  With the slot operand
//     A[t, (g, j)]   = c * O[t, (g, r)]   if expert g*n+j is the token's r-th choice, else 0
//                      (c = 1 for gqe / hard_concat, c = p of that expert for weighted_concat)
//     A[t, rslot g]  = sum_r w_r O[t, (g, r)]            (gqe only)
//     A[t, shared]   = O[t, shared]
// the layer output is y = A @ W_stack, W_stack = [W_o[g*n..g*n+n-1]; W_oR[g] for g; W_os].
// A is never materialised: its fragments are formed in registers from the head outputs.
//
// Work item: 128 tokens x 128 output columns; eight waves in 2 x 4, each 64 tokens x 32 columns =
// 2 blocks of v_mfma_f32_32x32x16_bf16 computing y^T = W_stack^T A^T (every lane stores four
// consecutive output columns); two work groups per CU, four waves per SIMD.  The reduction runs slot by slot (one stage = d_h rows of W_stack):
//   W_stack   pre-packed per (column tile, slot) as the exact LDS image ([128 cols][odd pitch]
//             16-byte chunks, zero pad chunk) and copied by global_load_lds_dwordx4 into a ring
//             of three stages, two slots ahead of the one being multiplied
//   O         the rows of one unit (a group's k heads, or the shared head) for the 128 tokens are
//             copied the same way into one of two buffers when the previous unit starts
//   routing   the tile's choices (and coefficients where needed) are staged in LDS once; each
//             lane keeps those of its two tokens for the current group in registers
//   fragments a token fragment (8 consecutive head dims of one token) is the LDS chunk of the
//             chosen head (copy), that chunk or zero (select), or a coefficient-weighted sum of
//             the group's heads rounded once to bf16 (scale); with one choice per group the
//             renormalised weight is exactly 1 (p / p): the gqe slot's weights are then folded
//             into the group's expert slots when the weights are packed (one slot per expert)
// No compiler-visible global load sits in the loop, so every wait is an explicit vmcnt.
#include "gqe_common.h"
#include "gqe_internal.h"

namespace {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kWaves = 8;           // 2 x 4: waves along the tokens x along the output columns
constexpr int kWN = 4;
constexpr int kCB = kBN / kWN / 32;  // 32-column blocks per wave
constexpr int kThreads = 64 * kWaves;
constexpr int kGKMax = 16;  // routing entries per token staged in LDS (groups x choices)

__host__ __device__ constexpr int odd_pitch(int chunks) { return (chunks & 1) ? chunks : chunks + 1; }

struct CombArgs {
    const bf16_t* O;       // [T][H][DH]
    const bf16_t* wo;      // [d / 128][NS][128][PW * 8]
    const int32_t* idx;    // [T][G][k]
    const float* wsel;     // [T][G][k]
    const float* psel;     // [T][G][k]
    bf16_t* y;             // [T][d]
    int64_t T;
    int d, G, k, n, H, variant, dense, s;
    int NS;        // stages (slots)
    int PG;        // stages per unit (n + rslot; 1 when every head is its own unit)
    int NUM;       // units before the shared head's
    int KHU;       // heads per unit
};

template <int DH, int KH, bool COEF>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) combine_kernel(CombArgs a) {
    constexpr int C8 = DH / 8;                // 16-byte chunks per head row
    constexpr int PW = odd_pitch(C8);         // W_stack stage pitch (chunks per output column)
    constexpr int PO = odd_pitch(KH * C8);    // O stage pitch (chunks per token)
    constexpr int SEGW = kBN * PW * 16 / 1024, LW = (SEGW + kWaves - 1) / kWaves;
    constexpr int SEGO = kBM * PO * 16 / 1024, LO = (SEGO + kWaves - 1) / kWaves;
    constexpr int KS = DH / 16;
    constexpr int WST = kBN * PW * 8, OST = kBM * PO * 8;  // stage sizes (bf16)
    // W ring (three stages) and O double buffer in one array: the epilogue reuses all of it
    __shared__ __align__(1024) uint16_t lbuf[3 * WST + 2 * OST];
    uint16_t* const wl = lbuf;
    uint16_t* const ol = lbuf + 3 * WST;
    __shared__ __align__(16) uint8_t rj[kBM * kGKMax];  // expert index inside the group, per choice
    __shared__ float rc[COEF ? kBM * kGKMax : 1]; // p (weighted_concat) or w (gqe) per choice
    __shared__ __align__(16) uint16_t zr[C8 * 8];   // a zero token row: unchosen tokens read it
    static_assert(COEF || KH == 1, "the select-only form handles one head per unit");

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w / kWN, wn = w % kWN;
    const int ncol = a.d / kBN;
    const int ntile = (int)ceil_div(a.T, kBM);
    // XCD-aware: the column tiles of one token tile run on one XCD (they share the O rows)
    int tile, ct;
    const int L = blockIdx.x;
    if (ntile % 8 == 0) {
        const int xcd = L % 8, i = L / 8;
        tile = (i / ncol) * 8 + xcd;
        ct = i % ncol;
    } else {
        tile = L / ncol;
        ct = L % ncol;
    }
    tile = __builtin_amdgcn_readfirstlane(tile);
    ct = __builtin_amdgcn_readfirstlane(ct);
    const int64_t t0 = (int64_t)tile * kBM;
    const int NU = a.NUM + a.s;  // units, the shared head's last

    // ---- loaders
    const bf16_t* wtile = a.wo + (int64_t)ct * a.NS * kBN * PW * 8;
    auto issue_w = [&](int st) {
        const bf16_t* src = wtile + (int64_t)st * kBN * PW * 8;
#pragma unroll
        for (int i = 0; i < LW; ++i) {
            const int seg = min(w + kWaves * i, SEGW - 1);
            dma16(src, (uint32_t)(seg * 1024 + 16 * lane), wl + (st % 3) * WST + seg * 512);
        }
    };
    // O rows: chunk slot q of the stage = (token row q / PO, chunk q % PO); rows past the last
    // token repeat it, pad chunks repeat chunk 0
    uint32_t orow[LO];
    int ochk[LO];
#pragma unroll
    for (int i = 0; i < LO; ++i) {
        const int q = min(w + kWaves * i, SEGO - 1) * 64 + lane;
        const int64_t rmax = a.T - 1 - t0;
        const int r = q / PO;
        orow[i] = (uint32_t)((r < rmax ? r : rmax) * a.H * DH * 2);
        ochk[i] = q % PO;
    }
    auto issue_o = [&](int unit) {
        const int nh = unit < a.NUM ? a.KHU : 1;
        const bf16_t* base = a.O + (t0 * a.H + (int64_t)unit * a.KHU) * DH;
#pragma unroll
        for (int i = 0; i < LO; ++i) {
            const int c = ochk[i] < nh * C8 ? ochk[i] : 0;
            dma16(base, orow[i] + 16 * c, ol + (unit & 1) * OST + min(w + kWaves * i, SEGO - 1) * 512);
        }
    };

    issue_o(0);
    issue_w(0);
    if (a.NS > 1) issue_w(1);
    if (tid < C8) *reinterpret_cast<u32x4_t*>(&zr[8 * tid]) = u32x4_t{0u, 0u, 0u, 0u};

    // ---- routing of the tile's tokens (routed mode): expert index inside the group per choice
    if (!a.dense) {
        const int GK = a.G * a.k;
        for (int q = tid; q < kBM * GK; q += kThreads) {
            const int row = q / GK, e = q % GK;
            const int64_t t = t0 + row;
            uint8_t j = 0xff;
            float c = 0.f;
            if (t < a.T) {
                const int g = e / a.k;
                j = (uint8_t)(a.idx[t * GK + e] - g * a.n);
                if (COEF) c = a.variant == GQE_VARIANT_WEIGHTED_CONCAT ? a.psel[t * GK + e] : a.wsel[t * GK + e];
            }
            rj[row * kGKMax + e] = j;
            if (COEF) rc[row * kGKMax + e] = c;
        }
    }
    if (a.NS > 1) __builtin_amdgcn_s_waitcnt(vmcnt_wait(LW));
    else __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    __syncthreads();

    f32x16_t acc[2][kCB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < kCB; ++j) acc[i][j] = f32x16_t{};

    const int trow0 = 64 * wm + (lane & 31);          // token rows trow0, trow0 + 32
    const int wcol0 = 32 * kCB * wn + (lane & 31);    // output columns wcol0 (+ 32)
    const int hsel = lane >> 5;                       // which 8 of the 16 reduction rows
    // the choices of the lane's two tokens for every group (one byte each), kept in registers
    u32x4_t jw[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
        jw[i] = a.dense ? u32x4_t{0u, 0u, 0u, 0u} : *reinterpret_cast<const u32x4_t*>(&rj[(trow0 + 32 * i) * kGKMax]);
    int jr[2][KH];
    float cr[2][KH];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < KH; ++r) {
            jr[i][r] = -1;
            cr[i][r] = 0.f;
        }

    int unit = 0, u = 0;  // position of the stage: unit, slot inside the unit (wave-uniform)
    for (int st = 0; st < a.NS; ++st) {
        const bool routed = unit < a.NUM && !a.dense;
        if (!COEF && routed && u == 0) {
#pragma unroll
            for (int i = 0; i < 2; ++i) jr[i][0] = rj[(trow0 + 32 * i) * kGKMax + unit];
        }
        if (COEF && routed && u == 0) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < KH; ++r) {
                    const int byte = unit * KH + r, q = byte >> 2;
                    const uint32_t dw = q == 0 ? jw[i][0] : q == 1 ? jw[i][1] : q == 2 ? jw[i][2] : jw[i][3];
                    jr[i][r] = (int)((dw >> (8 * (byte & 3))) & 0xffu);
                    if (COEF) cr[i][r] = rc[(trow0 + 32 * i) * kGKMax + byte];
                }
        }
        // kind: 0 copy (dense head, shared head, gqe slot with one choice), 1 select (expert slot,
        // coefficient 1), 2 scale (weighted expert slot, gqe slot with several choices)
        int kind = 0;
        if (routed) {
            if (u < a.n) kind = a.variant == GQE_VARIANT_WEIGHTED_CONCAT ? 2 : 1;
            else kind = KH == 1 ? 0 : 2;
        }
        // token rows of this slot's fragments: the select-only form points an unchosen token at
        // the zero row, so its fragments need no per-element select
        const uint16_t* const ob = ol + (unit & 1) * OST;
        const uint16_t* tb[2];
        const bool sel = routed && u < a.n;
#pragma unroll
        for (int i = 0; i < 2; ++i)
            tb[i] = (!COEF && sel && jr[i][0] != u) ? zr : ob + (trow0 + 32 * i) * PO * 8;
        int off[2];
        bool valid[2];
        float coef[2][KH];
#pragma unroll
        for (int i = 0; COEF && i < 2; ++i) {
            off[i] = 0;
            valid[i] = true;
            if (kind == 1) {
                valid[i] = false;
#pragma unroll
                for (int r = 0; r < KH; ++r)
                    if (jr[i][r] == u) {
                        valid[i] = true;
                        off[i] = r * C8;
                    }
            }
#pragma unroll
            for (int r = 0; r < KH; ++r)
                coef[i][r] = (u < a.n) ? (jr[i][r] == u ? cr[i][r] : 0.f) : cr[i][r];
        }

        // loads of this step, spread over its k-steps so that the transfers overlap the matrix
        // work: the next unit's rows when this unit starts, then the slot two ahead
        const bool o_next = u == 0 && unit + 1 < NU;
        const bool ahead = st + 2 < a.NS;
        const uint16_t* wb = wl + (st % 3) * WST;
        auto frag = [&](int kk, bf16x8_t (&wf)[kCB], bf16x8_t (&tf)[2]) {
#pragma unroll
            for (int cb = 0; cb < kCB; ++cb)
                wf[cb] = *reinterpret_cast<const bf16x8_t*>(wb + ((wcol0 + 32 * cb) * PW + 2 * kk + hsel) * 8);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if (!COEF) {
                    tf[i] = *reinterpret_cast<const bf16x8_t*>(tb[i] + (2 * kk + hsel) * 8);
                } else if (kind != 2) {
                    u32x4_t v = *reinterpret_cast<const u32x4_t*>(tb[i] + (2 * kk + hsel + off[i]) * 8);
                    if (!valid[i]) v = u32x4_t{0u, 0u, 0u, 0u};
                    tf[i] = __builtin_bit_cast(bf16x8_t, v);
                } else {
                    float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int r = 0; r < KH; ++r) {
                        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(tb[i] + (2 * kk + hsel + r * C8) * 8);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            f[2 * e] += coef[i][r] * __uint_as_float(v[e] << 16);
                            f[2 * e + 1] += coef[i][r] * __uint_as_float(v[e] & 0xffff0000u);
                        }
                    }
                    const u32x4_t pk = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                                        pack_bf16x2(f[6], f[7])};
                    tf[i] = __builtin_bit_cast(bf16x8_t, pk);
                }
            }
        };
        bf16x8_t wf[2][kCB], tf[2][2];
        frag(0, wf[0], tf[0]);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            if (kk + 1 < KS) frag(kk + 1, wf[(kk + 1) & 1], tf[(kk + 1) & 1]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int cb = 0; cb < kCB; ++cb)
                    acc[i][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[kk & 1][cb], tf[kk & 1][i], acc[i][cb], 0, 0, 0);
            if (kk == 0 && o_next) issue_o(unit + 1);
            if (kk == 1 && ahead) issue_w(st + 2);
        }
        if (st + 1 < a.NS) {
            // the next slot must have landed, and the next unit's rows if the next slot starts
            // it; loads of this step that the next slot does not read may stay in flight
            const bool o_pending = o_next && unit < a.NUM && u + 1 < a.PG;
            if (ahead) {
                if (o_pending) __builtin_amdgcn_s_waitcnt(vmcnt_wait(LW + LO));
                else __builtin_amdgcn_s_waitcnt(vmcnt_wait(LW));
            } else {
                if (o_pending) __builtin_amdgcn_s_waitcnt(vmcnt_wait(LO));
                else __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
            }
        }
        __syncthreads();
        if (unit < a.NUM && u + 1 < a.PG) {
            ++u;
        } else {
            ++unit;
            u = 0;
        }
    }

    // ---- epilogue: acc[i][cb] is y^T for token trow0 + 32 i, columns 32 (kCB wn + cb) + rows.
    // The tile goes through LDS (the stage buffers are free: the last slot's barrier is behind
    // every wave's reads of them, and no copy is in flight) so that y is written as whole 256-byte token rows:
    // stored straight from the accumulators, every store instruction would write 16-byte pieces of
    // 32 different rows.
    constexpr int YP = kBN + 8;  // row pitch in bf16 (272 bytes: consecutive rows 4 banks apart)
    static_assert(kBM * YP <= 3 * WST + 2 * OST, "the output tile fits in the stage buffers");
    uint16_t* ys = lbuf;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = 32 * kCB * wn + 32 * cb + 8 * q + 4 * hsel;
                *reinterpret_cast<u32x2_t*>(&ys[(trow0 + 32 * i) * YP + col]) =
                    u32x2_t{pack_bf16x2(acc[i][cb][4 * q], acc[i][cb][4 * q + 1]),
                            pack_bf16x2(acc[i][cb][4 * q + 2], acc[i][cb][4 * q + 3])};
            }
    __syncthreads();
    constexpr int CH = kBN / 8;  // 16-byte chunks per token row of the tile
#pragma unroll
    for (int it = 0; it < kBM * CH / kThreads; ++it) {
        const int q = tid + kThreads * it, row = q / CH, ch = q % CH;
        const int64_t t = t0 + row;
        if (t < a.T)
            *reinterpret_cast<u32x4_t*>(a.y + t * a.d + ct * kBN + 8 * ch) =
                *reinterpret_cast<const u32x4_t*>(&ys[row * YP + 8 * ch]);
    }
}

template <int DH>
hipError_t launch_dh(const CombArgs& a, bool coef, unsigned grid, hipStream_t st) {
    if (a.KHU == 1) {
        if (coef) combine_kernel<DH, 1, true><<<grid, kThreads, 0, st>>>(a);
        else combine_kernel<DH, 1, false><<<grid, kThreads, 0, st>>>(a);
    } else {
        combine_kernel<DH, 2, true><<<grid, kThreads, 0, st>>>(a);
    }
    return hipGetLastError();
}

}  // namespace

int combine_stage_pitch(int dh) { return odd_pitch(dh / 8); }

bool combine_mfma_supported(const GqeDims& D) {
    if (D.d % kBN != 0) return false;
    if (!D.dense && (D.k > 2 || D.G * D.k > kGKMax)) return false;
    return true;
}

hipError_t launch_combine_mfma(const GqeDims& D, const WorkPlan& P, const void* packed,
                               const PackedLayout& pl, void* y, char* ws, hipStream_t st, KernelMarks* km) {
    CombArgs a{};
    a.O = (const bf16_t*)(ws + P.o);
    a.wo = (const bf16_t*)((const char*)packed + pl.wo);
    a.idx = (const int32_t*)(ws + P.idx);
    a.wsel = (const float*)(ws + P.wsel);
    a.psel = (const float*)(ws + P.psel);
    a.y = (bf16_t*)y;
    a.T = P.T;
    a.d = D.d;
    a.G = D.G;
    a.k = D.k;
    a.n = D.n;
    a.H = D.H;
    a.variant = D.variant;
    a.dense = D.dense;
    a.s = D.s;
    a.NS = pl.slots;
    if (D.dense) {
        // every head is its own unit (head e = expert e), one slot each
        a.PG = 1;
        a.NUM = D.N;
        a.KHU = 1;
    } else {
        a.PG = D.n + (D.variant == GQE_VARIANT_GQE && !pl.rslot_fused ? 1 : 0);
        a.NUM = D.G;
        a.KHU = D.k;
    }
    if (!combine_mfma_supported(D)) return hipErrorInvalidValue;
    // coefficients are needed by weighted_concat and by gqe with several choices per group
    const bool coef = !D.dense && (D.variant == GQE_VARIANT_WEIGHTED_CONCAT || (D.variant == GQE_VARIANT_GQE && D.k > 1));
    const unsigned grid = (unsigned)(ceil_div(P.T, kBM) * (a.d / kBN));
    hipError_t e;
    if (km) km->begin(KT_COMBINE);
    switch (D.dh) {
        case 32: e = launch_dh<32>(a, coef, grid, st); break;
        case 48: e = launch_dh<48>(a, coef, grid, st); break;
        case 64: e = launch_dh<64>(a, coef, grid, st); break;
        default: return hipErrorInvalidValue;
    }
    if (km) km->mark(KT_COMBINE);
    return e;
}
