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
// The weighted combine is fused into the GEMM: A is built tile by tile in LDS straight from
// O_act and the routing decisions, never written to HBM.
//
// Tile: 128 tokens x 128 output columns, K in 32-wide stages (two 16-wide pieces, each inside one
// slot); four waves in 2 x 2, each 64 x 64 = 2 x 2 blocks of v_mfma_f32_32x32x16_bf16 computing
// y^T = W_stack^T A^T so every lane stores four consecutive output columns.
#include "gqe_common.h"
#include "gqe_internal.h"

namespace {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kKC = 32;
constexpr int kAP = kKC + 8;  // LDS pitches (elements)
constexpr int kBP = kKC + 8;

struct CombArgs {
    const bf16_t* O;       // [T][H][DH]
    const bf16_t* wo;      // [d][Ktot]
    const int32_t* idx;    // [T][G][k]
    const float* wsel;     // [T][G][k]
    const float* psel;     // [T][G][k]
    bf16_t* y;             // [T][d]
    int64_t T;
    int d, G, k, n, H, s, dense, variant, slots, per_group, ktot;
};

template <int DH>
__global__ void __launch_bounds__(256, 2) combine_kernel(CombArgs a) {
    constexpr int PPS = DH / 16;  // 16-wide pieces per slot
    __shared__ __align__(16) uint16_t as[2][kBM * kAP];
    __shared__ __align__(16) uint16_t bs[2][kBN * kBP];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w >> 1, wn = w & 1;
    const int ncol = a.d / kBN;
    const int ntile = (int)ceil_div(a.T, kBM);
    // XCD-aware: the column tiles of one token tile run on one XCD (they share O_act rows)
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
    const int64_t t0 = (int64_t)tile * kBM;
    const int c0 = ct * kBN;

    // ---- A stage: 128 tokens x 2 pieces x 16 = 512 half-pieces of 8 elements, 2 per thread
    u32x4_t ar[2];
    auto build_a = [&](int kc) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int task = tid + 256 * u;      // token = task >> 2, piece = (task >> 1) & 1, half = task & 1
            const int row = task >> 2;
            const int piece = kc * 2 + ((task >> 1) & 1);
            const int half = task & 1;
            const int slot = piece / PPS;
            const int off = (piece % PPS) * 16 + 8 * half;
            const int64_t t = t0 + row;
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = 0.f;
            if (t < a.T) {
                const bf16_t* ot = a.O + t * a.H * DH;
                auto addrow = [&](int head, float c) {
                    const u32x4_t q = *reinterpret_cast<const u32x4_t*>(ot + head * DH + off);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        v[2 * i] += c * __uint_as_float(q[i] << 16);
                        v[2 * i + 1] += c * __uint_as_float(q[i] & 0xffff0000u);
                    }
                };
                if (slot < a.G * a.per_group) {
                    const int g = slot / a.per_group, u2 = slot % a.per_group;
                    const int64_t rb = (t * a.G + g) * a.k;
                    if (u2 < a.n) {
                        const int e = g * a.n + u2;
                        if (a.dense) {
                            addrow(g * a.k + u2, 1.f);
                        } else {
                            for (int r = 0; r < a.k; ++r)
                                if (a.idx[rb + r] == e)
                                    addrow(g * a.k + r, a.variant == GQE_VARIANT_WEIGHTED_CONCAT ? a.psel[rb + r] : 1.f);
                        }
                    } else {
                        for (int r = 0; r < a.k; ++r) addrow(g * a.k + r, a.wsel[rb + r]);
                    }
                } else if (slot < a.slots) {
                    addrow(a.G * a.k, 1.f);  // shared head
                }                            // else: zero padding past the last slot
            }
            ar[u] = u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                            pack_bf16x2(v[6], v[7])};
        }
    };
    // ---- B stage: 128 output columns x 32 k = 512 chunks, 2 per thread
    u32x4_t br[2];
    auto load_b = [&](int kc) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int ch = tid + 256 * u;
            const int col = ch >> 2, c = ch & 3;
            br[u] = *reinterpret_cast<const u32x4_t*>(a.wo + (int64_t)(c0 + col) * a.ktot + kc * kKC + 8 * c);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int task = tid + 256 * u;
            const int row = task >> 2, q = task & 3;  // q = 8-element column group (piece*2 + half)
            *reinterpret_cast<u32x4_t*>(&as[buf][row * kAP + 8 * q]) = ar[u];
            const int col = task >> 2;
            *reinterpret_cast<u32x4_t*>(&bs[buf][col * kBP + 8 * q]) = br[u];
        }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x16_t{};

    const int nk = a.ktot / kKC;
    build_a(0);
    load_b(0);
    lstore(0);
    __syncthreads();
    for (int kc = 0; kc < nk; ++kc) {
        const int buf = kc & 1;
        if (kc + 1 < nk) {
            build_a(kc + 1);
            load_b(kc + 1);
        }
        const uint16_t* ab = as[buf];
        const uint16_t* bb = bs[buf];
#pragma unroll
        for (int ks = 0; ks < kKC / 16; ++ks) {
            bf16x8_t af[2], bf[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                af[i] = *reinterpret_cast<const bf16x8_t*>(ab + (64 * wm + 32 * i + (lane & 31)) * kAP + 16 * ks + 8 * (lane >> 5));
                bf[i] = *reinterpret_cast<const bf16x8_t*>(bb + (64 * wn + 32 * i + (lane & 31)) * kBP + 16 * ks + 8 * (lane >> 5));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
        }
        if (kc + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: acc[i][j] is y^T for tokens 64wm + 32i + (lane & 31), columns 64wn + 32j + rows
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t t = t0 + 64 * wm + 32 * i + (lane & 31);
        if (t >= a.T) continue;
        bf16_t* yr = a.y + t * a.d + c0 + 64 * wn;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = 32 * j + 8 * q + 4 * (lane >> 5);
                u32x2_t pk = {pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                              pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
                *reinterpret_cast<u32x2_t*>(yr + col) = pk;
            }
    }
}

}  // namespace

hipError_t launch_combine_mfma(const GqeDims& D, const WorkPlan& P, const void* packed,
                               const PackedLayout& pl, void* y, char* ws, hipStream_t st) {
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
    a.s = D.s;
    a.dense = D.dense;
    a.variant = D.variant;
    a.slots = pl.slots;
    a.per_group = D.n + ((!D.dense && D.variant == GQE_VARIANT_GQE) ? 1 : 0);
    a.ktot = pl.ktot_pad;
    if (a.d % kBN != 0 || a.ktot % kKC != 0) return hipErrorInvalidValue;
    const unsigned grid = (unsigned)(ceil_div(P.T, kBM) * (a.d / kBN));
    switch (D.dh) {
        case 32: combine_kernel<32><<<grid, 256, 0, st>>>(a); break;
        case 48: combine_kernel<48><<<grid, 256, 0, st>>>(a); break;
        case 64: combine_kernel<64><<<grid, 256, 0, st>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
