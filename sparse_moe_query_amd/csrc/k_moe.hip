// Top-k mixture-of-experts MLP on gfx950 (cseroadmap tutorial "Grouped-query attention and mixture
// of experts", section "Mixture of experts (MoE)": a router picks top_k of E expert MLPs per token
// and mixes their outputs with the renormalised router weights).
//
//   router      the attention layer's router with one group of E experts (float64 logits, softmax,
//               top-k with the lower index on ties, renormalised weights, per-expert statistics)
//   bucketing   the global stable token-to-expert bucketing (histogram, scan, scatter, inverse)
//   up          H[p] = act(x[perm[p]] W1[e])  for every bucket position p of expert e
//   down        Y[p] = H[p] W2[e]
//   combine     y[t] = sum_r w[t, r] Y[inv[t, r]]
//
// The two expert products are one grouped matrix-core GEMM kernel (moe_gemm_kernel): a work group
// takes 128 (up) or 256 (down) consecutive bucket positions of one expert (so every row of the tile uses the same
// weights; the tile table is walked on the device from the bucket offsets) and 256 output
// features.  It computes C^T = W^T X^T with v_mfma_f32_32x32x16_bf16, the weights (pre-transposed
// by the packing, k contiguous) as the A operand and the token rows as the B operand, so every lane
// ends with four consecutive output features of one token: 8-byte bf16 stores of H, 16-byte float32
// stores of Y.  Operands pass through LDS in k-slices of 32 (64-byte rows; the 16 rows that one
// 16-byte fragment read serves per cycle fall in distinct banks by an XOR swizzle of the chunks),
// loaded straight from global memory into a ring of three LDS stages (global_load_lds_dwordx4, no
// registers), two slices ahead of the one that multiplies; one barrier per slice.  Each of the
// four (up) or eight (down) waves owns 128 features x 64 tokens (4 x 2 accumulator tiles of 32 x 32).
#include "gqe_common.h"
#include "gqe_internal.h"

namespace {

constexpr int kBF = 256;    // output features per tile
constexpr int kBK = 32;     // k per LDS slice (64-byte rows of four 16-byte chunks)
constexpr int kStages = 3;  // LDS ring: slices s + 1 and s + 2 load while slice s multiplies
// bucket positions per tile and waves (2 feature halves x BT / 64 position quarters): 256 and 8
// for the down product, 128 and 4 for the up product (measured: 256 positions made down 8 % faster
// and up 7 % slower)
template <int MODE> constexpr int moe_bt() { return MODE == 1 ? 256 : 128; }
template <int MODE> constexpr int moe_waves() { return moe_bt<MODE>() / 32; }

// 16-byte chunk swizzle of 64-byte LDS rows: 16 consecutive rows reading the same chunk hit 16
// distinct 4-bank groups (row r starts at bank 16 (r % 4); the chunk moves with r / 4).
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

struct MoeGemmArgs {
    const uint16_t* w;      // [E][NF][K] expert weights, k contiguous
    const uint16_t* src;    // up: x [T][K]; down: H [P][K]
    const int32_t* offs;    // [E + 1] bucket offsets
    const int32_t* perm;    // [P] token of every bucket position (up)
    void* out;              // up: H [P][NF] bf16; down: Y [P][NF] float32
    int E, NF, K;
    int ntiles;             // upper bound of the position tiles over all experts
};

__device__ __forceinline__ float gelu(float v) { return 0.5f * v * (1.f + erff(v * 0.70710678118654752f)); }

template <int MODE, int ACT>  // MODE 0: up (gathered x rows, activation, bf16 out); 1: down (float32 out)
__global__ void __launch_bounds__(64 * moe_waves<MODE>(), MODE == 1 ? 1 : 2) moe_gemm_kernel(MoeGemmArgs a) {
    constexpr int kBT = moe_bt<MODE>(), NW = moe_waves<MODE>();
    constexpr int WJ = kBF / (16 * NW), XJ = kBT / (16 * NW);  // load instructions per wave and slice
    constexpr int kLoadsPerSlice = WJ + XJ;
    __shared__ __align__(1024) uint16_t Ws[kStages][kBF * kBK];
    __shared__ __align__(1024) uint16_t Xs[kStages][kBT * kBK];
    // XCD-aware order: work groups are dealt round-robin to the 8 XCDs, so group b runs on XCD
    // b % 8; logical tile L = (b % 8) * per + b / 8 gives each XCD a contiguous run of tiles, with
    // the feature tiles of one position tile adjacent: the XCD's L2 holds that tile's token
    // rows for all its feature tiles and the weights of about one expert at a time.
    const int nft = (a.NF + kBF - 1) / kBF;
    const int per = (int)((gridDim.x + 7) / 8);
    const int L = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (L >= a.ntiles * nft) return;
    const int ft = L % nft;
    // this work group's (expert, kBT positions): walk the experts' tile counts
    int rem = L / nft, e = 0, M = 0, p0 = 0;
    for (; e < a.E; ++e) {
        const int b0 = a.offs[e], b1 = a.offs[e + 1];
        const int nt = (b1 - b0 + kBT - 1) / kBT;
        if (rem < nt) {
            p0 = b0 + rem * kBT;
            M = min(kBT, b1 - p0);
            break;
        }
        rem -= nt;
    }
    if (e == a.E) return;  // beyond the last tile (the grid is an upper bound)
    const int f0 = ft * kBF;
    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, in a scalar register
    const int wf = (w / (NW / 2)) * 128, wt = (w % (NW / 2)) * 64;
    // Direct global -> LDS loads: one wave instruction fills 16 rows of a stage (1 KB); lane q takes
    // row q / 4 of them and the 16-byte slot q % 4, which holds chunk slot ^ swz(row).  Rows past
    // the tile's end load a valid row (their results are never stored).
    const uint16_t* wsrc[WJ];
    const uint16_t* xsrc[XJ];
#pragma unroll
    for (int j = 0; j < WJ; ++j) {
        const int row = (w * WJ + j) * 16 + (lane >> 2);
        const int f = f0 + row < a.NF ? f0 + row : f0;
        wsrc[j] = a.w + ((int64_t)e * a.NF + f) * a.K + 8 * ((lane & 3) ^ swz(row));
    }
#pragma unroll
    for (int j = 0; j < XJ; ++j) {
        const int row = (w * XJ + j) * 16 + (lane >> 2);
        const int m = row < M ? row : 0;
        const int64_t src_row = MODE == 0 ? (int64_t)a.perm[p0 + m] : (int64_t)(p0 + m);
        xsrc[j] = a.src + src_row * a.K + 8 * ((lane & 3) ^ swz(row));
    }
    auto issue = [&](int slice, int stage) {
        const int k0 = slice * kBK;
#pragma unroll
        for (int j = 0; j < WJ; ++j) dma16(wsrc[j] + k0, &Ws[stage][(w * WJ + j) * 16 * kBK]);
#pragma unroll
        for (int j = 0; j < XJ; ++j) dma16(xsrc[j] + k0, &Xs[stage][(w * XJ + j) * 16 * kBK]);
    };
    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    const int nst = a.K / kBK;
    issue(0, 0);
    if (nst > 1) issue(1, 1);
    for (int s = 0; s < nst; ++s) {
        // this wave's loads of slice s have landed (those of slice s + 1 may still fly); the
        // barrier publishes every wave's and frees the stage of slice s - 1
        if (s + 1 < nst) __builtin_amdgcn_s_waitcnt(vmcnt_wait(kLoadsPerSlice));
        else __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
        __syncthreads();
        if (s + 2 < nst) issue(s + 2, (s + 2) % kStages);
        const int st = s % kStages;
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 16) {
            const int c = kk / 8 + hi;  // 16-byte chunk of the fragment
            bf16x8_t af[4], bq[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wf + 32 * i + l32;
                af[i] = *reinterpret_cast<const bf16x8_t*>(&Ws[st][row * kBK + 8 * (c ^ swz(row))]);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int row = wt + 32 * j + l32;
                bq[j] = *reinterpret_cast<const bf16x8_t*>(&Xs[st][row * kBK + 8 * (c ^ swz(row))]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bq[j], acc[i][j], 0, 0, 0);
        }
    }
    // accumulator r of tile (i, j): feature 32 i + 8 (r / 4) + 4 hi + r % 4 of the wave's block,
    // position 32 j + l32
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int m = wt + 32 * j + l32;
        if (m >= M) continue;
        const int64_t p = p0 + m;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int f = f0 + wf + 32 * i + 8 * q + 4 * hi;
                if (f >= a.NF) continue;
                float v[4];
#pragma unroll
                for (int z = 0; z < 4; ++z) v[z] = acc[i][j][4 * q + z];
                if (MODE == 0) {
#pragma unroll
                    for (int z = 0; z < 4; ++z) v[z] = ACT == GQE_ACT_RELU ? fmaxf(v[z], 0.f) : gelu(v[z]);
                    *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(a.out) + p * a.NF + f) =
                        u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                } else {
                    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(a.out) + p * a.NF + f) =
                        f32x4_t{v[0], v[1], v[2], v[3]};
                }
            }
    }
}

// y[t] = sum_r w[t, r] Y[inv[t, r]], thread per (token, 8 columns), rounded once to bf16
__global__ void moe_combine_kernel(const float* __restrict__ Y, const int32_t* __restrict__ inv,
                                   const float* __restrict__ wsel, uint16_t* __restrict__ y, int64_t T, int k, int d) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int c8 = d / 8;
    if (q >= T * c8) return;
    const int64_t t = q / c8;
    const int c = (int)(q % c8) * 8;
    float acc[8];
#pragma unroll
    for (int z = 0; z < 8; ++z) acc[z] = 0.f;
    for (int r = 0; r < k; ++r) {
        const int64_t p = inv[t * k + r];
        const float wv = wsel[t * k + r];
        const f32x4_t u = *reinterpret_cast<const f32x4_t*>(Y + p * d + c);
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(Y + p * d + c + 4);
#pragma unroll
        for (int z = 0; z < 4; ++z) {
            acc[z] += wv * u[z];
            acc[4 + z] += wv * v[z];
        }
    }
    *reinterpret_cast<u32x4_t*>(y + t * d + c) = u32x4_t{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                                         pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
}

// dst[e][c][r] = src[e][r][c] (bf16), 64 x 64 tiles through LDS
__global__ void moe_transpose_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, int R, int C) {
    __shared__ uint16_t tile[64][66];
    const int e = blockIdx.z, r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    const uint16_t* s = src + (int64_t)e * R * C;
    uint16_t* o = dst + (int64_t)e * R * C;
    for (int i = threadIdx.x; i < 64 * 64; i += blockDim.x) {
        const int rr = i >> 6, cc = i & 63;
        if (r0 + rr < R && c0 + cc < C) tile[rr][cc] = s[(int64_t)(r0 + rr) * C + c0 + cc];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += blockDim.x) {
        const int cc = i >> 6, rr = i & 63;
        if (r0 + rr < R && c0 + cc < C) o[(int64_t)(c0 + cc) * R + r0 + rr] = tile[rr][cc];
    }
}

template <int MODE>
void gemm(const MoeGemmArgs& g, int act, int64_t P, hipStream_t st) {
    MoeGemmArgs a = g;
    a.ntiles = (int)(ceil_div(P, moe_bt<MODE>()) + g.E);
    const int64_t n = (int64_t)a.ntiles * ceil_div(g.NF, kBF);
    const dim3 grid((unsigned)(8 * ceil_div(n, 8)));
    if (act == GQE_ACT_RELU) moe_gemm_kernel<MODE, GQE_ACT_RELU><<<grid, 64 * moe_waves<MODE>(), 0, st>>>(a);
    else moe_gemm_kernel<MODE, GQE_ACT_GELU><<<grid, 64 * moe_waves<MODE>(), 0, st>>>(a);
}

}  // namespace

hipError_t launch_moe_pack(const MoeDims& M, const void* w1, const void* w2, void* packed, const MoePacked& pl,
                           hipStream_t st) {
    char* pk = (char*)packed;
    // W1 [E][d][d_ff] -> [E][d_ff][d]; W2 [E][d_ff][d] -> [E][d][d_ff]
    moe_transpose_kernel<<<dim3((unsigned)ceil_div(M.dff, 64), (unsigned)ceil_div(M.d, 64), (unsigned)M.E), 256, 0,
                           st>>>((const uint16_t*)w1, (uint16_t*)(pk + pl.w1t), M.d, M.dff);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    moe_transpose_kernel<<<dim3((unsigned)ceil_div(M.d, 64), (unsigned)ceil_div(M.dff, 64), (unsigned)M.E), 256, 0,
                           st>>>((const uint16_t*)w2, (uint16_t*)(pk + pl.w2t), M.dff, M.d);
    return hipGetLastError();
}

hipError_t launch_moe_experts(const MoeDims& M, const MoePlan& P, const void* x, void* y, const void* packed,
                              const MoePacked& pl, char* ws, hipStream_t st, KernelMarks* km) {
    const char* pk = (const char*)packed;
    const int64_t np = P.r.T * M.k;
    MoeGemmArgs g{};
    g.offs = (const int32_t*)(ws + P.offs);
    g.perm = (const int32_t*)(ws + P.perm);
    g.E = M.E;
    if (km) km->begin(KM_MOE_UP);
    g.w = (const uint16_t*)(pk + pl.w1t);
    g.src = (const uint16_t*)x;
    g.out = ws + P.H;
    g.NF = M.dff;
    g.K = M.d;
    gemm<0>(g, M.act, np, st);
    if (km) km->mark(KM_MOE_UP);
    if (km) km->begin(KM_MOE_DOWN);
    g.w = (const uint16_t*)(pk + pl.w2t);
    g.src = (const uint16_t*)(ws + P.H);
    g.out = ws + P.Y;
    g.NF = M.d;
    g.K = M.dff;
    gemm<1>(g, M.act, np, st);
    if (km) km->mark(KM_MOE_DOWN);
    if (km) km->begin(KM_MOE_COMBINE);
    const int64_t n = P.r.T * (M.d / 8);
    moe_combine_kernel<<<(unsigned)ceil_div(n, 256), 256, 0, st>>>(
        (const float*)(ws + P.Y), (const int32_t*)(ws + P.inv), (const float*)(ws + P.r.wsel), (uint16_t*)y, P.r.T, M.k,
        M.d);
    if (km) km->mark(KM_MOE_COMBINE);
    return hipGetLastError();
}
