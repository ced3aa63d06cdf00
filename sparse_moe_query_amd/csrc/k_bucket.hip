// Global token-to-expert bucketing of a forward's routing (gfx950).
//
// GQE README "Algorithm Overview": a router picks k experts per token in every GQA group and only
// those experts' query heads are computed.  The projection kernel gathers each routed expert's rows
// tile by tile; this is the global form of the same gather: the T*G*k assignments (t, g, r),
// sorted stably by expert id (tokens ascending inside each expert), with the inverse map.
//
//   histogram  the router already counts every expert per 64-token block (part_cnt [blk][N])
//   scan       one wave per expert: exclusive prefix of its block counts (each lane sums a
//              contiguous run of blocks, then a wave-wide shuffle scan); expert totals give offs
//   scatter    one wave per 64-token block: for every expert a ballot of the lanes whose token
//              chose it (at any rank); a lane's place is the popcount of the ballot below it, so
//              positions follow token order exactly as a stable sort does
#include "gqe_common.h"
#include "gqe_internal.h"

namespace {

constexpr int kBlk = 64;  // tokens per router block (the router's statistics granularity)

__device__ __forceinline__ int wave_excl_scan(int v, int lane, int* total) {
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    *total = __shfl(x, 63);
    return x - v;
}

// offs[e] and boff[blk][e] = assignments to expert e in blocks before blk.
__global__ void __launch_bounds__(1024) bucket_scan_kernel(const int32_t* __restrict__ part_cnt, int64_t nblk, int N,
                                                          int32_t* __restrict__ boff, int32_t* __restrict__ offs) {
    __shared__ int tot[64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t per = (nblk + 63) / 64;
    for (int e = wv; e < N; e += 16) {
        const int64_t b0 = lane * per, b1 = min(nblk, b0 + per);
        int s = 0;
        for (int64_t b = b0; b < b1; ++b) s += part_cnt[b * N + e];
        int total;
        int run = wave_excl_scan(s, lane, &total);
        for (int64_t b = b0; b < b1; ++b) {
            boff[b * N + e] = run;
            run += part_cnt[b * N + e];
        }
        if (lane == 0) tot[e] = total;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int acc = 0;
        for (int e = 0; e < N; ++e) {
            offs[e] = acc;
            acc += tot[e];
        }
        offs[N] = acc;
    }
}

__global__ void __launch_bounds__(64) bucket_scatter_kernel(const int32_t* __restrict__ idx, const int32_t* __restrict__ boff,
                                                           const int32_t* __restrict__ offs, int64_t T, int G, int k, int n,
                                                           int N, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    const int lane = threadIdx.x;
    const int64_t blk = blockIdx.x;
    const int64_t t = blk * kBlk + lane;
    const bool valid = t < T;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int g = 0; g < G; ++g) {
        // the lane's choices in this group (each expert at most once)
        for (int j = 0; j < n; ++j) {
            const int ej = g * n + j;
            int rj = -1;
            if (valid)
                for (int r = 0; r < k; ++r)
                    if (idx[(t * G + g) * k + r] == ej) rj = r;
            const uint64_t m = __builtin_amdgcn_ballot_w64(rj >= 0);
            if (rj >= 0) {
                const int pos = offs[ej] + boff[blk * N + ej] + __builtin_popcountll(m & below);
                perm[pos] = (int32_t)t;
                inv[(t * G + g) * k + rj] = pos;
            }
        }
    }
}

}  // namespace

hipError_t launch_bucket(const GqeDims& D, const WorkPlan& P, char* ws, int32_t* offs, int32_t* perm, int32_t* inv,
                         hipStream_t st) {
    const int32_t* part_cnt = (const int32_t*)(ws + P.part_cnt);
    int32_t* boff = (int32_t*)(ws + P.bucket_boff);
    bucket_scan_kernel<<<1, 1024, 0, st>>>(part_cnt, P.nblk_router, D.N, boff, offs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    bucket_scatter_kernel<<<(unsigned)P.nblk_router, 64, 0, st>>>((const int32_t*)(ws + P.idx), boff, offs, P.T, D.G,
                                                                  D.k, D.n, D.N, perm, inv);
    return hipGetLastError();
}
