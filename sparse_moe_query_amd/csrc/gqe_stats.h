// Final reduction of the router's per-block expert statistics (one work group of at least 256
// threads, all of which call it; LDS scratch passed in: ps and pc 256 entries each, fp 64): counts, mean in-group probability, and the Switch-style balance loss.
//
// GQE README "Algorithm Overview": a Switch-style load-balancing auxiliary loss.  With T tokens
// and k choices per group: f_e = count_e / (T k), P_e = (1/T) sum_t p_e(t), per group
// n sum_{e in g} f_e P_e, averaged over the groups.  The partial sums are added in a fixed order,
// so the result does not depend on scheduling.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

__device__ __forceinline__ void stats_finalize_block(const int32_t* __restrict__ part_cnt,
                                                     const double* __restrict__ part_psum, int64_t nblk,
                                                     int64_t T, int N, int G, int k, char* __restrict__ stats,
                                                     double* ps, int64_t* pc, double* fp) {
    int64_t* counts = reinterpret_cast<int64_t*>(stats);
    double* mean = reinterpret_cast<double*>(stats + 8 * N);
    double* aux = reinterpret_cast<double*>(stats + 16 * N);
    const int J = 256 / N;
    const bool mine = threadIdx.x < 256;  // larger work groups: the other threads only meet the barriers
    const int e = threadIdx.x % N, j = threadIdx.x / N;
    double s = 0.0;
    int64_t c = 0;
    if (mine && j < J) {
        for (int64_t b = j; b < nblk; b += J) {
            c += part_cnt[b * N + e];
            s += part_psum[b * N + e];
        }
    }
    if (mine) {
        ps[threadIdx.x] = s;
        pc[threadIdx.x] = c;
    }
    __syncthreads();
    if (threadIdx.x < N) {
        double tot = 0.0;
        int64_t ct = 0;
        for (int jj = 0; jj < J; ++jj) {
            tot += ps[jj * N + threadIdx.x];
            ct += pc[jj * N + threadIdx.x];
        }
        counts[threadIdx.x] = ct;
        const double P = tot / (double)T;
        mean[threadIdx.x] = P;
        fp[threadIdx.x] = ((double)ct / ((double)T * (double)k)) * P;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int n = N / G;
        double tot = 0.0;
        for (int g = 0; g < G; ++g) {
            double Lg = 0.0;
            for (int jj = 0; jj < n; ++jj) Lg += fp[g * n + jj];
            tot += (double)n * Lg;
        }
        *aux = tot / (double)G;
    }
}
