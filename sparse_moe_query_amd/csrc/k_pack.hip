// Weight repacking (layout, plus one addition for the fused output slots below):
//  - the router weights widened to float64 (exact) in the lane order of the router kernel;
//  - bf16 path: every projection head block transposed to [d_h][d] so that each matrix-core
//    lane reads eight consecutive hidden-dimension values with one 16-byte load;
//  - bf16 path: the output projections stacked into one [d][slots * d_h] matrix, slot order
//    per group g: its n expert slots, then (variant gqe) its renormalised slot; then the shared
//    head's slot.  Variant gqe with one choice per group: the renormalised weight of the single
//    choice is exactly 1, so the group's slot operand equals the chosen head's output and
//    O W_o[e] + O W_oR[g] = O (W_o[e] + W_oR[g]); each expert slot then carries that sum (formed
//    in float32, rounded once to bf16) and the renormalised slot is dropped.
#include "gqe_common.h"
#include "gqe_internal.h"

namespace {

// Router weights in float64 (exact widening of float32), zero-padded to Np = 16*NB columns:
//  lane order (matrix-core router): dst[o][cb][c][s] = W_r[8o + s][16cb + c]
//  plain (generic router):          dst[i][c]        = W_r[i][c]
__global__ void pack_router_kernel(const float* __restrict__ w, const float* __restrict__ b, int d,
                                   int N, int Np, int lane_order, double* __restrict__ dst,
                                   double* __restrict__ bd) {
    const int64_t total = (int64_t)d * Np;
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q < total) {
        int i, c;
        if (lane_order) {
            const int s = (int)(q % 8);
            const int64_t r = q / 8;
            const int col = (int)(r % 16);
            const int64_t r2 = r / 16;
            const int NB = Np / 16;
            const int cb = (int)(r2 % NB);
            const int o = (int)(r2 / NB);
            i = 8 * o + s;
            c = 16 * cb + col;
        } else {
            i = (int)(q / Np);
            c = (int)(q % Np);
        }
        dst[q] = (w && c < N) ? (double)w[(int64_t)i * N + c] : 0.0;
    }
    if (q < N) bd[q] = b ? (double)b[q] : 0.0;
}

__global__ void pack_proj_kernel(const uint16_t* __restrict__ wk, const uint16_t* __restrict__ wv,
                                 const uint16_t* __restrict__ wqs, const uint16_t* __restrict__ wq,
                                 int d, int G, int dh, int s, int N, uint16_t* __restrict__ dst) {
    const int64_t per = (int64_t)dh * d;
    const int64_t total = (int64_t)(2 * G + s + N) * per;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
         q += (int64_t)gridDim.x * blockDim.x) {
        const int hb = (int)(q / per);
        const int64_t r = q % per;
        const int j = (int)(r / d), i = (int)(r % d);
        uint16_t v;
        if (hb < G) v = wk[(int64_t)i * G * dh + (int64_t)hb * dh + j];
        else if (hb < 2 * G) v = wv[(int64_t)i * G * dh + (int64_t)(hb - G) * dh + j];
        else if (s && hb == 2 * G) v = wqs[(int64_t)i * dh + j];
        else {
            const int e = hb - 2 * G - s;
            v = wq[((int64_t)e * d + i) * dh + j];
        }
        dst[q] = v;
    }
}

// dst[col][slot * dh + j] = W_slot[j][col]
// W_stack for the matrix-core combine, as the LDS image of each (128-column tile, slot) stage:
// dst[((ct * slots + slot) * 128 + c) * pitch * 8 + j] = W_stack[slot * dh + j][ct * 128 + c] for
// j < dh, zero for the pad chunk (pitch = d_h / 8 rounded up to odd, in 16-byte chunks).
// Slot order: per group its n experts then (gqe) its weighted-sum slot; the shared head last.
// fuse: no weighted-sum slot, W_oR[g] added into each expert slot of group g.
__global__ void pack_wo_kernel(const uint16_t* __restrict__ wo, const uint16_t* __restrict__ wor,
                               const uint16_t* __restrict__ wos, int d, int G, int n, int dh,
                               int rslot, int fuse, int slots, int pitch, uint16_t* __restrict__ dst) {
    const int64_t per_col = (int64_t)pitch * 8;
    const int64_t total = (int64_t)d * slots * per_col;
    const int per_group = n + rslot;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
         q += (int64_t)gridDim.x * blockDim.x) {
        const int j = (int)(q % per_col);
        const int64_t rest = q / per_col;
        const int c = (int)(rest % 128);
        const int64_t rest2 = rest / 128;
        const int slot = (int)(rest2 % slots);
        const int ct = (int)(rest2 / slots);
        const int col = ct * 128 + c;
        uint16_t v = 0;
        if (j < dh) {
            if (slot < G * per_group) {
                const int g = slot / per_group, u = slot % per_group;
                if (u < n) {
                    v = wo[((int64_t)(g * n + u) * dh + j) * d + col];
                    if (fuse) {
                        const float f = __uint_as_float((uint32_t)v << 16) +
                                        __uint_as_float((uint32_t)wor[((int64_t)g * dh + j) * d + col] << 16);
                        v = from_f32<bf16_t>(f).bits;
                    }
                } else {
                    v = wor[((int64_t)g * dh + j) * d + col];
                }
            } else {
                v = wos[(int64_t)j * d + col];
            }
        }
        dst[q] = v;
    }
}

// Rotary embedding frequencies in cycles per position: rev[i] = base^(-2i/d_h) / (2 pi), float64.
__global__ void rope_table_kernel(double base, int dh, double* __restrict__ rev) {
    const int i = threadIdx.x;
    if (i < 64) rev[i] = (base > 0.0 && 2 * i < dh) ? pow(base, -2.0 * i / dh) / 6.283185307179586476925 : 0.0;
}

}  // namespace

hipError_t launch_pack_router(const GqeDims& D, const float* w_router, const float* b_router, size_t wr64_off,
                              size_t br64_off, void* packed, hipStream_t st) {
    char* pk = (char*)packed;
    const int Np = (int)round_up(D.N, 16);
    const int64_t m = (int64_t)D.d * Np + D.N;
    pack_router_kernel<<<(unsigned)ceil_div(m, 256), 256, 0, st>>>(w_router, b_router, D.d, D.N, Np,
                                                                   router_uses_mfma(D) ? 1 : 0,
                                                                   (double*)(pk + wr64_off), (double*)(pk + br64_off));
    return hipGetLastError();
}

hipError_t launch_pack(const GqeDims& D, const gqe_weights_t& w, const PackedLayout& pl,
                       void* packed, bool mfma, hipStream_t st) {
    char* pk = (char*)packed;
    hipError_t e = launch_pack_router(D, w.w_router, w.b_router, pl.wr64, pl.br64, packed, st);
    if (e != hipSuccess) return e;
    rope_table_kernel<<<1, 64, 0, st>>>((double)D.rope, D.dh, (double*)(pk + pl.rope));
    e = hipGetLastError();
    if (e != hipSuccess || !mfma) return e;
    pack_proj_kernel<<<1024, 256, 0, st>>>((const uint16_t*)w.w_k, (const uint16_t*)w.w_v,
                                           (const uint16_t*)w.w_q_shared, (const uint16_t*)w.w_q,
                                           D.d, D.G, D.dh, D.s, D.N, (uint16_t*)(pk + pl.wproj));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int rslot = (!D.dense && D.variant == GQE_VARIANT_GQE && !pl.rslot_fused) ? 1 : 0;
    if (pl.wo_pitch == 0) return hipSuccess;  // combine on the scalar path
    pack_wo_kernel<<<1024, 256, 0, st>>>((const uint16_t*)w.w_o, (const uint16_t*)w.w_o_rslot,
                                         (const uint16_t*)w.w_o_shared, D.d, D.G, D.n, D.dh, rslot,
                                         pl.rslot_fused, pl.slots, pl.wo_pitch, (uint16_t*)(pk + pl.wo));
    return hipGetLastError();
}
