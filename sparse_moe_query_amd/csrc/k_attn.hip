// Causal flash attention of the GQE layer on gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// GQE README "Algorithm Overview": the routed query heads of a group and the always-on shared
// head attend to the group's dense, unchanged KV head.  A work item is (batch b, group g, block of
// positions); its 256 query columns are all (position, head) pairs of the group's active heads, so
// every K/V tile staged in LDS serves the k routed heads (+ the shared head for its group) at once.
// A work group runs one job of the schedule (built in the workspace by k_sched.hip): an item, or a
// chunk of consecutive key tiles of a long item (its unnormalised partial result is combined by
// attn_merge_kernel).
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
// Fast interior tiles run in phases so that matrix-core and exp / convert work overlap inside a
// wave (S of query tile 1 under the softmax of tile 0, P.V of tile 0 under the softmax of tile 1).
#include <type_traits>

#include "gqe_common.h"
#include "gqe_internal.h"

namespace {

constexpr int kWaves = 4;
constexpr int kQW = 64;                // query columns per wave
constexpr int kCols = kWaves * kQW;    // query columns per work item
static_assert(kCols == GQE_ATTN_COLS, "the schedule's item width");
constexpr int kBN = GQE_KV_TILE;       // keys per LDS tile
constexpr float kLazy = 8.0f;          // raise the running offset only when it grows by > 2^8
constexpr float kFastBound = 64.0f;    // |S| <= 64 (log2 units) keeps exp2 in range without offset

struct AttnArgs {
    const bf16_t* Q;
    const bf16_t* K;
    const bf16_t* Vt;
    const float* knt;     // largest key norm of every 64-key tile [B][G][S_pad / 64]
    const int32_t* jobs;  // AttnJob records (8 int32 each), dispatch order
    bf16_t* O;
    float* part_o;        // partial results of split items: [slot][256 columns][d_h]
    float* part_ml;       //   and their (running offset m, row sum l) [slot][256 columns][2]
    float* lse;           // row log-sum-exp m + log2(l) of every stored query row [T][H] (the backward's)
    int64_t S, S_pad;
    int G, H, k;
};

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

// LDS rows of the K and V^T tiles sit at an odd pitch of 16-byte chunks (K: d_h/8 chunks, plus one
// pad chunk when that is even; V^T: 8 chunks of keys + 1 pad), so that a fragment read -- sixteen
// lanes per LDS cycle, sixteen consecutive rows, the same chunk -- touches sixteen distinct
// 16-byte bank groups of the 256-byte bank row, and every fragment of a tile is one base address
// plus a constant offset.
template <int DH>
__host__ __device__ constexpr int kpitch() { return (DH / 8) | 1; }
constexpr int kVP = 9;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o));
    return v;
}

// Masks the keys past the lane's position (keys of the diagonal tile): S^T register j of subtile
// kst is key key0 + 32 kst + 8 (j / 4) + 4 (lane / 32) + j % 4 of the lane's query column.
__device__ __forceinline__ void mask_diag(f32x16_t (&sacc)[2], int key0, int pos, int lane) {
    const int lim = pos - key0 - 4 * (lane >> 5);
#pragma unroll
    for (int kst = 0; kst < 2; ++kst)
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (32 * kst + 8 * (j >> 2) + (j & 3) > lim) sacc[kst][j] = -INFINITY;
}

// Online softmax step of one query tile (tiles that fail the range test): the tile maximum of the
// lane's column (combined with lane l^32 by v_permlane32_swap); the running offset is raised
// lazily, only when the maximum exceeds it by more than 2^8, and then the tile's O accumulators
// are rescaled (alpha of each accumulator row fetched from the lane that owns that column).
// Returns the additive offset for exp2 (-m, or 0 while nothing is accumulated).
template <int NCB>
__device__ __forceinline__ float tile_offset(const f32x16_t (&sacc)[2], float& mrun, f32x16_t (&oacc)[NCB], float& lsum,
                                             int lane) {
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
        lsum *= alpha;  // the lane's own column
        // accumulator register j of this lane is query row 8 (j / 4) + 4 (lane / 32) + j % 4,
        // whose alpha lives in the lane of that column
        // (the lane id is made opaque here so that the sixteen source addresses are formed in
        // this rare branch, one base plus constant offsets, instead of being hoisted out of the
        // tile loop as sixteen live registers)
        int lsrc = lane;
        asm volatile("" : "+v"(lsrc));
        const int base = 16 * (lsrc >> 5);  // byte address of lane 4 (lane / 32)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float aj = __int_as_float(
                __builtin_amdgcn_ds_bpermute(base + 4 * (8 * (j >> 2) + (j & 3)), __float_as_int(alpha)));
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) oacc[cb][j] *= aj;
        }
    }
    return mrun == -INFINITY ? 0.f : -mrun;
}

// P = exp2(S + nm) for one half-group (hg = 0..7) of a query tile's scores, packed to bf16 (nm = 0
// on fast tiles): registers 8 u + 4 half .. +3 of subtile kst (hg = 4 kst + 2 u + half) -> words
// 2 half, 2 half + 1 of p[2 kst + u], the A operand of 16-key chunk 2 kst + u.
template <bool FAST, bool ROWSUM>
__device__ __forceinline__ void exp_pack_half(const f32x16_t (&sacc)[2], u32x4_t (&p)[4], int hg, float nm, float& lsum) {
    const int kst = hg >> 2, u = (hg >> 1) & 1, hf = hg & 1;
    const int j = 8 * u + 4 * hf;
    float e[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) e[t] = __builtin_amdgcn_exp2f(FAST ? sacc[kst][j + t] : sacc[kst][j + t] + nm);
    p[2 * kst + u][2 * hf] = pack_bf16x2(e[0], e[1]);
    p[2 * kst + u][2 * hf + 1] = pack_bf16x2(e[2], e[3]);
    if constexpr (ROWSUM) {
        // the lane's partial row sum of the same bf16 P that multiplies V (dot with (1, 1)).  The
        // words go through an empty asm first: fed straight from the 128-bit operand tuple, the
        // compiler gave every v_dot2c of a group the tuple's first register.
        const bf16x2_t one2 = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
        uint32_t w0 = p[2 * kst + u][2 * hf], w1 = p[2 * kst + u][2 * hf + 1];
        asm("" : "+v"(w0), "+v"(w1));
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w0), one2, lsum, false);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w1), one2, lsum, false);
    }
    // an empty use keeps the work at this point of the instruction stream (otherwise it is sunk
    // to the matrix instruction that consumes it, and the interleaving is lost)
    asm volatile("" ::"v"(p[2 * kst + u][2 * hf]), "v"(p[2 * kst + u][2 * hf + 1]));
}

template <int DH>
__global__ void __launch_bounds__(256, 2) attn_fwd_kernel(AttnArgs a) {
    constexpr int KS = DH / 16;        // k-steps of the 32x32x16 QK^T product
    // Row sums: when d_h is not a multiple of 32 (48), the last 32-wide column block of the P.V
    // product has room for a column of ones and the matrix core forms them ([V | 1 | 0]); otherwise
    // each lane sums its bf16 P with v_dot2 (no extra column block).
    constexpr bool ONES = DH % 32 != 0;
    constexpr int NCB = ONES ? DH / 32 + 1 : DH / 32;  // 32-wide column blocks of the P.V product
    constexpr int CBS = DH / 32;       // the column block holding row DH (the ones row), if ONES
    constexpr int KC8 = DH / 8;        // 16-byte chunks per key row
    constexpr int KP = kpitch<DH>();   // LDS pitch of a key row in chunks (odd)
    constexpr int SEGK = KP;           // 1 KB segments (64 chunks, one wave-wide load) per K tile
    constexpr int SEGV = (DH * kVP + 63) / 64;  // per V^T tile (the last one may run past row DH-1)
    constexpr int TILE_K = SEGK * 512;  // elements of a K tile in LDS
    constexpr int TILE_V = SEGV * 512;
    constexpr int LK = (SEGK + 3) / 4;  // direct loads per wave per tile (same for every wave)
    constexpr int LV = (SEGV + 3) / 4;
    constexpr int NSTAGE = 3;
    constexpr int XR = ONES ? NCB * 32 - DH : 1;  // rows of the last block past d_h: row DH is ones
    __shared__ __align__(1024) uint16_t ks_lds[NSTAGE][TILE_K];
    __shared__ __align__(1024) uint16_t vs_lds[NSTAGE][TILE_V];
    __shared__ __align__(1024) uint16_t one_lds[XR * kVP * 8];  // rows DH.. of [V | 1 | 0]^T
    constexpr int KNL = 1024;                  // key-tile maxima of a job kept in LDS
    __shared__ float knt_lds[KNL];
    __shared__ float knt_tail[kWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // the job: eight wave-uniform int32 (scalar loads)
    typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
    const_i32_ptr jb = (const_i32_ptr)(a.jobs + 8 * (int64_t)blockIdx.x);
    const int ib = jb[0], ig = jb[1], NH = jb[2], p0 = jb[3], np = jb[4];
    const int kt0 = jb[5], kt_end = jb[6], part = jb[7];
    if (kt_end <= kt0) return;  // an empty job does nothing
    const int S = (int)a.S;  // the host limits a call to 2^28 tokens
    const int last_pos = min(p0 + np, S) - 1;  // last query position of the item

    const bf16_t* Kg = a.K + ((int64_t)ib * a.G + ig) * a.S_pad * DH;
    const bf16_t* Vg = a.Vt + ((int64_t)ib * a.G + ig) * (int64_t)DH * a.S_pad;

    // ---------------------------------------------------------------- query columns of the lane
    bf16x8_t qf[2][KS];
    int posq[2];
    float mrun[2] = {-INFINITY, -INFINITY};
    float qsq[2];  // sum of squares of the lane's half of the query column's dims
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        const int c = w * kQW + qt * 32 + (lane & 31);
        const int p = c / NH, h = c % NH;
        const int pos = p0 + p;
        const bool valid = (p < np) && (pos < S);
        posq[qt] = valid ? pos : S - 1;
        const int vh = h < a.k ? ig * a.k + h : a.G * a.k;
        const bf16_t* qr = a.Q + (((int64_t)ib * a.H + vh) * S + posq[qt]) * DH + 8 * (lane >> 5);
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
    const int wfirst = min(p0 + cfirst / NH, S - 1);
    const int wlast = min(min(p0 + min(clast / NH, np - 1), S - 1), last_pos);
    const int wtiles = wlast / kBN + 1;

    // O accumulators: [qt][column block], 32 query rows x 32 columns of [V | 1 | 0] each
    f32x16_t oacc[2][NCB];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) oacc[qt][cb] = f32x16_t{};
    float lsum[2] = {0.f, 0.f};  // !ONES: the lane's partial row sums (its half of the keys)
    bool offset_zero = true;  // wave-uniform: every lane's offset is 0 or unset

    // rows DH.. of the [V | 1 | 0]^T operand: row DH all ones, the rest zero
    for (int i = tid; i < XR * kVP * 8; i += 256) one_lds[i] = (i < kVP * 8) ? (uint16_t)0x3f80 : (uint16_t)0;

    // Tiles go straight from global memory into LDS (global_load_lds_dwordx4: each wave-wide load
    // fills one contiguous 1 KB segment, lane i its 16 bytes at 16 i).  Every lane therefore loads
    // the global chunk that belongs at its LDS position (pad chunks: any chunk of the same row).
    // Three stages: while tile kt computes, tile kt+1 has landed or is landing and tile kt+2 is in
    // flight.  Every wave issues the same number of loads per tile (segments past the end are
    // re-issued, same bytes), so the wait is a compile-time vmcnt.
    // Per lane and load, the source relative to the tile's first key: K as a byte offset from the
    // tile's first key row, V^T as an element offset (row r, chunk c).
    uint32_t koff[LK];
    int64_t voff[LV];
#pragma unroll
    for (int i = 0; i < LK; ++i) {
        const int seg = min(w + 4 * i, SEGK - 1);
        const int q = seg * 64 + lane;          // chunk position in the tile
        const int r = q / KP, cpos = q % KP;    // key row, chunk slot
        const int c = cpos < KC8 ? cpos : 0;
        koff[i] = (uint32_t)((r * DH + 8 * c) * 2);
    }
#pragma unroll
    for (int i = 0; i < LV; ++i) {
        const int seg = min(w + 4 * i, SEGV - 1);
        const int q = seg * 64 + lane;
        const int r = min(q / kVP, DH - 1), cpos = q % kVP;  // LDS rows past DH-1 are never read
        const int c = cpos < 8 ? cpos : 0;
        voff[i] = (int64_t)r * a.S_pad + 8 * c;
    }
    auto issue = [&](int kt, int stage) {
        const int64_t key0 = (int64_t)kt * kBN;
        const bf16_t* kbase = Kg + key0 * DH;
#pragma unroll
        for (int i = 0; i < LK; ++i) dma16(kbase, koff[i], &ks_lds[stage][min(w + 4 * i, SEGK - 1) * 512]);
#pragma unroll
        for (int i = 0; i < LV; ++i) dma16(Vg + key0 + voff[i], &vs_lds[stage][min(w + 4 * i, SEGV - 1) * 512]);
    };
    // the largest key norm of each of the job's tiles, staged in LDS (read one tile ahead in the
    // loop); tiles past the first KNL (jobs longer than 64K keys) share one maximum
    {
        const float* kg = a.knt + ((int64_t)ib * a.G + ig) * (a.S_pad / kBN) + kt0;
        float tail = 0.f;
        for (int i = tid; i < kt_end - kt0; i += 256) {
            const float v = kg[i];
            if (i < KNL) knt_lds[i] = v;
            else tail = __builtin_fmaxf(tail, v);
        }
        tail = wave_max(tail);
        if (lane == 0) knt_tail[w] = tail;
    }
    constexpr int NLOAD = LK + LV;  // vector-memory operations issued per tile per wave

    // Fragment reads: K row 32 kst + (lane & 31), chunk 2 kk + hsel; [V | 1 | 0]^T row
    // n = 32 cb + (lane & 31), chunk 2 ch + hsel (the lane's half of 16-key chunk ch of the slotted
    // key order).  Rows n >= DH come from one_lds; in the last column block that choice is per lane.
    const int hsel = lane >> 5;
    const int lrow = lane & 31;
    const int kfo = (lrow * KP + hsel) * 8;  // element offsets of the lane's fragment bases
    const int vfo = (lrow * kVP + hsel) * 8;
    const bool lane_ones = 32 * CBS + lrow >= DH;
    const uint16_t* one_base = one_lds + (lane_ones ? (32 * CBS + lrow - DH) * kVP * 8 : 0) + hsel * 8;
    auto vfrag = [&](const uint16_t* vb, int ch, int cb) {
        const uint16_t* src =
            (ONES && cb == CBS && lane_ones) ? one_base + 16 * ch : vb + vfo + (32 * cb * kVP + 2 * ch) * 8;
        return *reinterpret_cast<const bf16x8_t*>(src);
    };

    // One 64-key tile, in phases so that the matrix core and the exp / convert work of the
    // softmax overlap inside the wave: S of query tile 0; S of query tile 1, each matrix
    // instruction followed by its share of tile 0's exp2 + pack; P.V of tile 0, each followed by
    // its share of tile 1's exp2 + pack; P.V of tile 1.  DIAG tiles mask the keys past each
    // column's position first; tiles that fail the range test (!FAST) take the online-softmax
    // offset step before their exponentials.
    auto body = [&](int kt, bool fast, bool diag) {
        const int stage = (kt - kt0) % NSTAGE;
        const uint16_t* kb = ks_lds[stage];
        const uint16_t* vb = vs_lds[stage];
        // Rare tiles (diagonal, or failing the range test) adjust S in place before its
        // exponentials -- mask the keys past each column's position; take the online-softmax
        // offset step and subtract the offset -- so that every tile then runs the same code
        // (one set of matrix instructions; variant bodies would leave the accumulators in
        // different registers and cost copies at every join).
        const bool adjust = diag || !fast;
        auto adjust_tile = [&](f32x16_t (&sc)[2], int qt) {
            if (diag) mask_diag(sc, kt * kBN, posq[qt], lane);
            if (!fast) {
                const float nm = tile_offset<NCB>(sc, mrun[qt], oacc[qt], lsum[qt], lane);
#pragma unroll
                for (int kst = 0; kst < 2; ++kst)
#pragma unroll
                    for (int j = 0; j < 16; ++j) sc[kst][j] += nm;
            }
        };
        // K fragments of both 32-key subtiles (shared by the two query tiles)
        bf16x8_t kf[2][KS];
#pragma unroll
        for (int kst = 0; kst < 2; ++kst)
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
                kf[kst][kk] = *reinterpret_cast<const bf16x8_t*>(kb + kfo + (32 * kst * KP + 2 * kk) * 8);
        if constexpr (DH > 48) {
            // d_h = 64 (64 accumulator registers + 32 of queries): one query tile at a time,
            // re-reading the K fragments for the second, then P.V of both tiles per V fragment
            u32x4_t pa[2][4];
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                if (qt == 1) {
#pragma unroll
                    for (int kst = 0; kst < 2; ++kst)
#pragma unroll
                        for (int kk = 0; kk < KS; ++kk)
                            kf[kst][kk] = *reinterpret_cast<const bf16x8_t*>(kb + kfo + (32 * kst * KP + 2 * kk) * 8);
                }
                f32x16_t sc[2] = {};
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
#pragma unroll
                    for (int kst = 0; kst < 2; ++kst)
                        sc[kst] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kst][kk], qf[qt][kk], sc[kst], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                if (adjust) adjust_tile(sc, qt);
#pragma unroll
                for (int hg = 0; hg < 8; ++hg) exp_pack_half<true, !ONES>(sc, pa[qt], hg, 0.f, lsum[qt]);
            }
#pragma unroll
            for (int ch = 0; ch < 4; ++ch)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    const bf16x8_t vf = vfrag(vb, ch, cb);
#pragma unroll
                    for (int qt = 0; qt < 2; ++qt)
                        oacc[qt][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, pa[qt][ch]),
                                                                               vf, oacc[qt][cb], 0, 0, 0);
                }
        } else {
            // d_h <= 48, in phases so that the matrix core and the exp / convert work of the
            // softmax overlap inside the wave: S of query tile 0; S of query tile 1, each matrix
            // instruction followed by its share of tile 0's exp2 + pack (and, as the K fragments
            // die, one [V | 1 | 0] fragment read); P.V of tile 0, each followed by its share of
            // tile 1's exp2 + pack; P.V of tile 1.
            constexpr int MA = 2 * KS, MB = 4 * NCB;
            f32x16_t s0[2] = {}, s1[2] = {};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
#pragma unroll
                for (int kst = 0; kst < 2; ++kst)
                    s0[kst] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kst][kk], qf[0][kk], s0[kst], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (adjust) adjust_tile(s0, 0);
            u32x4_t p0[4], p1[4];
            bf16x8_t vf[MB];  // index ch * NCB + cb
#pragma unroll
            for (int i = 0; i < MA; ++i) {
                const int kk = i >> 1, kst = i & 1;
                s1[kst] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kst][kk], qf[1][kk], s1[kst], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int hg = 0; hg < 8; ++hg)
                    if (hg * MA / 8 == i) exp_pack_half<true, !ONES>(s0, p0, hg, 0.f, lsum[0]);
                if (i < MB) vf[i] = vfrag(vb, i / NCB, i % NCB);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int i = MA; i < MB; ++i) vf[i] = vfrag(vb, i / NCB, i % NCB);
            if (adjust) adjust_tile(s1, 1);
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const int ch = i / NCB, cb = i % NCB;
                oacc[0][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, p0[ch]), vf[i],
                                                                      oacc[0][cb], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int hg = 0; hg < 8; ++hg)
                    if (hg * MB / 8 == i) exp_pack_half<true, !ONES>(s1, p1, hg, 0.f, lsum[1]);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int i = 0; i < MB; ++i)
                oacc[1][i % NCB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, p1[i / NCB]), vf[i],
                                                                          oacc[1][i % NCB], 0, 0, 0);
        }
        if (fast) {
            mrun[0] = 0.f;  // from unset (nothing accumulated) or already 0
            mrun[1] = 0.f;
        }
    };

    // The query fragments are the only loads into registers the compiler tracks; waiting for them
    // here leaves it nothing outstanding, so it never adds a vmcnt wait inside the loop (it does not
    // see the direct-to-LDS loads, and a wait of its own there would drain the prefetch).
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    issue(kt0, 0);
    if (kt_end > kt0 + 1) {
        issue(kt0 + 1, 1);
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(NLOAD));
    } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_wait(0));
    }
    __syncthreads();

    const float knt_far = fmax3(knt_tail[0], knt_tail[1], __builtin_fmaxf(knt_tail[2], knt_tail[3]));
    auto kmax_of = [&](int kt) { return kt - kt0 < KNL ? knt_lds[kt - kt0] : knt_far; };
    float kmax_next = kmax_of(kt0);
    for (int kt = kt0; kt < kt_end; ++kt) {
        const bool ahead = kt + 2 < kt_end;
        if (ahead) issue(kt + 2, (kt + 2 - kt0) % NSTAGE);
        const float kmax_cur = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(kmax_next)));
        kmax_next = kmax_of(min(kt + 1, kt_end - 1));
        if (kt < wtiles) {
            const bool fast = offset_zero && (qmax_w * kmax_cur * 1.02f <= kFastBound);
            const bool diag = kt * kBN + kBN - 1 > wfirst;
            body(kt, fast, diag);
            if (!fast) {
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
    constexpr int CS = DH % 32;
    if (part >= 0) {
        // a chunk of a split item: the unnormalised accumulators, the row sums and the running
        // offsets of all 256 columns go to the partial slot (a wave with no tile in the chunk
        // writes O = 0, l = 0, m = -inf)
        float* po = a.part_o + (int64_t)part * kCols * DH;
        float* pml = a.part_ml + (int64_t)part * kCols * 2;
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
            const int cbase = w * kQW + qt * 32;
            if constexpr (!ONES) {
                const uint32_t lb = __float_as_uint(lsum[qt]);
                auto sw = __builtin_amdgcn_permlane32_swap(lb, lb, false, false);
                if (lane < 32) pml[2 * (cbase + lane) + 1] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            }
            if (lane < 32) pml[2 * (cbase + lane)] = mrun[qt];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int c = cbase + 8 * (j >> 2) + 4 * hsel + (j & 3);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    const int n = 32 * cb + lrow;
                    if (n < DH) po[c * DH + n] = oacc[qt][cb][j];
                    else if (ONES && n == DH) pml[2 * c + 1] = oacc[qt][cb][j];
                }
            }
        }
        return;
    }
    // The normalised bf16 tile of the wave's 64 query columns goes through a wave-private LDS
    // region (the K / V stages are free: the loop's last barrier is behind every wave's reads and
    // no load is in flight) so that each (token, head) row of O is written in 16-byte pieces;
    // from the accumulators a lane holds one head dim of a row, and every store would write
    // 2-byte elements of two rows.
    constexpr int SP = DH + 8;  // staging pitch (bf16): 16-byte aligned rows; the pad holds l and m
    static_assert(2 * kQW * SP <= NSTAGE * TILE_K && 2 * kQW * SP <= NSTAGE * TILE_V, "staging fits");
    uint16_t* const ost = (w < 2 ? &ks_lds[0][0] : &vs_lds[0][0]) + (w & 1) * kQW * SP;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
        float ltot = 0.f;  // !ONES: the full row sum of the lane's column (both key halves)
        if constexpr (!ONES) {
            const uint32_t lb = __float_as_uint(lsum[qt]);
            auto sw = __builtin_amdgcn_permlane32_swap(lb, lb, false, false);
            ltot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int row = 8 * (j >> 2) + 4 * hsel + (j & 3);
            const float lrow_sum = ONES ? __shfl(oacc[qt][CBS < NCB ? CBS : 0][j], CS + 32 * hsel) : __shfl(ltot, row);
            const float sc = 1.0f / lrow_sum;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const int n = 32 * cb + lrow;
                if (n < DH) ost[(qt * 32 + row) * SP + n] = from_f32<bf16_t>(oacc[qt][cb][j] * sc).bits;
            }
            // the row sum goes to the row's pad (elements DH, DH + 1), for the log-sum-exp
            if (lrow == 0) *reinterpret_cast<float*>(&ost[(qt * 32 + row) * SP + DH]) = lrow_sum;
        }
    }
    // the offset of each column (lanes 0..31 hold those of both query tiles) beside its row sum
    if (lane < 32)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) *reinterpret_cast<float*>(&ost[(qt * 32 + lane) * SP + DH + 2]) = mrun[qt];
    __syncthreads();
    constexpr int C8 = DH / 8;  // 16-byte pieces per row
#pragma unroll
    for (int it = 0; it < C8; ++it) {
        const int q = lane + 64 * it, r = q / C8, ch = q - r * C8;
        const int c = w * kQW + r;
        const int p = c / NH, h = c - p * NH;
        const int pos = p0 + p;
        if (p < np && pos < S) {
            const int v = h < a.k ? ig * a.k + h : a.G * a.k;
            const int64_t orow = ((int64_t)ib * S + pos) * a.H + v;
            *reinterpret_cast<u32x4_t*>(a.O + orow * DH + 8 * ch) = *reinterpret_cast<const u32x4_t*>(&ost[r * SP + 8 * ch]);
        }
    }
    {
        // the row log-sum-exp m + log2(l) of the lane's row, kept for the backward
        const int c = w * kQW + lane;
        const int p = c / NH, h = c - p * NH;
        const int pos = p0 + p;
        if (p < np && pos < S) {
            const float l = *reinterpret_cast<const float*>(&ost[lane * SP + DH]);
            const float m = *reinterpret_cast<const float*>(&ost[lane * SP + DH + 2]);
            a.lse[((int64_t)ib * S + pos) * a.H + (h < a.k ? ig * a.k + h : a.G * a.k)] = m + __builtin_amdgcn_logf(l);
        }
    }
}

// Combines the key-range chunks of one split item: per query column, M = max_i m_i,
// l = sum_i l_i 2^(m_i - M), O = sum_i O_i 2^(m_i - M) / l -- the online-softmax merge of partial
// results over disjoint key ranges -- then one rounding to bf16, and the row log-sum-exp
// M + log2(l) for the backward.  Four work groups per item, 64
// columns each; every thread keeps all its 16-byte loads of a chunk in flight.
template <int DH>
__global__ void __launch_bounds__(256) attn_merge_kernel(const int32_t* __restrict__ merges,
                                                         const float* __restrict__ part_o,
                                                         const float* __restrict__ part_ml, bf16_t* __restrict__ O,
                                                         float* __restrict__ lse, int64_t S, int G, int H, int k) {
    constexpr int CPB = kCols / 4;          // columns per work group
    constexpr int NV = CPB * DH / 4 / 256;  // 16-byte vectors per thread per chunk
    static_assert(CPB * DH % 1024 == 0, "whole vectors per thread");
    __shared__ float coef[GQE_ATTN_MAX_CHUNKS][CPB];
    typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
    const_i32_ptr mg = (const_i32_ptr)(merges + 8 * (int64_t)(blockIdx.x >> 2));
    const int b = mg[0], g = mg[1], nh = mg[2], p0 = mg[3], np = mg[4], slot0 = mg[5], nc = mg[6];
    const int c0 = (blockIdx.x & 3) * CPB;
    if (threadIdx.x < CPB) {
        const int c = c0 + threadIdx.x;
        float M = -INFINITY;
        for (int i = 0; i < nc; ++i) M = fmaxf(M, part_ml[((int64_t)(slot0 + i) * kCols + c) * 2]);
        float l = 0.f;
        for (int i = 0; i < nc; ++i) {
            const float* ml = part_ml + ((int64_t)(slot0 + i) * kCols + c) * 2;
            const float e = ml[0] == -INFINITY ? 0.f : exp2f(ml[0] - M);
            coef[i][threadIdx.x] = e;
            l += ml[1] * e;
        }
        const float inv = l > 0.f ? 1.0f / l : 0.f;  // l > 0 for every column that is stored
        for (int i = 0; i < nc; ++i) coef[i][threadIdx.x] *= inv;
        const int p = c / nh, h = c - p * nh;
        const int64_t pos = p0 + p;
        if (p < np && pos < S) lse[((int64_t)b * S + pos) * H + (h < k ? g * k + h : G * k)] = M + __builtin_amdgcn_logf(l);
    }
    __syncthreads();
    f32x4_t acc[NV];
    int cc[NV], n[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        const int e = 4 * (threadIdx.x + 256 * u);  // element of the [CPB][DH] slice
        cc[u] = e / DH;
        n[u] = e - cc[u] * DH;
        acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const float* base = part_o + ((int64_t)slot0 * kCols + c0) * DH;
    for (int i = 0; i < nc; ++i) {
        f32x4_t v[NV];
#pragma unroll
        for (int u = 0; u < NV; ++u)
            v[u] = *reinterpret_cast<const f32x4_t*>(base + (int64_t)i * kCols * DH + cc[u] * DH + n[u]);
#pragma unroll
        for (int u = 0; u < NV; ++u) acc[u] += coef[i][cc[u]] * v[u];
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
        const int c = c0 + cc[u];
        const int p = c / nh, h = c - p * nh;
        const int64_t pos = p0 + p;
        if (p >= np || pos >= S) continue;
        const int vh = h < k ? g * k + h : G * k;
        const u32x2_t pk = {pack_bf16x2(acc[u][0], acc[u][1]), pack_bf16x2(acc[u][2], acc[u][3])};
        *reinterpret_cast<u32x2_t*>(O + (((int64_t)b * S + pos) * H + vh) * DH + n[u]) = pk;
    }
}

}  // namespace

hipError_t launch_attn_mfma(const GqeDims& D, const WorkPlan& P, char* ws, hipStream_t st, KernelMarks* km, bool prep) {
    AttnArgs a{};
    a.Q = (const bf16_t*)(ws + P.q);
    a.K = (const bf16_t*)(ws + P.kk);
    a.Vt = (const bf16_t*)(ws + P.vt);
    a.knt = (const float*)(ws + P.knt);
    a.jobs = (const int32_t*)(ws + P.sched_jobs);
    a.O = (bf16_t*)(ws + P.o);
    a.part_o = (float*)(ws + P.part_o);
    a.part_ml = (float*)(ws + P.part_ml);
    a.lse = (float*)(ws + P.lse);
    a.S = P.S;
    a.S_pad = P.S_pad;
    a.G = D.G;
    a.H = D.H;
    a.k = D.k;
    if (P.ac.njobs <= 0) return hipErrorInvalidValue;
    if (prep) {
        const int64_t BG = P.B * D.G;
        const int64_t work = BG * (P.S_pad / 64) + BG * D.dh * (P.S_pad - P.S);
        const unsigned pg = (unsigned)std::min<int64_t>(ceil_div(work, 256), 1024);
        if (km) km->begin(KT_ATTN_PREP);
        attn_prep_kernel<<<pg, 256, 0, st>>>((const float*)(ws + P.kn), (float*)(ws + P.knt), (bf16_t*)(ws + P.vt),
                                             BG, P.S, P.S_pad, D.dh);
        if (km) km->mark(KT_ATTN_PREP);
    }
    {
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (km) km->begin(KT_ATTN);
    const unsigned grid = (unsigned)P.ac.njobs;
    switch (D.dh) {
        case 32: attn_fwd_kernel<32><<<grid, 256, 0, st>>>(a); break;
        case 48: attn_fwd_kernel<48><<<grid, 256, 0, st>>>(a); break;
        case 64: attn_fwd_kernel<64><<<grid, 256, 0, st>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    if (km) km->mark(KT_ATTN);
    if (P.ac.nmerges > 0) {
        {
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        if (km) km->begin(KT_ATTN_MERGE);
        const unsigned mgrid = (unsigned)P.ac.nmerges * 4;
        const int32_t* mj = (const int32_t*)(ws + P.sched_merges);
        switch (D.dh) {
            case 32: attn_merge_kernel<32><<<mgrid, 256, 0, st>>>(mj, a.part_o, a.part_ml, a.O, a.lse, P.S, D.G, D.H, D.k); break;
            case 48: attn_merge_kernel<48><<<mgrid, 256, 0, st>>>(mj, a.part_o, a.part_ml, a.O, a.lse, P.S, D.G, D.H, D.k); break;
            case 64: attn_merge_kernel<64><<<mgrid, 256, 0, st>>>(mj, a.part_o, a.part_ml, a.O, a.lse, P.S, D.G, D.H, D.k); break;
            default: return hipErrorInvalidValue;
        }
        if (km) km->mark(KT_ATTN_MERGE);
    }
    return hipGetLastError();
}
