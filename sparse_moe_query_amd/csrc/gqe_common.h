// Internal helpers shared by the HIP kernels of libgqe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- element type traits
// Storage is either float32 or bfloat16 (raw 16-bit patterns); arithmetic is float32.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) {
    return __uint_as_float(((uint32_t)v.bits) << 16);
}
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// float32 -> bfloat16, round to nearest even (finite inputs; NaN stays NaN).
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return bf16_t{(uint16_t)((u >> 16) | 0x40)};
    u += 0x7fffu + ((u >> 16) & 1u);
    return bf16_t{(uint16_t)(u >> 16)};
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two float32 -> two bfloat16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Position, inside its 16-key chunk, at which key offset o (0..15) of V^T is stored: bits 2 and 3
// of the offset swapped, i.e. keys 0-3, 8-11, 4-7, 12-15.  A 32x32 matrix-core score tile leaves
// each lane with keys {0-3, 8-11} (lanes 0-31) or {4-7, 12-15} (lanes 32-63) of every 16-key chunk;
// with this order one 16-byte read of V^T gives each lane exactly those eight keys, so the
// probabilities feed the P.V product straight from the score registers (see k_attn).
__host__ __device__ __forceinline__ int vt_slot(int o) {
    return (o & ~12) | ((o & 4) << 1) | ((o & 8) >> 1);
}
__host__ __device__ __forceinline__ int64_t vt_pos(int64_t s) {
    return (s & ~(int64_t)15) | vt_slot((int)(s & 15));
}

__host__ __device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ __forceinline__ int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

#define GQE_KV_TILE 64  // keys per attention tile; K and V^T are padded to a multiple of this

// Rotary position embedding of one pair (a, b) of a query or key head vector at position pos:
// rotation by the angle 2 pi * pos * rev, where rev = base^(-2i/d_h) / (2 pi) is the pair's
// frequency in cycles per position (float64 table written by gqe_pack_weights).  The cycle count
// is reduced to [-1/2, 1/2] in float64, so the float32 hardware sine and cosine (argument in
// cycles) see a small argument at any position.
__device__ __forceinline__ void rope_pair(float& a, float& b, int64_t pos, double rev) {
    double f = (double)pos * rev;
    f -= __builtin_rint(f);
    const float ff = (float)f;
    const float sn = __builtin_amdgcn_sinf(ff), cs = __builtin_amdgcn_cosf(ff);
    const float a0 = a, b0 = b;
    a = a0 * cs - b0 * sn;
    b = a0 * sn + b0 * cs;
}
// The two pairs (v0, v1), (v2, v3) of four consecutive head dims.
__device__ __forceinline__ void rope_quad(f32x4_t& v, int64_t pos, double rev0, double rev1) {
    float a = v[0], b = v[1], c = v[2], d = v[3];
    rope_pair(a, b, pos, rev0);
    rope_pair(c, d, pos, rev1);
    v = f32x4_t{a, b, c, d};
}

// ---------------------------------------------------------------- direct global -> LDS loads
// One wave-wide global_load_lds_dwordx4: lane i's 16 bytes from gsrc land in LDS at
// ldst + 16 i (ldst wave-uniform).  Written as inline assembly so that the compiler does not
// order every later LDS read behind it; the kernels wait for these loads themselves (vmcnt)
// before the barrier that publishes a stage.  No register of the asm is an output.  The LDS
// destination comes from M0, which needs one wait state between its SALU write and the load.
__device__ __forceinline__ void dma16(const void* gsrc, const void* ldst) {
    const uint32_t m0v = (uint32_t)(uintptr_t)ldst;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_nop 4"
                 :
                 : "s"(m0v), "v"(gsrc)
                 : "memory", "m0");
}

// The same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane byte offset.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, const void* ldst) {
    const uint32_t m0v = (uint32_t)(uintptr_t)ldst;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_nop 4"
                 :
                 : "s"(m0v), "v"(voff), "s"(gbase)
                 : "memory", "m0");
}

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector-memory operations are
// outstanding and leaves the other counters unconstrained.
__host__ __device__ constexpr int vmcnt_wait(int n) {
    return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8);
}
