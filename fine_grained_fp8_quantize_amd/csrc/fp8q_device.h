// fp8q_device.h -- device helpers shared by the gfx950 kernels of libfp8q.
//
// Internal to the library (not part of the C ABI). Everything here is written
// for CDNA4 (gfx950): 64-lane wavefronts, DPP row operations, the hardware
// FP8 conversion v_cvt_pk_fp8_f32 and the bf16 conversion v_cvt_pk_bf16_f32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

// Largest finite E4M3FN value; each group's scale maps its amax onto it.
constexpr float kE4M3Max = 448.0f;
// Below this scale the reciprocal path can lose exactness in its residual
// (see group_scale); such groups take IEEE division element by element.
constexpr float kSmallScale = 0x1p-60f;

// ------------------------------------------------------------- bf16 <-> f32

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two fp32 -> packed bf16x2, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v;
    v.x = (__bf16)lo;
    v.y = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// 16-byte streaming load (read once: non-temporal hint).
__device__ __forceinline__ uint4 load_nt16(const void* p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ------------------------------------------------------------ amax helpers

// Packed unsigned 16-bit max of two bf16x2 magnitude words (v_pk_max_u16).
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    u16x2 x = __builtin_bit_cast(u16x2, a), y = __builtin_bit_cast(u16x2, b);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}

__device__ __forceinline__ uint32_t umax32(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Max over each DPP row of 16 lanes; every lane of the row gets the result.
// quad_perm [1,0,3,2] and [2,3,0,1] reduce each quad, row_half_mirror joins
// the two quads of each half-row, row_mirror joins the two half-rows.
// Max over each quad of lanes (DPP quad permutations).
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
    v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    return v;
}

__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
    v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
    v = umax32(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
    return v;
}

// Max over the whole 64-lane wavefront (every lane gets the result).
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
    v = row16_max(v);
    v = umax32(v, (uint32_t)__shfl_xor((int)v, 16));
    v = umax32(v, (uint32_t)__shfl_xor((int)v, 32));
    return v;
}

// ------------------------------------------------------------ group scale

// The per-group scale and its correctly rounded reciprocal.
//   s = fl32(amax / 448) (IEEE division), y = fl32(1 / s).
// For s >= 2^-60 the quotient fl32(x / s) of every bf16 |x| <= amax is
// reproduced by q0 = fl32(x*y), r = x - q0*s (exact by FMA), q = fl32(q0 + r*y)
// wherever it can reach a nonzero E4M3 code (quotients >= 2^-12; checked
// exhaustively over all bf16 pairs). Smaller scales, and s == 0 (all-zero
// group), take the division path.
struct GroupScale {
    float s;
    float y;
    bool slow;
};

__device__ __forceinline__ GroupScale group_scale_f32(float amax) {
    GroupScale g;
    g.s = amax / kE4M3Max;
    g.slow = !(g.s >= kSmallScale);
    g.y = g.slow ? 0.0f : 1.0f / g.s;
    return g;
}

__device__ __forceinline__ GroupScale group_scale(uint32_t amax_bf16_bits) {
    return group_scale_f32(__uint_as_float(amax_bf16_bits << 16));
}

// fl32(|x| / s) for a magnitude ax >= 0 (the caller clamps to 448). For
// binary32 numerators in general (not only bf16 ones) this is Markstein's
// correction: with y the correctly rounded 1/s and q0 within one ulp of
// ax/s, the residual r is exact and fl32(q0 + r*y) is the correctly rounded
// quotient, barring underflow, which s >= 2^-60 rules out where a code can
// be nonzero.
__device__ __forceinline__ float quot_fast(float ax, const GroupScale& g) {
    float q0 = ax * g.y;
    float r = __builtin_fmaf(-q0, g.s, ax);
    return __builtin_fmaf(r, g.y, q0);
}
__device__ __forceinline__ float quot_slow(float ax, const GroupScale& g) {
    return g.s == 0.0f ? 0.0f : ax / g.s;
}

// Four non-negative quotients -> four E4M3 magnitude codes in one dword
// (element i in byte i), with the sign bits (bit 7 of each byte of
// `signs`) inserted afterwards: the code's sign is always the sign of x.
__device__ __forceinline__ uint32_t pack_e4m3x4(float q0, float q1, float q2, float q3,
                                                uint32_t signs) {
    q0 = __builtin_fminf(q0, kE4M3Max);
    q1 = __builtin_fminf(q1, kE4M3Max);
    q2 = __builtin_fminf(q2, kE4M3Max);
    q3 = __builtin_fminf(q3, kE4M3Max);
    uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
    w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, (int)w, true);
    return (w & 0x7F7F7F7Fu) | (signs & 0x80808080u);
}

// Sign bytes of four bf16 values held as two bf16x2 words: byte i of the
// result carries the high byte (sign + exponent MSBs) of element i.
__device__ __forceinline__ uint32_t bf16x4_sign_bytes(uint32_t w01, uint32_t w23) {
    return __builtin_amdgcn_perm(w23, w01, 0x07050301u);
}

// Byte `byte` (0..3) of each of four words, gathered into bytes 0..3.
__device__ __forceinline__ uint32_t gather_byte4(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                                 uint32_t byte) {
    uint32_t sel = byte | ((4u + byte) << 8) | 0x0C0C0000u;  // selector 0x0C yields 0x00
    uint32_t ab = __builtin_amdgcn_perm(b, a, sel);
    uint32_t cd = __builtin_amdgcn_perm(d, c, sel);
    return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// ------------------------------------------------------------ LDS / waits

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

}  // namespace fp8q
