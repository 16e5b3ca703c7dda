// Device-side numeric helpers shared by the kernels of the W4A4 layer (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mg {

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Raw buffer resource over `bytes` bytes from p (clamped to 2^32 - 1): loads
// past the end return 0 and stores past it are dropped by the hardware range
// check.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint64_t bytes) {
    const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}

// Round-to-nearest-even f32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// E8M0 block-scale code from the bit pattern of a non-negative f32 amax:
// floor(log2 amax) - 2 + 127 = biased exponent - 2, clamped at 0.
__device__ __forceinline__ uint32_t e8m0_from_amax_bits(uint32_t amax_bits) {
    int e = (int)(amax_bits >> 23);
    return (uint32_t)(e > 2 ? e - 2 : 0);
}

// IEEE f32 quotient x / s from rcp = RN(1/s) with Markstein's FMA-based
// correction (P. Markstein, IBM J. Res. Dev. 1990; Muller et al., Handbook of
// Floating-Point Arithmetic, division with a fused multiply-add): q0 = x*rcp,
// t = q0*s - x (exact), q = q0 - t*rcp.  The result is the correctly rounded
// quotient when nothing overflows and the remainder cannot underflow; the
// callers check their conditions (div_fast_ok_s, and bounds on the quotients)
// and otherwise divide with __fdiv_rn.  The remainder is formed as q0*s - x
// and subtracted, so a zero x keeps its sign (-0 / s = -0) without a separate
// sign fix-up.
__device__ __forceinline__ float div_fast(float x, float s, float rcp) {
    const float q0 = x * rcp;
    const float t = __builtin_fmaf(q0, s, -x);
    return __builtin_fmaf(-t, rcp, q0);
}

// Divisor range of the fast division: with 2^-20 <= s <= 2^20, div_fast is
// the IEEE quotient for every bf16 x with |x| >= 2^-100 and |x * rcp| < 2^126
// (the remainder is then representable and nothing overflows).
__device__ __forceinline__ bool div_fast_ok_s(float s) { return s >= 0x1p-20f && s <= 0x1p20f; }

// GELU (tanh form) in f32 of one value: 0.5 y (1 + tanh u) with
// u = sqrt(2/pi) (y + 0.044715 y^3), evaluated as the equal
// y / (1 + e^(-2u)) = y * sigmoid(2u): one hardware exp2 (v_exp_f32) of
// t = -2u log2(e) = y (C2 y^2 + C1) and one hardware reciprocal (v_rcp_f32),
// with no cancellation in 1 + tanh u for negative y.
__device__ __forceinline__ float gelu_f32(float y) {
    constexpr float C1 = -2.302208198144325f;    // -2 sqrt(2/pi) log2(e)
    constexpr float C2 = -0.1029432395800235f;   // 0.044715 C1
    const float t = y * __builtin_fmaf(C2, y * y, C1);
    return y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}

typedef __bf16 mg_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float mg_f32x2_t __attribute__((ext_vector_type(2)));

// GELU of the two bf16 values packed in w (first in the low half), each
// rounded to bf16 (nearest even, v_cvt_pk_bf16_f32).  The result is a
// faithful bf16 rounding of the exact GELU for every finite bf16 input where
// that is at least 2^-24 in magnitude (smaller results come out as at most
// 2^-24; very negative y give -0).  The GELU kernel and the fused GELU +
// quantize path both use this, so their outputs are the same bits.
__device__ __forceinline__ uint32_t gelu_bf16x2(uint32_t w) {
    const mg_f32x2_t v = {gelu_f32(__uint_as_float(w << 16)), gelu_f32(__uint_as_float(w & 0xFFFF0000u))};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, mg_bf16x2_t));
}

// f32 bit patterns of 2^126, 2^-74 and 2^-78: the bounds of the activation
// quantizer's checks on its fast division (see the quantizer)
constexpr uint32_t kF32Pow126 = 0x7E800000u, kF32PowM74 = 0x1A800000u, kF32PowM78 = 0x18800000u;
// integer predicates of __builtin_amdgcn_uicmp (a wave mask of the lanes where
// the unsigned comparison holds)
constexpr int kCmpNE = 33, kCmpUGE = 35, kCmpULT = 36;

// Max over the 4 lanes of a quad (one 32-block: quad_perm [1,0,3,2] then
// [2,3,0,1]) of the bit patterns of non-negative f32 values, whose unsigned
// integer order is their numeric order.
__device__ __forceinline__ uint32_t quad_max_bits(uint32_t v) {
    v = __builtin_elementwise_max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));
    v = __builtin_elementwise_max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));
    return v;
}

// E8M0 code c -> the scale operand of the hardware converter, which takes
// the E8M0 code from the exponent field of its f32 scale: 2^(c - 127) for
// c >= 1, and for c = 0 a value whose exponent field is 0 (the converter then
// scales by 2^-127; checked bit for bit against the oracle on blocks with
// that code).
__device__ __forceinline__ float e8m0_to_f32(uint32_t c) {
    return __uint_as_float(c ? (c << 23) : 0x00200000u);
}

// Hardware E2M1 encode of two f32 values divided by an f32 power-of-two scale
// (v_cvt_scalef32_pk_fp4_f32: nearest, ties to even, saturating, sign kept),
// written into byte `sel` of `word` (first value in the low nibble); the
// other bytes of `word` are kept.  The quantizer's codes are checked bit for
// bit against the oracle's threshold encoder on every finite bf16 value under
// scale-setting blocks, at s = 1 and at the workloads' smoothing scales.
#define MG_CVT_FP4X2(word, a, b, scale, sel) \
    (word) = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((word), (a), (b), (scale), (sel))

}  // namespace mg
