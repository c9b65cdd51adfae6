// Device helpers shared by the libptpc kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ptpc {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));

// Raw buffer descriptor over [base, base + bytes): loads at offsets past
// `bytes` return zero instead of touching memory.
constexpr int kBufferDword3 = 0x00020000;   // raw buffer, 32-bit data format
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kBufferDword3);
}
constexpr int kCacheNonTemporal = 2;        // buffer-load cache policy: nt

// bf16 bit patterns packed two to a 32-bit word: low half is the element at
// the lower address.
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// |bf16| ordering equals unsigned ordering of the bits with the sign cleared
// (no NaN/Inf inputs), so the amax of a row is an integer max on 15-bit
// magnitudes, two lanes per 32-bit word.
__device__ __forceinline__ us2 abs_bits2(uint32_t w) {
    uint32_t a = w & 0x7FFF7FFFu;
    return __builtin_bit_cast(us2, a);
}
__device__ __forceinline__ us2 max2(us2 a, us2 b) { return __builtin_elementwise_max(a, b); }
__device__ __forceinline__ uint32_t hmax(us2 a) { return a.x > a.y ? a.x : a.y; }

// Scale of a vector whose largest magnitude is amax (fp32): amax / 448,
// IEEE division; an all-zero vector gets 1.
__device__ __forceinline__ float scale_from_amax(float amax) {
    return amax == 0.0f ? 1.0f : amax / 448.0f;
}

// Division x / d correctly rounded, for many x and one d.  r = RN(1/d) is
// computed once (IEEE division); per element q0 = RN(x*r) is within about an
// ulp of x/d, the negated residual q0*d - x is exact in one fma, and the
// corrected quotient RN(q0 - nres*r) is RN(x/d) (Markstein's correction step
// with a correctly rounded reciprocal).  Writing the residual negated keeps
// the sign of a zero numerator: -0 / d gives -0, as IEEE division does.
// Divisors below 2^-60 are handled by scaling numerator and divisor by 2^96
// (exact for every value such a row can hold), so 1/d stays finite and the
// residual stays representable.  Quotients that underflow are far below
// 2^-10 and encode to a signed zero whatever their last bits.
// The identity RN-code(divide(x, d)) == RN-code(x / d) holds for every pair
// of bf16 values |x| <= amax with d = amax / 448; the GPU tests check this
// exhaustively through the quantization kernel.
struct Divisor {
    float d;    // divisor (pre-scaled)
    float r;    // RN(1/d)
    float pre;  // 1 or 2^96, applied to the numerator
};

__device__ __forceinline__ Divisor make_divisor(float d) {
    Divisor v;
    v.pre = (d < 0x1p-60f) ? 0x1p96f : 1.0f;
    v.d = d * v.pre;
    v.r = 1.0f / v.d;
    return v;
}

__device__ __forceinline__ float divide(float x, const Divisor& v) {
    float xs = x * v.pre;
    float q0 = xs * v.r;
    float nres = __builtin_fmaf(q0, v.d, -xs);
    return __builtin_fmaf(nres, -v.r, q0);
}

// Two fp32 values -> two OCP E4M3 codes (gfx950 v_cvt_pk_fp8_f32: round to
// nearest even under the default rounding mode).  The quotients fed here are
// at most 448 * (1 + 2^-23) in magnitude, which rounds to 448.  word_hi
// selects which 16-bit half of `old` receives the pair.
template <bool WORD_HI>
__device__ __forceinline__ uint32_t cvt_e4m3x2(float a, float b, uint32_t old) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, WORD_HI);
}

// Clamp a quotient to the largest finite E4M3 magnitude.  A scale derived
// from the data's own amax keeps every quotient within 448 (up to rounding,
// which the conversion rounds back to 448); a scale given ahead of time can
// leave quotients far beyond it, which the conversion alone does not
// saturate.  Quotients within +-448 pass unchanged.
__device__ __forceinline__ float sat448(float q) {
    return __builtin_amdgcn_fmed3f(q, -448.0f, 448.0f);
}

// Eight bf16 (one 16-byte vector) divided by one divisor -> eight E4M3 codes
// (SAT: clamp the quotients first, for given scales).
template <bool SAT = false>
__device__ __forceinline__ uint2 quantize8(uint4 v, const Divisor& dv) {
    auto q = [&](float f) { return SAT ? sat448(divide(f, dv)) : divide(f, dv); };
    uint32_t lo = 0, hi = 0;
    lo = cvt_e4m3x2<false>(q(bf16lo_to_f32(v.x)), q(bf16hi_to_f32(v.x)), lo);
    lo = cvt_e4m3x2<true>(q(bf16lo_to_f32(v.y)), q(bf16hi_to_f32(v.y)), lo);
    hi = cvt_e4m3x2<false>(q(bf16lo_to_f32(v.z)), q(bf16hi_to_f32(v.z)), hi);
    hi = cvt_e4m3x2<true>(q(bf16lo_to_f32(v.w)), q(bf16hi_to_f32(v.w)), hi);
    return make_uint2(lo, hi);
}

// Two fp32 values -> two bf16 bit patterns in one word (low half from lo),
// rounded to nearest even.  gfx950 converts the pair in one instruction
// (v_cvt_pk_bf16_f32); checked on the GPU against integer round-to-nearest-even
// for every fp32 bit pattern in both halves: identical, subnormals kept,
// NaN stays NaN.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Max over the 64 lanes of a wavefront.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, m, 64);
        v = v > o ? v : o;
    }
    return v;
}

// Max over groups of G consecutive lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, m, 64);
        v = v > o ? v : o;
    }
    return v;
}

}  // namespace ptpc
