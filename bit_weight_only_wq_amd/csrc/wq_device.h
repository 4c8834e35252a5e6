// Device helpers for the gfx950 kernels: packed-half types, exact rounding
// primitives for the quantizer, and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ h2_t as_h2(uint32_t u) { return __builtin_bit_cast(h2_t, u); }
__device__ __forceinline__ uint32_t as_u32(h2_t h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ uint16_t float_to_half_bits_rne(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);  // v_cvt_f16_f32, round to nearest even
}

// ---------------------------------------------------------------------------
// Exact rounding for the quantizer.
//
// Every operand below holds an fp16 value, so all of them are short multiples
// of 2^-24.  The decisions the codec takes (round(x/s), round(-min/s), the fp16
// rounding of (max-min)/M) must be the exact-rational ones; these helpers reach
// them with hardware arithmetic plus an exact correction step.
// ---------------------------------------------------------------------------

// round-half-even(x / s) for fp16-valued x and s > 0.  The estimate x*rcp is
// clamped to [lo, hi] (callers choose the window outside of which the result
// no longer matters) and rounded; the fused remainder x - k*s is exact (it fits
// in 24 bits whenever |x/s - k| < 2), so comparing 2*(x - k*s) with +-s decides
// the true nearest integer and the tie, which goes to the even neighbour.
__device__ __forceinline__ float rne_div_exact(float x, float s, float rcp, float lo, float hi) {
    float t = __builtin_fminf(__builtin_fmaxf(x * rcp, lo), hi);
    float k = __builtin_rintf(t);
    float d2 = 2.0f * __builtin_fmaf(-k, s, x);
    bool odd = ((int)k & 1) != 0;
    float up = (d2 > s || (d2 == s && odd)) ? 1.0f : 0.0f;
    float dn = (d2 < -s || (d2 == -s && odd)) ? 1.0f : 0.0f;
    return k + up - dn;
}

// fp16 bits of round-half-even((mx - mn) / M) for fp16-valued mn <= mx.
// The range is exact in double, the double quotient sits on the same side of
// every fp16 rounding boundary as the exact one (they are at least 2^-49
// apart in relative terms), and rounding to float with round-to-odd before the
// hardware fp32 -> fp16 conversion avoids a double-rounding error.
// A scale that rounds to zero becomes 1.0 (0x3C00).
__device__ __forceinline__ uint16_t scale_bits_exact(float mn, float mx, int M) {
    double v = ((double)mx - (double)mn) / (double)M;
    float f = (float)v;
    double fd = (double)f;
    if (fd != v) {
        uint32_t u = __builtin_bit_cast(uint32_t, f);
        if (fd > v) u -= 1u;  // v > 0 here: step down to the truncated value
        u |= 1u;              // round to odd
        f = __builtin_bit_cast(float, u);
    }
    uint16_t b = float_to_half_bits_rne(f);
    return b == 0 ? (uint16_t)0x3C00 : b;
}

// fp16 bits of the stored zero point for an exact integer k (as float):
// round half to even into fp16, saturating at +-65504, with 0 stored as +0.0.
__device__ __forceinline__ uint16_t zero_bits_from_int(float k) {
    uint16_t b = float_to_half_bits_rne(k);
    if ((b & 0x7FFFu) >= 0x7C00u) b = (uint16_t)((b & 0x8000u) | 0x7BFFu);
    if (k == 0.0f) b = 0;
    return b;
}

// Per-group header of the asymmetric codec from the exact min and max of a
// group with M = 2^b - 1 steps: fp16 scale and zero point, and what the
// encoder needs (reciprocal, zero point as a float, tie-safety threshold).
struct GroupHeader {
    float s, rcp, Z, thr;
    uint16_t sbits, zbits;
};

__device__ __forceinline__ GroupHeader make_header(float mn, float mx, int M) {
    GroupHeader h;
    h.sbits = scale_bits_exact(mn, mx, M);
    h.s = half_bits_to_float(h.sbits);
    h.rcp = __builtin_amdgcn_rcpf(h.s);
    // z = round(-min / s): estimates beyond +-2^17 all saturate the fp16 zero.
    float k = rne_div_exact(-mn, h.s, h.rcp, -131072.0f, 131072.0f);
    h.zbits = zero_bits_from_int(k);
    h.Z = half_bits_to_float(h.zbits);
    // |x*rcp - x/s| <= |x/s| * 2^-22 (rcp within 1 ulp, one rounding of the
    // product).  A fraction |t - rint(t)| at most thr therefore cannot be a tie
    // or on the wrong side of one; thr keeps a 4x margin on that bound.
    const float tmax = __builtin_fmaxf(__builtin_fabsf(mn), __builtin_fabsf(mx)) * h.rcp;
    h.thr = 0.5f - (tmax + 1.0f) * 0x1p-20f;
    return h;
}

// ---------------------------------------------------------------------------
// Wavefront reductions.  DPP moves inside 16-lane rows, then cross-row steps.
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of W lanes (W in {1,2,4,...,64}); every lane of the
// group receives the group's total.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (W >= 2) v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (W >= 4) v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (W >= 8) v += dpp_f<0x141>(v);   // row_half_mirror: pairs quads in 8
    if constexpr (W >= 16) v += dpp_f<0x140>(v);  // row_mirror: pairs halves of a row
    if constexpr (W >= 32) v += __shfl_xor(v, 16, 64);
    if constexpr (W >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// Min / max over aligned groups of W lanes (butterfly; every lane gets the result).
template <int W>
__device__ __forceinline__ void group_minmax(float& mn, float& mx) {
#pragma unroll
    for (int o = 1; o < W; o <<= 1) {
        mn = __builtin_fminf(mn, __shfl_xor(mn, o, 64));
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, o, 64));
    }
}

// A 32-bit constant held in a VGPR.  gfx9 VOP3 instructions take no literal
// operand, so keeping unpack masks in registers lets every unpack step be a
// single v_and_or_b32 (mask from a VGPR, the 0x6400 exponent from an SGPR).
__device__ __forceinline__ uint32_t vgpr_const(uint32_t v) {
    uint32_t r;
    asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
    return r;
}

// 128-bit load that bypasses cache allocation: every code byte is read once.
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

// Unsigned nibble/byte codes to fp16 pairs via the exponent trick: OR-ing a
// code c < 1024 into the mantissa of 1024.0 (0x6400) gives exactly 1024 + c.
// 4-bit: word w holds codes k..k+7 (code i in bits 4i..4i+3).  Pair p (0..3)
//        holds (code p, code p+4).
// 8-bit: word w holds codes k..k+3 (code i in byte i).  Pair p (0..1) holds
//        (code p, code p+2).
__device__ __forceinline__ uint32_t nib_pair(uint32_t w, int p) {
    return ((w >> (4 * p)) & 0x000F000Fu) | 0x64006400u;
}
__device__ __forceinline__ uint32_t byte_pair(uint32_t w, int p) {
    return ((w >> (8 * p)) & 0x00FF00FFu) | 0x64006400u;
}

}  // namespace wq
