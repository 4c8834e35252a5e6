// In-register fp16 dequantization for the matrix-core kernels' weight operand
// ("Quantization": the kernel rebuilds an approximate float from the integer
// and the group's endpoints as it reads the codes).
//
// A 32-bit word of 4-bit codes holds k0..k7 (k0 in bits 0-3, the page's
// even-low-nibble byte order); it unpacks as exact fp16 pairs
//   (w & 0x000F000F) | 0x60006000 = (512 + q0/2, 512 + q4/2)
//   (w & 0x00F000F0) | 0x50005000 = ( 32 + q1/2,  32 + q5/2)
// and the same of w >> 8 for (q2, q6), (q3, q7); minus (512 + z/2) or
// (32 + z/2), times s, rounded once, that is (q - z) * s / 2.  The factor 1/2
// keeps every operand finite for any fp16 weights and is undone on the fp32
// result.  The k order of an operand is therefore (0,4,1,5,2,6,3,7) within
// each 8 k (8-bit codes: (0,2,1,3) within each 4 k), and the X operand is
// permuted to match.
#pragma once

#include "wq_device.h"

namespace wq {
namespace dq {

// Reorder one 8-value X vector into the order in which the codes unpack:
// 4-bit (q0,q4,q1,q5,q2,q6,q3,q7); 8-bit (q0,q2,q1,q3,q4,q6,q5,q7).
// v_perm_b32 selector bytes 0-3 take src1 bytes 0-3, 4-7 take src0 bytes 0-3.
template <int BITS>
__device__ __forceinline__ uint4 permute8(uint4 in) {
    uint4 o;
    if constexpr (BITS == 4) {
        o.x = __builtin_amdgcn_perm(in.z, in.x, 0x05040100u);  // x0 | x4 << 16
        o.y = __builtin_amdgcn_perm(in.z, in.x, 0x07060302u);  // x1 | x5 << 16
        o.z = __builtin_amdgcn_perm(in.w, in.y, 0x05040100u);  // x2 | x6 << 16
        o.w = __builtin_amdgcn_perm(in.w, in.y, 0x07060302u);  // x3 | x7 << 16
    } else {
        o.x = __builtin_amdgcn_perm(in.y, in.x, 0x05040100u);  // x0 | x2 << 16
        o.y = __builtin_amdgcn_perm(in.y, in.x, 0x07060302u);  // x1 | x3 << 16
        o.z = __builtin_amdgcn_perm(in.w, in.z, 0x05040100u);  // x4 | x6 << 16
        o.w = __builtin_amdgcn_perm(in.w, in.z, 0x07060302u);  // x5 | x7 << 16
    }
    return o;
}

struct DqConsts {
    uint32_t m_lo, m_hi, g_lo, g_hi;  // nibble/byte masks and exponent patterns
};

// B operand of k-step j of one lane's chunk: (q - z) * s / 2 in fp16, with
// nz = (512 + z/2, 32 + z/2) and ss = (s, s).
template <int BITS>
__device__ __forceinline__ h8_t dequant(const uint4& cw, int j, const DqConsts& c, h2_t nz, h2_t ss) {
    const h2_t na = {nz.x, nz.x};
    h2_t p0, p1, p2, p3;
    if constexpr (BITS == 4) {
        const h2_t nb = {nz.y, nz.y};
        const uint32_t w = j == 0 ? cw.x : j == 1 ? cw.y : j == 2 ? cw.z : cw.w;
        const uint32_t w8 = w >> 8;
        p0 = (as_h2((w & c.m_lo) | c.g_lo) - na) * ss;
        p1 = (as_h2((w & c.m_hi) | c.g_hi) - nb) * ss;
        p2 = (as_h2((w8 & c.m_lo) | c.g_lo) - na) * ss;
        p3 = (as_h2((w8 & c.m_hi) | c.g_hi) - nb) * ss;
    } else {
        const uint32_t w0 = j == 0 ? cw.x : cw.z;
        const uint32_t w1 = j == 0 ? cw.y : cw.w;
        p0 = (as_h2((w0 & c.m_lo) | c.g_lo) - na) * ss;
        p1 = (as_h2(((w0 >> 8) & c.m_lo) | c.g_lo) - na) * ss;
        p2 = (as_h2((w1 & c.m_lo) | c.g_lo) - na) * ss;
        p3 = (as_h2(((w1 >> 8) & c.m_lo) | c.g_lo) - na) * ss;
    }
    const uint4 a = {as_u32(p0), as_u32(p1), as_u32(p2), as_u32(p3)};
    return __builtin_bit_cast(h8_t, a);
}

}  // namespace dq
}  // namespace wq
