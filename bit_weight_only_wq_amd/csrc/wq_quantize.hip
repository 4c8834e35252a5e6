// Quantize/pack kernels (gfx950): fp16 W[N, K] -> codes, fp16 scales, fp16 zeros.
//
// Codec of "What actually happens when you quantize a KV cache", §3 steps 3-5
// and §4, per group of G consecutive k of a row:
//   min/max -> s = (max-min)/(2^b-1) stored fp16 -> z = round(-min/s) stored
//   fp16 -> q = clamp(round(x/s) + z, 0, 2^b-1) -> packed little-endian per row
//   (b = 4: even k in the low nibble).
// Rounding is half-to-even and every decision is the exact-rational one (see
// wq_device.h).  Degenerate scale -> 1.0; zero point saturates at +-65504.
//
// Float-offset scheme ("Quantization & inference optimisation",
// "Quantization"): the scale as above, the group minimum stored in place of
// the zero point, codes round((x - min)/s) clamped to [0, 2^b - 1].
//
// Symmetric scheme ("Quantization & inference optimisation", "Quantize a
// matrix by hand" and "Per-channel, and what it buys"): s = A/(2^(b-1)-1) with
// A = max|x| of the group (or of the whole matrix), the signed integer
// clamp(round(x/s), -2^(b-1), 2^(b-1)-1) stored offset by 2^(b-1), which is
// the stored zero point.  That is the asymmetric encoder with z = 2^(b-1), so
// both schemes share the encode and pack code and differ only in the header.
// One scale per tensor takes A from two small reduction launches first.
//
// Layout: W, codes, scales and zeros are all flat row-major, and K % G == 0,
// so group gi covers W[gi*G .. gi*G + G) and writes scales[gi], zeros[gi]
// and codes bytes [gi*G*b/8, (gi+1)*G*b/8).  Each lane handles 8 consecutive
// values (one 16-byte load, one 4- or 8-byte store), so loads and stores of a
// wave are contiguous.
#include "wq_device.h"
#include "wq_launch.h"
#include "wq_nf4_levels.h"

namespace wq {

namespace {

__device__ __forceinline__ void load8(const uint16_t* p, float* x, uint4& raw) {
    raw = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = half_bits_to_float((uint16_t)(w[i] & 0xFFFFu));
        x[2 * i + 1] = half_bits_to_float((uint16_t)(w[i] >> 16));
    }
}

// Min and max of 8 fp16 values on packed halves (exact comparisons).
__device__ __forceinline__ void minmax8(const uint4& raw, float& mn, float& mx) {
    const h2_t a = as_h2(raw.x), b = as_h2(raw.y), c = as_h2(raw.z), d = as_h2(raw.w);
    const h2_t lo = __builtin_elementwise_min(__builtin_elementwise_min(a, b),
                                              __builtin_elementwise_min(c, d));
    const h2_t hi = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                              __builtin_elementwise_max(c, d));
    mn = __builtin_fminf((float)lo.x, (float)lo.y);
    mx = __builtin_fmaxf((float)hi.x, (float)hi.y);
}

// Symmetric header from the scope's absolute maximum A: s = A / qmax rounded
// once to fp16 (1.0 when that is 0), zero point 2^(b-1) (exact in fp16).
__device__ __forceinline__ GroupHeader make_header_sym(float A, int bits) {
    GroupHeader h;
    const int half = 1 << (bits - 1);
    h.sbits = scale_bits_exact(0.0f, A, half - 1);
    h.s = half_bits_to_float(h.sbits);
    h.rcp = __builtin_amdgcn_rcpf(h.s);
    h.Z = (float)half;
    h.zbits = zero_bits_from_int(h.Z);
    h.thr = 0.5f - (A * h.rcp + 1.0f) * 0x1p-20f;   // as in make_header
    return h;
}

// Header of one group for the scheme: 0 asymmetric, 1 symmetric per group,
// 2 symmetric with the tensor's absolute maximum Aall.
__device__ __forceinline__ GroupHeader header_for(int scheme, float mn, float mx, float Aall,
                                                  int bits) {
    if (scheme == 0) return make_header(mn, mx, (1 << bits) - 1);
    return make_header_sym(scheme == 2 ? Aall : __builtin_fmaxf(-mn, mx), bits);
}

// NF4 (scheme 3, 4-bit codes only; "Gör inference billig", the NF4
// paragraph): scale s = the group's largest |w| (an fp16 input, so exact;
// 1.0 for an all-zero group) and code = the level nearest to w / s, ties to
// the lower code.  The levels are symmetric, so with a = |w| the code is
// 8 + #{j >= 8 : mid_j * s < a} for w > 0 and 7 - #{j >= 8 : mid_j * s <= a}
// otherwise; mid_j * s is exact in fp32 (12 + 11 significant bits), so every
// comparison is exact.
struct Nf4Group {
    float th[7];        // mid_j * s, j = 8..14
    uint16_t sbits;
};

__device__ __forceinline__ Nf4Group nf4_group(float mn, float mx) {
    Nf4Group g;
    float A = __builtin_fmaxf(-mn, mx);
    A = A == 0.0f ? 1.0f : A;
    g.sbits = float_to_half_bits_rne(A);
#pragma unroll
    for (int j = 0; j < 7; ++j) g.th[j] = kNf4Mid[8 + j] * A;
    return g;
}

__device__ __forceinline__ uint32_t nf4_code(float x, const Nf4Group& g) {
    // th <= a is th < nextup(a) (every threshold is a normal float), so both
    // signs take one strict comparison per threshold.
    const float a = __builtin_fabsf(x);
    const bool pos = x > 0.0f;
    const float a2 = pos ? a : __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, a) + 1u);
    int c = 0;
#pragma unroll
    for (int j = 0; j < 7; ++j) c += g.th[j] < a2 ? 1 : 0;
    return (uint32_t)(pos ? 8 + c : 7 - c);
}

// Eight NF4 codes packed as eight nibbles (even position low).
__device__ __forceinline__ uint32_t nf4_encode8(const float* x, const Nf4Group& g) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= nf4_code(x[i], g) << (4 * i);
    return w;
}

// fp16 bits of the tensor's absolute maximum, written by the reduction
// launches (finite fp16 magnitudes order like their bit patterns).
__device__ __forceinline__ float load_amax(int scheme, const uint32_t* amax) {
    return scheme == 2 ? half_bits_to_float((uint16_t)amax[0]) : 0.0f;
}

// Codes of 8 values packed into BITS bytes: the little-endian bit stream
// (code i at bits [i*BITS, i*BITS+BITS)).  4-bit: one word, even position in
// the low nibble; 8-bit: one byte per code; other widths: the low 8*BITS bits
// of a 64-bit value.
template <int BITS>
struct Packed8 {
    typedef uint64_t type;
};
template <>
struct Packed8<4> {
    typedef uint32_t type;
};
template <>
struct Packed8<8> {
    typedef uint2 type;
};

template <int BITS>
__device__ __forceinline__ typename Packed8<BITS>::type pack8(const float* q);

template <int BITS>
__device__ __forceinline__ typename Packed8<BITS>::type encode8(const float* x, const GroupHeader& h) {
    constexpr float M = (float)((1 << BITS) - 1);
    // Fast path: rint of the fp32 quotient estimate, exact unless the estimate
    // falls within the error band around a half-integer.
    float k[8];
    bool near = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float t = x[i] * h.rcp;
        k[i] = __builtin_rintf(t);
        near |= __builtin_fabsf(t - k[i]) > h.thr;
    }
    if (__builtin_amdgcn_ballot_w64(near) != 0) {
        // Exact path (taken when a lane of the wave lies near a half-integer;
        // exact ties x/s = k + 1/2 are common with fp16 x and s).  With
        // kl = floor(t) and t within 2^-20 of x/s, round-half-even(x/s) is kl
        // below kl + 1/2, kl + 1 above it, and the even one of the two on it;
        // the side is the sign of r = x - (kl + 1/2) s, computed exactly by
        // one fma (every operand is a short multiple of 2^-25, so r is zero
        // only when x/s is exactly kl + 1/2).  Outside [-Z-2, M-Z+2] every
        // value clamps to code 0 or M anyway, so t is clamped there first.
        const float lo = -h.Z - 2.0f, hi = M - h.Z + 2.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float t = __builtin_amdgcn_fmed3f(x[i] * h.rcp, lo, hi);
            const float kl = __builtin_floorf(t);
            const float r = __builtin_fmaf(-(kl + 0.5f), h.s, x[i]);
            const float half = kl * 0.5f;
            const bool odd = __builtin_rintf(half) != half;
            const bool inc = (r > 0.0f) | ((r == 0.0f) & odd);   // no short-circuit branches
            k[i] = inc ? kl + 1.0f : kl;
        }
    }
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = __builtin_amdgcn_fmed3f(k[i] + h.Z, 0.0f, M);
    return pack8<BITS>(q);
}

// Float-offset variant (scheme 4; "Quantization & inference optimisation",
// "Quantization"): q = clamp(round((x - mn) / s), 0, 2^b - 1).  In double,
// x - mn is exact (fp16 inputs: at most 41 significant bits), and with
// kl = floor(t) for t ~ (x - mn)/s the remainder (x - mn) - (kl + 1/2) s is
// exact too, so its sign takes the rounding decision, ties to even.  An
// estimate t one off at an exact integer is corrected by the same test.
template <int BITS>
__device__ __forceinline__ typename Packed8<BITS>::type encode8_offset(const float* x, float mn, float s) {
    constexpr float M = (float)((1 << BITS) - 1);
    const double sd = (double)s, rcp = 1.0 / sd, md = (double)mn;
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const double d = (double)x[i] - md;
        const double kl = __builtin_floor(d * rcp);
        const double r = __builtin_fma(-(kl + 0.5), sd, d);
        const bool odd = ((int)kl & 1) != 0;            // 0 <= kl < 2^20
        const double k = (r > 0.0) | ((r == 0.0) & odd) ? kl + 1.0 : kl;
        q[i] = __builtin_amdgcn_fmed3f((float)k, 0.0f, M);
    }
    return pack8<BITS>(q);
}

// Codes q[0..7] (integral floats in [0, 2^b - 1]) packed into BITS bytes.
template <int BITS>
__device__ __forceinline__ typename Packed8<BITS>::type pack8(const float* q) {
    if constexpr (BITS == 4) {
        // Bytes (q0,q2,q4,q6) and (q1,q3,q5,q7); byte j = q[2j] | q[2j+1] << 4.
        uint32_t ev = 0, od = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ev = __builtin_amdgcn_cvt_pk_u8_f32(q[2 * j], j, ev);
            od = __builtin_amdgcn_cvt_pk_u8_f32(q[2 * j + 1], j, od);
        }
        return ev | (od << 4);
    } else if constexpr (BITS == 8) {
        uint2 w = make_uint2(0u, 0u);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            w.x = __builtin_amdgcn_cvt_pk_u8_f32(q[j], j, w.x);
            w.y = __builtin_amdgcn_cvt_pk_u8_f32(q[4 + j], j, w.y);
        }
        return w;
    } else {
        uint64_t v = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) v |= (uint64_t)(uint32_t)q[i] << (i * BITS);
        return v;
    }
}

// Byte j (0 <= j < BITS) of a packed 8-code chunk.
template <int BITS>
__device__ __forceinline__ uint32_t chunk_byte(const typename Packed8<BITS>::type& p, int j) {
    if constexpr (BITS == 4) return (p >> (8 * j)) & 0xFFu;
    else if constexpr (BITS == 8) return ((j < 4 ? p.x : p.y) >> (8 * (j & 3))) & 0xFFu;
    else return (uint32_t)(p >> (8 * j)) & 0xFFu;
}

// Store the packed codes of CPL consecutive 8-value chunks with one vector
// store (4*CPL bytes at 4 bits, 8*CPL bytes at 8 bits).
template <int BITS, int CPL>
__device__ __forceinline__ void store_codes(uint8_t* dst, const typename Packed8<BITS>::type* p) {
    if constexpr (BITS != 4 && BITS != 8) {
        // CPL*BITS bytes: the chunks' bytes in order.  Whole 32-bit words when
        // the lane's share is a multiple of 4 bytes (then also 4-byte
        // aligned), single bytes otherwise.
        constexpr int NB = CPL * BITS;
        if constexpr (NB % 4 == 0) {
#pragma unroll
            for (int w = 0; w < NB / 4; ++w) {
                uint32_t v = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int byte = 4 * w + b;
                    v |= chunk_byte<BITS>(p[byte / BITS], byte % BITS) << (8 * b);
                }
                reinterpret_cast<uint32_t*>(dst)[w] = v;
            }
        } else {
#pragma unroll
            for (int byte = 0; byte < NB; ++byte) dst[byte] = (uint8_t)chunk_byte<BITS>(p[byte / BITS], byte % BITS);
        }
    } else if constexpr (BITS == 4) {
        if constexpr (CPL == 4) *reinterpret_cast<uint4*>(dst) = make_uint4(p[0], p[1], p[2], p[3]);
        else if constexpr (CPL == 2) *reinterpret_cast<uint2*>(dst) = make_uint2(p[0], p[1]);
        else *reinterpret_cast<uint32_t*>(dst) = p[0];
    } else {
        if constexpr (CPL == 4) {
            reinterpret_cast<uint4*>(dst)[0] = make_uint4(p[0].x, p[0].y, p[1].x, p[1].y);
            reinterpret_cast<uint4*>(dst)[1] = make_uint4(p[2].x, p[2].y, p[3].x, p[3].y);
        } else if constexpr (CPL == 2) {
            *reinterpret_cast<uint4*>(dst) = make_uint4(p[0].x, p[0].y, p[1].x, p[1].y);
        } else {
            *reinterpret_cast<uint2*>(dst) = p[0];
        }
    }
}

// Groups of G = 8*CPL*T values: T lanes per group (a power of two <= 64), each
// lane owning CPL consecutive 8-value chunks (lane t of a team holds values
// [8*CPL*t, 8*CPL*(t+1)) of its group).  Lane u of the grid therefore covers
// the flat values [8*CPL*u, 8*CPL*(u+1)), the same for W and, packed, codes.
template <int BITS, int T, int CPL>
__global__ __launch_bounds__(256) void quantize_team_kernel(
    const uint16_t* __restrict__ W, uint8_t* __restrict__ codes,
    uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros, int64_t nlanes, int scheme,
    const uint32_t* __restrict__ amax) {
    const float Aall = load_amax(scheme, amax);
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool live = t < nlanes;            // teams are all live or all dead
    const int64_t u = live ? t : nlanes - 1;
    float x[CPL][8];
    float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        uint4 raw;
        load8(W + (u * CPL + i) * 8, x[i], raw);
        float a, b;
        minmax8(raw, a, b);
        mn = __builtin_fminf(mn, a);
        mx = __builtin_fmaxf(mx, b);
    }
    group_minmax<T>(mn, mx);
    if constexpr (BITS == 4) {
        if (scheme == 3) {
            const Nf4Group g = nf4_group(mn, mx);
            if (!live) return;
            uint32_t p[CPL];
#pragma unroll
            for (int i = 0; i < CPL; ++i) p[i] = nf4_encode8(x[i], g);
            store_codes<4, CPL>(codes + u * CPL * 4, p);
            if ((threadIdx.x & (T - 1)) == 0) {
                scales[u / T] = g.sbits;
                zeros[u / T] = 0;
            }
            return;
        }
    }
    if (scheme == 4) {
        const uint16_t sb = scale_bits_exact(mn, mx, (1 << BITS) - 1);
        const float s = half_bits_to_float(sb);
        if (!live) return;
        typename Packed8<BITS>::type p[CPL];
#pragma unroll
        for (int i = 0; i < CPL; ++i) p[i] = encode8_offset<BITS>(x[i], mn, s);
        store_codes<BITS, CPL>(codes + u * CPL * BITS, p);
        if ((threadIdx.x & (T - 1)) == 0) {
            scales[u / T] = sb;
            zeros[u / T] = float_to_half_bits_rne(mn);   // exact: mn is an fp16 input
        }
        return;
    }
    const GroupHeader h = header_for(scheme, mn, mx, Aall, BITS);
    if (!live) return;
    typename Packed8<BITS>::type p[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) p[i] = encode8<BITS>(x[i], h);
    store_codes<BITS, CPL>(codes + u * CPL * BITS, p);
    if ((threadIdx.x & (T - 1)) == 0) {
        scales[u / T] = h.sbits;
        zeros[u / T] = h.zbits;
    }
}

// One wave per group for wide groups (G > 512 or G/8 not a power of two):
// pass 1 reduces min/max over the group, pass 2 re-reads and encodes.
template <int BITS>
__global__ __launch_bounds__(256) void quantize_wave_kernel(
    const uint16_t* __restrict__ W, uint8_t* __restrict__ codes,
    uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros, int64_t ngroups,
    int64_t G, int scheme, const uint32_t* __restrict__ amax) {
    const float Aall = load_amax(scheme, amax);
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t g = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
    if (g >= ngroups) return;                // whole wave leaves together
    const int64_t cpg = G / 8;               // chunks per group
    const int64_t c0 = g * cpg;
    float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
    for (int64_t j = lane; j < cpg; j += kWave) {
        float x[8], a, b;
        uint4 raw;
        load8(W + (c0 + j) * 8, x, raw);
        minmax8(raw, a, b);
        mn = __builtin_fminf(mn, a);
        mx = __builtin_fmaxf(mx, b);
    }
    group_minmax<kWave>(mn, mx);
    if constexpr (BITS == 4) {
        if (scheme == 3) {
            const Nf4Group ng = nf4_group(mn, mx);
            for (int64_t j = lane; j < cpg; j += kWave) {
                float x[8];
                uint4 raw;
                load8(W + (c0 + j) * 8, x, raw);
                const uint32_t p = nf4_encode8(x, ng);
                store_codes<4, 1>(codes + (c0 + j) * 4, &p);
            }
            if (lane == 0) {
                scales[g] = ng.sbits;
                zeros[g] = 0;
            }
            return;
        }
    }
    if (scheme == 4) {
        const uint16_t sb = scale_bits_exact(mn, mx, (1 << BITS) - 1);
        const float s = half_bits_to_float(sb);
        for (int64_t j = lane; j < cpg; j += kWave) {
            float x[8];
            uint4 raw;
            load8(W + (c0 + j) * 8, x, raw);
            const typename Packed8<BITS>::type p = encode8_offset<BITS>(x, mn, s);
            store_codes<BITS, 1>(codes + (c0 + j) * BITS, &p);
        }
        if (lane == 0) {
            scales[g] = sb;
            zeros[g] = float_to_half_bits_rne(mn);
        }
        return;
    }
    const GroupHeader h = header_for(scheme, mn, mx, Aall, BITS);
    for (int64_t j = lane; j < cpg; j += kWave) {
        float x[8];
        uint4 raw;
        load8(W + (c0 + j) * 8, x, raw);
        const typename Packed8<BITS>::type p = encode8<BITS>(x, h);
        store_codes<BITS, 1>(codes + (c0 + j) * BITS, &p);
    }
    if (lane == 0) {
        scales[g] = h.sbits;
        zeros[g] = h.zbits;
    }
}

// Absolute maximum of the whole matrix, as fp16 magnitude bits: each block
// reduces a grid-strided share of the 16-byte chunks into part[block], then
// one block reduces the partials into *out.
constexpr int kAmaxBlocks = 1024;

__device__ __forceinline__ uint32_t max_u32(uint32_t a, uint32_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint32_t block_max_u32(uint32_t m) {
    __shared__ uint32_t red[4];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = max_u32(m, (uint32_t)__shfl_xor((int)m, o, kWave));
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = m;
    __syncthreads();
    return max_u32(max_u32(red[0], red[1]), max_u32(red[2], red[3]));
}

__global__ __launch_bounds__(256) void amax_partial_kernel(const uint16_t* __restrict__ W,
                                                           int64_t nchunks,
                                                           uint32_t* __restrict__ part) {
    uint32_t m = 0;
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < nchunks;
         c += (int64_t)gridDim.x * 256) {
        const uint4 r = *reinterpret_cast<const uint4*>(W + c * 8);
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
            m = max_u32(m, max_u32(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
    }
    m = block_max_u32(m);
    if (threadIdx.x == 0) part[blockIdx.x] = m;
}

__global__ __launch_bounds__(256) void amax_final_kernel(const uint32_t* __restrict__ part,
                                                         int nparts, uint32_t* __restrict__ out) {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < nparts; i += 256) m = max_u32(m, part[i]);
    m = block_max_u32(m);
    if (threadIdx.x == 0) out[0] = m;
}

template <int BITS, int T, int CPL>
hipError_t launch_team(const uint16_t* w, uint8_t* c, uint16_t* s, uint16_t* z, int64_t nvals,
                       int scheme, const uint32_t* amax, hipStream_t stream) {
    const int64_t nlanes = nvals / (8 * CPL);
    const dim3 grid((unsigned)((nlanes + 255) / 256));
    quantize_team_kernel<BITS, T, CPL><<<grid, dim3(256), 0, stream>>>(w, c, s, z, nlanes,
                                                                       scheme, amax);
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const void* W, int64_t N, int64_t K, int32_t G, void* codes,
                       void* scales, void* zeros, int scheme, const uint32_t* amax,
                       hipStream_t stream) {
    const uint16_t* w = static_cast<const uint16_t*>(W);
    uint8_t* c = static_cast<uint8_t*>(codes);
    uint16_t* s = static_cast<uint16_t*>(scales);
    uint16_t* z = static_cast<uint16_t*>(zeros);
    const int64_t nv = N * K;
    switch (G) {
        case 8: return launch_team<BITS, 1, 1>(w, c, s, z, nv, scheme, amax, stream);
        case 16: return launch_team<BITS, 1, 2>(w, c, s, z, nv, scheme, amax, stream);
        case 32: return launch_team<BITS, 1, 4>(w, c, s, z, nv, scheme, amax, stream);
        case 64: return launch_team<BITS, 2, 4>(w, c, s, z, nv, scheme, amax, stream);
        case 128: return launch_team<BITS, 4, 4>(w, c, s, z, nv, scheme, amax, stream);
        case 256: return launch_team<BITS, 8, 4>(w, c, s, z, nv, scheme, amax, stream);
        case 512: return launch_team<BITS, 16, 4>(w, c, s, z, nv, scheme, amax, stream);
        case 1024: return launch_team<BITS, 32, 4>(w, c, s, z, nv, scheme, amax, stream);
        case 2048: return launch_team<BITS, 64, 4>(w, c, s, z, nv, scheme, amax, stream);
        default: {
            const int64_t ngroups = nv / G;
            const dim3 grid((unsigned)((ngroups + 3) / 4));
            quantize_wave_kernel<BITS><<<grid, dim3(256), 0, stream>>>(w, c, s, z, ngroups, G,
                                                                       scheme, amax);
            return hipGetLastError();
        }
    }
}

}  // namespace

size_t quantize_scratch_bytes(int32_t scheme) {
    return scheme == 2 ? (size_t)(kAmaxBlocks + 1) * sizeof(uint32_t) : 0;
}

hipError_t launch_quantize_pack(const void* W, int64_t N, int64_t K, int32_t group,
                                int32_t bits, int32_t scheme, void* codes, void* scales,
                                void* zeros, void* scratch, hipStream_t stream) {
    const uint32_t* amax = nullptr;
    if (scheme == 2) {
        // Two reduction launches into the caller's scratch: kAmaxBlocks
        // partials, then the maximum in the word after them.
        if (!scratch) return hipErrorInvalidValue;
        uint32_t* words = static_cast<uint32_t*>(scratch);
        const int64_t nchunks = N * K / 8;
        const int64_t want = (nchunks + 255) / 256;
        const int blocks = (int)(want < kAmaxBlocks ? (want < 1 ? 1 : want) : kAmaxBlocks);
        amax_partial_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
            static_cast<const uint16_t*>(W), nchunks, words);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        amax_final_kernel<<<dim3(1), dim3(256), 0, stream>>>(words, blocks, words + kAmaxBlocks);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        amax = words + kAmaxBlocks;
    }
    switch (bits) {
        case 2: return launch_bits<2>(W, N, K, group, codes, scales, zeros, scheme, amax, stream);
        case 3: return launch_bits<3>(W, N, K, group, codes, scales, zeros, scheme, amax, stream);
        case 4: return launch_bits<4>(W, N, K, group, codes, scales, zeros, scheme, amax, stream);
        case 5: return launch_bits<5>(W, N, K, group, codes, scales, zeros, scheme, amax, stream);
        case 6: return launch_bits<6>(W, N, K, group, codes, scales, zeros, scheme, amax, stream);
        case 7: return launch_bits<7>(W, N, K, group, codes, scales, zeros, scheme, amax, stream);
        case 8: return launch_bits<8>(W, N, K, group, codes, scales, zeros, scheme, amax, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace wq
