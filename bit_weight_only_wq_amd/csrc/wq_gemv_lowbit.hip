// Bit-stream decode GEMV (gfx950, VALU) for 2- and 3-bit codes with integer
// zero points, and for 2-, 3-, 4- and 8-bit codes of the float-offset variant:
//   Y[B,N] = X[B,K] * dequant(W)[N,K]^T, W stored as the little-endian bit
//   stream of wq_quantize_pack (code k of a row at bits [k*b, k*b+b)), with
//   dequant (q - z) * s (integer zero point) or q * s + m (float offset,
//   "Quantization & inference optimisation", "Quantization").  A chunk adds
//   s * sum_k q_k x_k, then -s*z or m times sum_k x_k.
//
// Same plan as the 4/8-bit GEMV ("Quantization & inference optimisation",
// "Bandwidth, not compute": at small batch the time is the bytes streamed):
// codes are read once with 16-byte loads, X sits in LDS in the order the
// codes unpack, codes become fp16 (1024 + m*q) with one AND-OR per pair, and
// v_dot2_f32_f16 accumulates in fp32; the group header enters once per chunk
// through  sum_k (q_k - z) s x_k = s * (sum_k q_k x_k - z * sum_k x_k).
// Unlike the 4/8-bit kernels, the 1024 offset is removed in fp16 (exactly)
// before the dot product instead of through a precomputed constant: with
// 2 or 3 bits most codes sit within a step or two of z, so sum_k q_k x_k is
// small next to 1024 * sum_k |x_k|, and carrying the offset through the fp32
// sums would cost more than the one extra packed subtraction per pair.
//
// The unit of work is a chunk of 32 codes, which lies in one group (group %
// 32 == 0).  A lane reads CPL chunks at a time: two 2-bit chunks in one
// 16-byte load, four 3-bit chunks in three.  Unpacking:
//   2 bits: a word holds 16 codes (code i at bits 2i).  Masking bits 2m..2m+1
//     of both halves of w and of w >> 8 gives (1024 + 4^m q) for the pairs
//     (q_m, q_{m+8}) and (q_{m+4}, q_{m+12}), m = 0..3.
//   3 bits: the 96 bits of a chunk are four 24-bit units of 8 codes (code i
//     of a unit at bits 3i).  With t = (low half of u) | (high half of u << 4),
//     bits 3r..3r+2 of both halves of t are the pair (q_r, q_{r+4}) scaled by
//     8^r for r = 0..2; (q_3, q_7) comes from (u >> 9) and (u >> 5) the same way.
// Products of the scaled pairs are summed per scale and rescaled once per
// chunk.
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

namespace {

template <int BITS>
struct LowGeom;
template <>
struct LowGeom<2> {
    static constexpr int CPL = 2;     // 32-code chunks per lane unit
    static constexpr int LOADS = 1;   // 16-byte loads per lane unit
};
template <>
struct LowGeom<3> {
    static constexpr int CPL = 4;
    static constexpr int LOADS = 3;
};
template <>
struct LowGeom<4> {
    static constexpr int CPL = 1;     // one 16-byte load, 32 codes
    static constexpr int LOADS = 1;
};
template <>
struct LowGeom<8> {
    static constexpr int CPL = 1;     // two 16-byte loads, 32 codes
    static constexpr int LOADS = 2;
};

// uint4 per X record of one (batch row, unit): 4 per chunk of fp16 X pairs,
// then one uint4 with each chunk's sum of X (xT) as a float.
template <int BITS>
constexpr int low_rec() {
    return 4 * LowGeom<BITS>::CPL + 1;
}

// Pair P (0..15) of a chunk: the positions (a, b) of its two codes within the
// chunk and the factor m its unpacked codes carry (1024 + m*q).
template <int BITS>
__host__ __device__ constexpr void low_pair(int P, int& a, int& b, int& m) {
    if constexpr (BITS == 4) {
        const int j = P >> 2, r = P & 3;                     // word, pair in word
        a = 8 * j + r;
        b = a + 4;
        m = (r & 1) ? 16 : 1;
    } else if constexpr (BITS == 8) {
        const int j = P >> 1, r = P & 1;
        a = 4 * j + r;
        b = a + 2;
        m = 1;
    } else if constexpr (BITS == 2) {
        const int j = P >> 3, h = (P >> 2) & 1, s = P & 3;   // word, w >> 8h, mask 2s
        a = 16 * j + 4 * h + s;
        b = a + 8;
        m = 1 << (2 * s);
    } else {
        const int u = P >> 2, r = P & 3;                     // unit, pair in unit
        a = 8 * u + r;
        b = a + 4;
        m = r == 1 ? 8 : r == 2 ? 64 : 1;
    }
}

// Low half from lo, high half from hi.
__device__ __forceinline__ uint32_t halves(uint32_t hi, uint32_t lo) {
    return (hi & 0xFFFF0000u) | (lo & 0x0000FFFFu);
}

// m*q as fp16 pairs: (1024 + m*q) - 1024, exact.
__device__ __forceinline__ h2_t unpack_pair(uint32_t bits, uint32_t mask) {
    const h2_t off = {(_Float16)1024.0f, (_Float16)1024.0f};
    return as_h2((bits & mask) | 0x64006400u) - off;
}

// sum_k q_k x_k of one chunk against one batch row's X pairs (xp: the chunk's
// 4 uint4): fp32 partial sums by scale class, rescaled at the end.
template <int BITS>
__device__ __forceinline__ float chunk_dot(const uint32_t* cw, const uint4* xp,
                                           const uint32_t* mask) {
    float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    uint32_t x[16];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint4 v = xp[r];
        x[4 * r] = v.x;
        x[4 * r + 1] = v.y;
        x[4 * r + 2] = v.z;
        x[4 * r + 3] = v.w;
    }
    if constexpr (BITS == 2) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t v = h ? cw[j] >> 8 : cw[j];
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    p[s] = __builtin_amdgcn_fdot2(unpack_pair(v, mask[s]), as_h2(x[8 * j + 4 * h + s]), p[s], false);
            }
        return __builtin_fmaf(p[3], 0.015625f, __builtin_fmaf(p[2], 0.0625f, __builtin_fmaf(p[1], 0.25f, p[0])));
    } else if constexpr (BITS == 4) {
        // Word j holds codes 8j..8j+7: (q0,q4) and (q2,q6) as 1024 + q,
        // (q1,q5) and (q3,q7) as 1024 + 16q.
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t sh = cw[j] >> 8;
            p[0] = __builtin_amdgcn_fdot2(unpack_pair(cw[j], mask[0]), as_h2(x[4 * j]), p[0], false);
            p[1] = __builtin_amdgcn_fdot2(unpack_pair(cw[j], mask[1]), as_h2(x[4 * j + 1]), p[1], false);
            p[0] = __builtin_amdgcn_fdot2(unpack_pair(sh, mask[0]), as_h2(x[4 * j + 2]), p[0], false);
            p[1] = __builtin_amdgcn_fdot2(unpack_pair(sh, mask[1]), as_h2(x[4 * j + 3]), p[1], false);
        }
        return __builtin_fmaf(p[1], 0.0625f, p[0]);
    } else if constexpr (BITS == 8) {
        // Word j holds codes 4j..4j+3: (q0,q2) and (q1,q3) as 1024 + q.
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[0] = __builtin_amdgcn_fdot2(unpack_pair(cw[j], mask[0]), as_h2(x[2 * j]), p[0], false);
            p[1] = __builtin_amdgcn_fdot2(unpack_pair(cw[j] >> 8, mask[0]), as_h2(x[2 * j + 1]), p[1], false);
        }
        return p[0] + p[1];
    } else {
        const uint32_t u[4] = {cw[0], __builtin_amdgcn_alignbit(cw[1], cw[0], 24),
                               __builtin_amdgcn_alignbit(cw[2], cw[1], 16), cw[2] >> 8};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t t = halves(u[k] << 4, u[k]);
            const uint32_t t3 = halves(u[k] >> 5, u[k] >> 9);
            p[0] = __builtin_amdgcn_fdot2(unpack_pair(t, mask[0]), as_h2(x[4 * k]), p[0], false);
            p[1] = __builtin_amdgcn_fdot2(unpack_pair(t, mask[1]), as_h2(x[4 * k + 1]), p[1], false);
            p[2] = __builtin_amdgcn_fdot2(unpack_pair(t, mask[2]), as_h2(x[4 * k + 2]), p[2], false);
            p[3] = __builtin_amdgcn_fdot2(unpack_pair(t3, mask[0]), as_h2(x[4 * k + 3]), p[3], false);
        }
        return __builtin_fmaf(p[2], 0.015625f, __builtin_fmaf(p[1], 0.125f, p[0] + p[3]));
    }
}

// Grid: (persistent row-pass blocks, ceil(B / NB)).  TG threads per row,
// 256 / TG rows per block pass; thread tl of a row owns units tl, tl + TG, ...
// (CPT of them).  HPU = group headers per unit: 1 when a group spans whole
// units, CPL when every chunk may start a new group.  offset != 0: `zeros`
// holds float offsets (q * s + m) instead of integer zero points.
template <int BITS, int NB, int TG, int CPT, int HPU>
__global__ __launch_bounds__(256) void gemv_lowbit_kernel(
    const uint16_t* __restrict__ X, const uint4* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros,
    uint16_t* __restrict__ Y, int64_t B, int64_t N, int64_t K, int32_t G, int offset) {
    typedef LowGeom<BITS> LG;
    constexpr int CPL = LG::CPL;
    constexpr int LOADS = LG::LOADS;
    constexpr int REC = low_rec<BITS>();
    constexpr int RPB = 256 / TG;
    constexpr int CPH = CPL / HPU;              // chunks per loaded header
    extern __shared__ __align__(16) unsigned char smem[];
    uint4* xrec = reinterpret_cast<uint4*>(smem);

    const int tid = threadIdx.x;
    const int rs = tid / TG;
    const int tl = tid % TG;
    const int U = (int)(K / (32 * CPL));       // units per row
    const int64_t ngrp = K / G;
    const int64_t b0 = (int64_t)blockIdx.y * NB;
    const int nb = (int)((B - b0) < NB ? (B - b0) : NB);
    const int64_t passes = (N + RPB - 1) / RPB;

    uint32_t mask[4] = {0u, 0u, 0u, 0u};
    if constexpr (BITS == 4) {
        mask[0] = vgpr_const(0x000F000Fu);
        mask[1] = vgpr_const(0x00F000F0u);
    } else if constexpr (BITS == 8) {
        mask[0] = vgpr_const(0x00FF00FFu);
    } else if constexpr (BITS == 2) {
        mask[0] = vgpr_const(0x00030003u);
        mask[1] = vgpr_const(0x000C000Cu);
        mask[2] = vgpr_const(0x00300030u);
        mask[3] = vgpr_const(0x00C000C0u);
    } else {
        mask[0] = vgpr_const(0x00070007u);
        mask[1] = vgpr_const(0x00380038u);
        mask[2] = vgpr_const(0x01C001C0u);
        mask[3] = 0u;
    }

    // ---- X records into LDS ---------------------------------------------------
    for (int e = tid; e < NB * U; e += 256) {
        const int b = e / U, c = e % U;
        uint4* rec = xrec + (size_t)e * REC;
        float xt[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < CPL; ++k) {
            uint16_t xv[32];
            if (b < nb) {
                const uint4* src = reinterpret_cast<const uint4*>(
                    X + (b0 + b) * K + ((int64_t)c * CPL + k) * 32);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint4 t = src[v];
                    const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        xv[8 * v + 2 * q] = (uint16_t)(w[q] & 0xFFFFu);
                        xv[8 * v + 2 * q + 1] = (uint16_t)(w[q] >> 16);
                    }
                }
            } else {
#pragma unroll
                for (int v = 0; v < 32; ++v) xv[v] = 0;
            }
            uint32_t pr[16];
            float ts = 0.0f;
#pragma unroll
            for (int P = 0; P < 16; ++P) {
                int a = 0, bb = 0, m = 1;
                low_pair<BITS>(P, a, bb, m);
                pr[P] = (uint32_t)xv[a] | ((uint32_t)xv[bb] << 16);
                ts += half_bits_to_float(xv[a]) + half_bits_to_float(xv[bb]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                rec[4 * k + r] = make_uint4(pr[4 * r], pr[4 * r + 1], pr[4 * r + 2], pr[4 * r + 3]);
            xt[k] = ts;
        }
        rec[4 * CPL] = make_uint4(__builtin_bit_cast(uint32_t, xt[0]), __builtin_bit_cast(uint32_t, xt[1]),
                                  __builtin_bit_cast(uint32_t, xt[2]), __builtin_bit_cast(uint32_t, xt[3]));
    }
    __syncthreads();

    // This thread's units (clamped past the row's end; those add s = 0).
    int cidx[CPT];
    bool cin[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int c = tl + TG * i;
        cin[i] = c < U;
        cidx[i] = c < U ? c : U - 1;
    }

    for (int64_t pass = blockIdx.x; pass < passes; pass += gridDim.x) {
        int64_t n = pass * RPB + rs;
        const bool row_ok = n < N;
        n = row_ok ? n : N - 1;
        const uint4* rowc = codes + n * (int64_t)U * LOADS;
        const uint16_t* rows = scales + n * ngrp;
        const uint16_t* rowz = zeros + n * ngrp;
        uint4 w[CPT][LOADS];
        uint32_t hs[CPT][HPU], hz[CPT][HPU];
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
#pragma unroll
            for (int l = 0; l < LOADS; ++l) w[i][l] = load_stream(rowc + (int64_t)cidx[i] * LOADS + l);
#pragma unroll
            for (int h = 0; h < HPU; ++h) {
                const int64_t g = ((int64_t)cidx[i] * CPL + h * CPH) * 32 / G;
                hs[i][h] = rows[g];
                hz[i][h] = rowz[g];
            }
        }
        float acc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = 0.0f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            uint32_t cw[4 * LOADS];
#pragma unroll
            for (int l = 0; l < LOADS; ++l) {
                cw[4 * l] = w[i][l].x;
                cw[4 * l + 1] = w[i][l].y;
                cw[4 * l + 2] = w[i][l].z;
                cw[4 * l + 3] = w[i][l].w;
            }
            // The X records do not change between passes: an opaque copy of the
            // unit index keeps their LDS reads inside the pass loop (instead of
            // hoisted into registers), and its dependency on acc orders unit
            // i's reads after unit i-1's math, bounding the X held in flight.
            int ci = cidx[i];
            asm volatile("" : "+v"(ci) : "v"(acc[0]));
#pragma unroll
            for (int k = 0; k < CPL; ++k) {
                const float s = (row_ok && cin[i]) ? half_bits_to_float((uint16_t)hs[i][k / CPH]) : 0.0f;
                const float z = half_bits_to_float((uint16_t)hz[i][k / CPH]);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const uint4* rec = xrec + (size_t)(b * U + ci) * REC;
                    const uint4 kx = rec[4 * CPL];
                    const uint32_t xtw = k == 0 ? kx.x : k == 1 ? kx.y : k == 2 ? kx.z : kx.w;
                    const float xT = __builtin_bit_cast(float, xtw);
                    float t = chunk_dot<BITS>(cw + BITS * k, rec + 4 * k, mask);
                    if (offset) {
                        acc[b] = __builtin_fmaf(s, t, acc[b]);
                        acc[b] = __builtin_fmaf((row_ok && cin[i]) ? z : 0.0f, xT, acc[b]);
                    } else {
                        t = __builtin_fmaf(-z, xT, t);
                        acc[b] = __builtin_fmaf(s, t, acc[b]);
                    }
                }
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = group_sum<TG>(acc[b]);
        if (tl == 0 && row_ok) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (b < nb) Y[(b0 + b) * N + n] = float_to_half_bits_rne(acc[b]);
        }
    }
}

constexpr size_t kLowMaxLds = 128 * 1024;   // of the 160 KB a gfx950 workgroup may hold

struct LowChoice {
    int nb, tg, cpt, hpu;
};

bool low_choose(int64_t B, int64_t K, int32_t G, int32_t bits, LowChoice& ch) {
    const int cpl = bits == 2 ? LowGeom<2>::CPL : bits == 3 ? LowGeom<3>::CPL : 1;
    const size_t rec = (size_t)(bits == 2 ? low_rec<2>() : bits == 3 ? low_rec<3>() : low_rec<4>()) *
                       sizeof(uint4);
    if (K % (32 * cpl) != 0 || G % 32 != 0) return false;
    const int64_t U = K / (32 * cpl);
    ch.nb = B >= 2 && 4 * U * rec <= kLowMaxLds ? 4 : 1;
    if ((size_t)ch.nb * U * rec > kLowMaxLds) return false;
    if (U <= 16) ch.tg = 16, ch.cpt = 1;
    else if (U <= 32) ch.tg = 16, ch.cpt = 2;
    else if (U <= 64) ch.tg = 64, ch.cpt = 1;
    else if (U <= 128) ch.tg = 64, ch.cpt = 2;
    else if (U <= 256) ch.tg = 64, ch.cpt = 4;
    else if (U <= 512 && bits != 3) ch.tg = 64, ch.cpt = 8;
    else return false;
    ch.hpu = G % (32 * cpl) == 0 ? 1 : cpl;
    return true;
}

template <int BITS, int NB, int TG, int CPT, int HPU>
hipError_t low_launch(const void* X, const void* codes, const void* scales, const void* zeros,
                      void* Y, int64_t B, int64_t K, int64_t N, int32_t G, int offset, int num_cus,
                      hipStream_t stream) {
    constexpr int RPB = 256 / TG;
    const int64_t U = K / (32 * LowGeom<BITS>::CPL);
    const size_t lds = (size_t)NB * U * low_rec<BITS>() * sizeof(uint4);
    static thread_local size_t cached_lds = (size_t)-1;
    static thread_local int cached_per_cu = 1;
    if (cached_lds != lds) {
        int v = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, gemv_lowbit_kernel<BITS, NB, TG, CPT, HPU>, 256, lds) !=
                hipSuccess || v <= 0)
            v = 1;
        cached_lds = lds;
        cached_per_cu = v;
    }
    const int64_t passes = (N + RPB - 1) / RPB;
    const int64_t cap = (int64_t)num_cus * cached_per_cu;
    const dim3 grid((unsigned)(passes < cap ? passes : cap), (unsigned)((B + NB - 1) / NB));
    gemv_lowbit_kernel<BITS, NB, TG, CPT, HPU><<<grid, dim3(256), lds, stream>>>(
        static_cast<const uint16_t*>(X), static_cast<const uint4*>(codes),
        static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros),
        static_cast<uint16_t*>(Y), B, N, K, G, offset);
    return hipGetLastError();
}

template <int BITS, int NB, int HPU>
hipError_t low_by_shape(const LowChoice& ch, const void* X, const void* codes, const void* scales,
                        const void* zeros, void* Y, int64_t B, int64_t K, int64_t N, int32_t G,
                        int off, int cus, hipStream_t st) {
#define WQ_LOW_CASE(TG_, CPT_)                                                                   \
    if (ch.tg == TG_ && ch.cpt == CPT_)                                                          \
        return low_launch<BITS, NB, TG_, CPT_, HPU>(X, codes, scales, zeros, Y, B, K, N, G, off, cus, st);
    WQ_LOW_CASE(16, 1) WQ_LOW_CASE(16, 2) WQ_LOW_CASE(64, 1) WQ_LOW_CASE(64, 2) WQ_LOW_CASE(64, 4)
#undef WQ_LOW_CASE
    if constexpr (BITS != 3)
        if (ch.tg == 64 && ch.cpt == 8)
            return low_launch<BITS, NB, 64, 8, HPU>(X, codes, scales, zeros, Y, B, K, N, G, off, cus, st);
    return hipErrorInvalidValue;
}

template <int BITS>
hipError_t low_by_bits(const LowChoice& ch, const void* X, const void* codes, const void* scales,
                       const void* zeros, void* Y, int64_t B, int64_t K, int64_t N, int32_t G,
                       int off, int cus, hipStream_t st) {
    constexpr int CPL = LowGeom<BITS>::CPL;
    if (ch.nb == 1 && ch.hpu == 1) return low_by_shape<BITS, 1, 1>(ch, X, codes, scales, zeros, Y, B, K, N, G, off, cus, st);
    if (ch.nb == 4 && ch.hpu == 1) return low_by_shape<BITS, 4, 1>(ch, X, codes, scales, zeros, Y, B, K, N, G, off, cus, st);
    if constexpr (CPL > 1) {
        if (ch.nb == 1 && ch.hpu == CPL) return low_by_shape<BITS, 1, CPL>(ch, X, codes, scales, zeros, Y, B, K, N, G, off, cus, st);
        if (ch.nb == 4 && ch.hpu == CPL) return low_by_shape<BITS, 4, CPL>(ch, X, codes, scales, zeros, Y, B, K, N, G, off, cus, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool gemv_lowbit_supports(int64_t K, int32_t group, int32_t bits) {
    LowChoice ch;
    return (bits == 2 || bits == 3 || bits == 4 || bits == 8) && low_choose(1, K, group, bits, ch);
}

hipError_t launch_gemv_lowbit(const void* X, const void* codes, const void* scales,
                              const void* zeros, void* Y, int64_t B, int64_t K, int64_t N,
                              int32_t group, int32_t bits, int offset, int num_cus, hipStream_t stream) {
    LowChoice ch;
    if (!gemv_lowbit_supports(K, group, bits) || !low_choose(B, K, group, bits, ch)) return hipErrorInvalidValue;
    switch (bits) {
        case 2: return low_by_bits<2>(ch, X, codes, scales, zeros, Y, B, K, N, group, offset, num_cus, stream);
        case 3: return low_by_bits<3>(ch, X, codes, scales, zeros, Y, B, K, N, group, offset, num_cus, stream);
        case 4: return low_by_bits<4>(ch, X, codes, scales, zeros, Y, B, K, N, group, offset, num_cus, stream);
        case 8: return low_by_bits<8>(ch, X, codes, scales, zeros, Y, B, K, N, group, offset, num_cus, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace wq
