// Small-batch decode GEMV (gfx950, VALU): Y[B,N] = X[B,K] * dequant(W)[N,K]^T.
//
// The decode step is bandwidth-bound at small batch ("Quantization & inference
// optimisation", "Bandwidth, not compute": 2B/w FLOP per byte), so this path is
// built to stream the packed weights once at full HBM rate:
//   - each thread owns a fixed set of 16-byte code chunks of every row it
//     visits (chunk c, c+TG, c+2TG, ... of the row), read with one 128-bit
//     load each; TG consecutive threads cover a row, so a wave's loads are
//     contiguous;
//   - the matching X values live in registers for the whole kernel, already
//     permuted into the order the codes unpack in, so X is read once;
//   - codes become fp16 (1024 + q) with one AND-OR per pair ("the kernel
//     reconstructs an approximate float from the integer and the endpoints as
//     it reads", "Quantization"), and v_dot2_f32_f16 accumulates in fp32;
//   - the group header enters once per chunk through the factored form
//       sum_k (q_k - z) s x_k = s * (sum_k (1024 + q_k) x_k - (1024 + z) sum_k x_k),
//     which is exact up to fp32 rounding because 1024 + q and x are fp16 and
//     their products are exact in fp32;
//   - partial row sums are reduced across the TG threads with DPP row moves
//     and cross-row shuffles (plus LDS when a row spans several waves).
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

namespace {

template <int BITS>
struct ChunkGeom {
    static constexpr int VALS = 128 / BITS;          // codes per 16-byte chunk
    static constexpr int PAIRS = VALS / 2;           // fp16 pairs per chunk
    static constexpr int PAIRS_PER_WORD = PAIRS / 4;
};

// Pair p of word j pairs up the codes at chunk positions (first, second).
template <int BITS>
__device__ __forceinline__ void pair_positions(int j, int p, int& a, int& b) {
    if constexpr (BITS == 4) {
        a = 8 * j + p;
        b = 8 * j + p + 4;
    } else {
        a = 4 * j + p;
        b = 4 * j + p + 2;
    }
}

template <int BITS>
__device__ __forceinline__ uint32_t code_pair(uint32_t w, int p) {
    if constexpr (BITS == 4) return nib_pair(w, p);
    else return byte_pair(w, p);
}

template <int BITS, int NB, int TG, int CPT>
__global__ __launch_bounds__(256) void gemv_kernel(
    const uint16_t* __restrict__ X, const uint4* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros,
    uint16_t* __restrict__ Y, int64_t B, int64_t N, int64_t K, int32_t G) {
    typedef ChunkGeom<BITS> CG;
    constexpr int RPB = 256 / TG;      // rows per block pass
    constexpr int WPR = TG > 64 ? TG / 64 : 1;  // waves per row
    __shared__ float red[(TG > 64) ? 4 * NB : 1];

    const int tid = threadIdx.x;
    const int rs = tid / TG;           // row slot in the pass
    const int tl = tid % TG;           // thread within the row
    const int64_t C = K / CG::VALS;    // chunks per row
    const int64_t ngrp = K / G;        // groups per row
    const int cpg = G / CG::VALS;      // chunks per group
    const int64_t b0 = (int64_t)blockIdx.y * NB;
    const int nb = (int)((B - b0) < NB ? (B - b0) : NB);

    // ---- X fragments in registers (permuted pairs) and chunk sums ----------
    uint32_t xp[CPT][NB][CG::PAIRS];
    float xsum[CPT][NB];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int64_t c = tl + (int64_t)TG * i;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            uint16_t xv[CG::VALS];
            if (c < C && b < nb) {
                const uint4* src = reinterpret_cast<const uint4*>(X + (b0 + b) * K + c * CG::VALS);
#pragma unroll
                for (int v = 0; v < CG::VALS / 8; ++v) {
                    uint4 u = src[v];
                    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        xv[8 * v + 2 * e] = (uint16_t)(w[e] & 0xFFFFu);
                        xv[8 * v + 2 * e + 1] = (uint16_t)(w[e] >> 16);
                    }
                }
            } else {
#pragma unroll
                for (int v = 0; v < CG::VALS; ++v) xv[v] = 0;
            }
            float s = 0.0f;
#pragma unroll
            for (int v = 0; v < CG::VALS; ++v) s += half_bits_to_float(xv[v]);
            xsum[i][b] = s;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int p = 0; p < CG::PAIRS_PER_WORD; ++p) {
                    int a, bb;
                    pair_positions<BITS>(j, p, a, bb);
                    xp[i][b][j * CG::PAIRS_PER_WORD + p] = (uint32_t)xv[a] | ((uint32_t)xv[bb] << 16);
                }
        }
    }

    // ---- stream rows ---------------------------------------------------------
    const int64_t passes = (N + RPB - 1) / RPB;
    for (int64_t pass = blockIdx.x; pass < passes; pass += gridDim.x) {
        const int64_t n = pass * RPB + rs;
        const bool row_ok = n < N;
        uint4 w[CPT];
        float s[CPT], zc[CPT];
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int64_t c = tl + (int64_t)TG * i;
            if (row_ok && c < C) {
                w[i] = codes[n * C + c];
                const int64_t gi = n * ngrp + c / cpg;
                s[i] = half_bits_to_float(scales[gi]);
                zc[i] = 1024.0f + half_bits_to_float(zeros[gi]);
            } else {
                w[i] = make_uint4(0u, 0u, 0u, 0u);
                s[i] = 0.0f;
                zc[i] = 0.0f;
            }
        }
        float acc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = 0.0f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const uint32_t ww[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
            float part[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) part[b] = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int p = 0; p < CG::PAIRS_PER_WORD; ++p) {
                    const h2_t q = as_h2(code_pair<BITS>(ww[j], p));
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                        part[b] = __builtin_amdgcn_fdot2(
                            q, as_h2(xp[i][b][j * CG::PAIRS_PER_WORD + p]), part[b], false);
                }
#pragma unroll
            for (int b = 0; b < NB; ++b)
                acc[b] = __builtin_fmaf(s[i], __builtin_fmaf(-zc[i], xsum[i][b], part[b]), acc[b]);
        }
        // ---- reduce over the row's TG threads --------------------------------
        if constexpr (TG <= 64) {
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[b] = group_sum<TG>(acc[b]);
            if (tl == 0 && row_ok) {
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    if (b < nb) Y[(b0 + b) * N + n] = float_to_half_bits_rne(acc[b]);
            }
        } else {
            const int wave = tid / 64;       // 0..3
            const int lane = tid % 64;
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[b] = group_sum<64>(acc[b]);
            if (lane == 0) {
#pragma unroll
                for (int b = 0; b < NB; ++b) red[wave * NB + b] = acc[b];
            }
            __syncthreads();
            if (tl == 0 && row_ok) {
                const int w0 = rs * WPR;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    float t = 0.0f;
#pragma unroll
                    for (int k = 0; k < WPR; ++k) t += red[(w0 + k) * NB + b];
                    if (b < nb) Y[(b0 + b) * N + n] = float_to_half_bits_rne(t);
                }
            }
            __syncthreads();
        }
    }
}

struct GemvChoice {
    int nb, tg, cpt;
};

int pow2_ceil(int64_t v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// Batch tile NB covers the whole batch up to 8; X registers per thread are
// CPT*NB*PAIRS words, so CPT shrinks (and TG grows) as NB grows.
bool choose(int64_t B, int64_t K, int32_t bits, GemvChoice& ch) {
    const int vals = 128 / bits;
    if (K % vals != 0) return false;
    const int64_t C = K / vals;
    int nb = pow2_ceil(B < 8 ? B : 8);
    int cptmax = nb >= 4 ? 1 : 4 / nb;
    int tg = 16;
    while (tg < 256 && (int64_t)tg * cptmax < C) tg <<= 1;
    int64_t need = (C + tg - 1) / tg;
    if (need > 4) return false;
    int cpt = pow2_ceil(need);
    while (nb * cpt > 8 && nb > 1) nb >>= 1;
    ch.nb = nb;
    ch.tg = tg;
    ch.cpt = cpt;
    return true;
}

template <int BITS, int NB, int TG, int CPT>
hipError_t launch_one(const void* X, const void* codes, const void* scales, const void* zeros,
                      void* Y, int64_t B, int64_t K, int64_t N, int32_t G, int num_cus,
                      hipStream_t stream) {
    constexpr int RPB = 256 / TG;
    const int64_t passes = (N + RPB - 1) / RPB;
    const int64_t cap = (int64_t)num_cus * 8;
    const dim3 grid((unsigned)(passes < cap ? passes : cap), (unsigned)((B + NB - 1) / NB));
    gemv_kernel<BITS, NB, TG, CPT><<<grid, dim3(256), 0, stream>>>(
        static_cast<const uint16_t*>(X), static_cast<const uint4*>(codes),
        static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros),
        static_cast<uint16_t*>(Y), B, N, K, G);
    return hipGetLastError();
}

template <int BITS, int NB, int CPT>
hipError_t by_tg(int tg, const void* X, const void* codes, const void* scales,
                 const void* zeros, void* Y, int64_t B, int64_t K, int64_t N, int32_t G,
                 int cus, hipStream_t st) {
    switch (tg) {
        case 16: return launch_one<BITS, NB, 16, CPT>(X, codes, scales, zeros, Y, B, K, N, G, cus, st);
        case 32: return launch_one<BITS, NB, 32, CPT>(X, codes, scales, zeros, Y, B, K, N, G, cus, st);
        case 64: return launch_one<BITS, NB, 64, CPT>(X, codes, scales, zeros, Y, B, K, N, G, cus, st);
        case 128: return launch_one<BITS, NB, 128, CPT>(X, codes, scales, zeros, Y, B, K, N, G, cus, st);
        case 256: return launch_one<BITS, NB, 256, CPT>(X, codes, scales, zeros, Y, B, K, N, G, cus, st);
    }
    return hipErrorInvalidValue;
}

template <int BITS>
hipError_t by_shape(const GemvChoice& ch, const void* X, const void* codes, const void* scales,
                    const void* zeros, void* Y, int64_t B, int64_t K, int64_t N, int32_t G,
                    int cus, hipStream_t st) {
#define WQ_GEMV_CASE(NB_, CPT_)                                                           \
    if (ch.nb == NB_ && ch.cpt == CPT_)                                                   \
        return by_tg<BITS, NB_, CPT_>(ch.tg, X, codes, scales, zeros, Y, B, K, N, G, cus, st);
    WQ_GEMV_CASE(1, 1) WQ_GEMV_CASE(1, 2) WQ_GEMV_CASE(1, 4)
    WQ_GEMV_CASE(2, 1) WQ_GEMV_CASE(2, 2) WQ_GEMV_CASE(2, 4)
    WQ_GEMV_CASE(4, 1) WQ_GEMV_CASE(4, 2)
    WQ_GEMV_CASE(8, 1)
#undef WQ_GEMV_CASE
    return hipErrorInvalidValue;
}

}  // namespace

bool gemv_supports(int64_t K, int32_t bits) {
    GemvChoice ch;
    return choose(1, K, bits, ch) && choose(8, K, bits, ch);
}

hipError_t launch_gemv(const void* X, const void* codes, const void* scales,
                       const void* zeros, void* Y, int64_t B, int64_t K, int64_t N,
                       int32_t group, int32_t bits, int num_cus, hipStream_t stream) {
    GemvChoice ch;
    if (!choose(B, K, bits, ch)) return hipErrorInvalidValue;
    if (bits == 4)
        return by_shape<4>(ch, X, codes, scales, zeros, Y, B, K, N, group, num_cus, stream);
    return by_shape<8>(ch, X, codes, scales, zeros, Y, B, K, N, group, num_cus, stream);
}

}  // namespace wq
