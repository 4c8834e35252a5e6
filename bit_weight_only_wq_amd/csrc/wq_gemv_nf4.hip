// Decode GEMV for NF4 weights (gfx950, VALU):
//   Y[B,N] = X[B,K] * (level[q] * s)[N,K]^T
// NF4 ("Gör inference billig: KV cache, batching och kvantisering", the NF4
// paragraph): sixteen fixed levels at normal quantiles, one absolute-maximum
// scale per group, codes two per byte (even k in the low nibble).  Levels
// are not an affine function of the code, so the unpack is a table lookup:
// a 256-entry LDS table maps a code byte to the fp16 pair (level[low],
// level[high]), which v_dot2_f32_f16 multiplies with the matching X pair
// (k even, k odd: X in its natural order).  The scale enters once per
// 32-code chunk in fp32: sum_k x_k level[q_k] s = s * sum_k x_k level[q_k].
//
// Code bytes are random, so one shared table puts several lanes of a wave on
// one LDS bank with different addresses.  The table is therefore replicated
// NCP times, interleaved by entry (entry b of copy c at word b * NCP + c),
// and lane l reads copy l % NCP: with NCP = 32 every lane of a 32-lane LDS
// cycle owns its bank.  Larger X tiles (NB = 4) keep fewer copies.
//
// Same plan as the other GEMVs: persistent blocks stream 16-byte code chunks
// non-temporally, X staged once per block in LDS, fp32 accumulation, row sums
// across the TG lanes of a row by DPP.
#include "wq_device.h"
#include "wq_launch.h"
#include "wq_nf4_levels.h"

namespace wq {

namespace {

constexpr size_t kNf4MaxLds = 128 * 1024;   // of the 160 KB a gfx950 workgroup may hold

// Table copies per X tile height, and the table's LDS bytes.
constexpr int nf4_copies(int nb) { return nb == 1 ? 32 : 8; }
constexpr size_t nf4_lut_bytes(int nb) { return (size_t)256 * nf4_copies(nb) * sizeof(uint32_t); }

// Grid: (persistent row-pass blocks, ceil(B / NB)).  TG threads per row,
// 256 / TG rows per pass; thread tl owns chunks tl, tl + TG, ... (CPT).
template <int NB, int TG, int CPT>
__global__ __launch_bounds__(256) void gemv_nf4_kernel(
    const uint16_t* __restrict__ X, const uint4* __restrict__ codes,
    const uint16_t* __restrict__ scales, uint16_t* __restrict__ Y, int64_t B, int64_t N,
    int64_t K, int32_t G) {
    constexpr int RPB = 256 / TG;
    constexpr int NCP = nf4_copies(NB);
    extern __shared__ __align__(16) unsigned char smem[];
    uint32_t* lut = reinterpret_cast<uint32_t*>(smem);
    uint4* xs = reinterpret_cast<uint4*>(smem + nf4_lut_bytes(NB));   // [NB][K/8] uint4

    const int tid = threadIdx.x;
    const int rs = tid / TG;
    const int tl = tid % TG;
    const int C = (int)(K / 32);               // chunks per row
    const int64_t ngrp = K / G;
    const int64_t b0 = (int64_t)blockIdx.y * NB;
    const int nb = (int)((B - b0) < NB ? (B - b0) : NB);
    const int64_t passes = (N + RPB - 1) / RPB;

    for (int e = tid; e < 256 * NCP; e += 256) {
        const int b = e / NCP;
        lut[e] = (uint32_t)kNf4LevelBits[b & 15] | ((uint32_t)kNf4LevelBits[b >> 4] << 16);
    }
    const uint32_t* lutl = lut + (tid % NCP);  // this lane's copy
    const int xw = (int)(K / 8);               // uint4 per X row
    for (int e = tid; e < NB * xw; e += 256) {
        const int b = e / xw, c = e % xw;
        xs[e] = b < nb ? reinterpret_cast<const uint4*>(X + (b0 + b) * K)[c] : make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();

    int cidx[CPT];
    bool cin[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int c = tl + TG * i;
        cin[i] = c < C;
        cidx[i] = c < C ? c : C - 1;
    }

    // Codes and scales of a pass; rows past N read row N - 1 (their result
    // is dropped), so every pass issues the same loads.
    auto load_pass = [&](int64_t pass, uint4* w, uint32_t* hs) {
        int64_t n = pass * RPB + rs;
        n = n < N ? n : N - 1;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            w[i] = load_stream(codes + n * C + cidx[i]);
            hs[i] = scales[n * ngrp + ((int64_t)cidx[i] * 32) / G];
        }
    };
    auto compute_pass = [&](int64_t pass, const uint4* w, const uint32_t* hs) {
        const int64_t n = pass * RPB + rs;
        const bool row_ok = n < N;
        float acc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = 0.0f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            // X does not change between passes: an opaque copy of the chunk
            // index keeps its LDS reads inside the loop (not hoisted into
            // registers) and orders them after the previous chunk's math.
            int ci = cidx[i];
            asm volatile("" : "+v"(ci) : "v"(acc[0]));
            const uint32_t ww[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
            uint32_t pr[16];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int k = 0; k < 4; ++k) pr[4 * j + k] = lutl[((ww[j] >> (8 * k)) & 0xFFu) * NCP];
            const float s = (row_ok && cin[i]) ? half_bits_to_float((uint16_t)hs[i]) : 0.0f;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const uint4* xp = xs + (size_t)b * xw + (size_t)ci * 4;
                float p = 0.0f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint4 xv = xp[r];
                    p = __builtin_amdgcn_fdot2(as_h2(pr[4 * r]), as_h2(xv.x), p, false);
                    p = __builtin_amdgcn_fdot2(as_h2(pr[4 * r + 1]), as_h2(xv.y), p, false);
                    p = __builtin_amdgcn_fdot2(as_h2(pr[4 * r + 2]), as_h2(xv.z), p, false);
                    p = __builtin_amdgcn_fdot2(as_h2(pr[4 * r + 3]), as_h2(xv.w), p, false);
                }
                acc[b] = __builtin_fmaf(s, p, acc[b]);
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = group_sum<TG>(acc[b]);
        if (tl == 0 && row_ok) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (b < nb) Y[(b0 + b) * N + n] = float_to_half_bits_rne(acc[b]);
        }
    };

    // Ping-pong: the next pass's loads are in flight while this pass computes.
    const int64_t step = gridDim.x;
    uint4 wa[CPT], wb[CPT];
    uint32_t ha[CPT], hb[CPT];
    int64_t pass = blockIdx.x;
    load_pass(pass, wa, ha);
    for (; pass < passes; pass += 2 * step) {
        load_pass(pass + step, wb, hb);
        compute_pass(pass, wa, ha);
        if (pass + step >= passes) break;
        load_pass(pass + 2 * step, wa, ha);
        compute_pass(pass + step, wb, hb);
    }
}

struct Nf4Choice {
    int nb, tg, cpt;
};

bool nf4_choose(int64_t B, int64_t K, int32_t G, Nf4Choice& ch) {
    if (K % 32 != 0 || G % 32 != 0) return false;
    const int64_t C = K / 32;
    const size_t row = (size_t)K * 2;
    ch.nb = B >= 2 && nf4_lut_bytes(4) + 4 * row <= kNf4MaxLds ? 4 : 1;
    if (nf4_lut_bytes(ch.nb) + ch.nb * row > kNf4MaxLds) return false;
    if (C <= 16) ch.tg = 16, ch.cpt = 1;
    else if (C <= 32) ch.tg = 16, ch.cpt = 2;
    else if (C <= 64) ch.tg = 64, ch.cpt = 1;
    else if (C <= 128) ch.tg = 64, ch.cpt = 2;
    else if (C <= 256) ch.tg = 64, ch.cpt = 4;
    else if (C <= 512) ch.tg = 64, ch.cpt = 8;
    else return false;
    return true;
}

template <int NB, int TG, int CPT>
hipError_t nf4_launch(const void* X, const void* codes, const void* scales, void* Y, int64_t B,
                      int64_t K, int64_t N, int32_t G, int num_cus, hipStream_t stream) {
    constexpr int RPB = 256 / TG;
    const size_t lds = nf4_lut_bytes(NB) + (size_t)NB * K * 2;
    static thread_local size_t cached_lds = (size_t)-1;
    static thread_local int cached_per_cu = 1;
    if (cached_lds != lds) {
        int v = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, gemv_nf4_kernel<NB, TG, CPT>, 256, lds) !=
                hipSuccess || v <= 0)
            v = 1;
        cached_lds = lds;
        cached_per_cu = v;
    }
    const int64_t passes = (N + RPB - 1) / RPB;
    const int64_t cap = (int64_t)num_cus * cached_per_cu;
    const dim3 grid((unsigned)(passes < cap ? passes : cap), (unsigned)((B + NB - 1) / NB));
    gemv_nf4_kernel<NB, TG, CPT><<<grid, dim3(256), lds, stream>>>(
        static_cast<const uint16_t*>(X), static_cast<const uint4*>(codes),
        static_cast<const uint16_t*>(scales), static_cast<uint16_t*>(Y), B, N, K, G);
    return hipGetLastError();
}

template <int NB>
hipError_t nf4_by_shape(const Nf4Choice& ch, const void* X, const void* codes, const void* scales,
                        void* Y, int64_t B, int64_t K, int64_t N, int32_t G, int cus, hipStream_t st) {
#define WQ_NF4_CASE(TG_, CPT_) \
    if (ch.tg == TG_ && ch.cpt == CPT_) return nf4_launch<NB, TG_, CPT_>(X, codes, scales, Y, B, K, N, G, cus, st);
    WQ_NF4_CASE(16, 1) WQ_NF4_CASE(16, 2) WQ_NF4_CASE(64, 1) WQ_NF4_CASE(64, 2) WQ_NF4_CASE(64, 4)
    WQ_NF4_CASE(64, 8)
#undef WQ_NF4_CASE
    return hipErrorInvalidValue;
}

}  // namespace

bool gemv_nf4_supports(int64_t K, int32_t group) {
    Nf4Choice ch;
    return nf4_choose(1, K, group, ch);
}

hipError_t launch_gemv_nf4(const void* X, const void* codes, const void* scales, void* Y, int64_t B,
                           int64_t K, int64_t N, int32_t group, int num_cus, hipStream_t stream) {
    Nf4Choice ch;
    if (!nf4_choose(B, K, group, ch)) return hipErrorInvalidValue;
    if (ch.nb == 4) return nf4_by_shape<4>(ch, X, codes, scales, Y, B, K, N, group, num_cus, stream);
    return nf4_by_shape<1>(ch, X, codes, scales, Y, B, K, N, group, num_cus, stream);
}

}  // namespace wq
