// Skinny GEMM on the matrix cores (gfx950 MFMA) for batches past the GEMV regime:
// Y[B,N] = X[B,K] * dequant(W)[N,K]^T with fp16 operands and fp32 accumulation.
//
// Once 2B/w approaches the ridge ("Quantization & inference optimisation",
// "Bandwidth, not compute") the product is a real dense contraction, so it
// runs on v_mfma_f32_16x16x32_f16:
//   - a block owns 64 weight rows (4 waves x 16 rows) and BT batch columns;
//   - every lane streams its row's codes with one 128-bit load per round
//     (4 lanes x 16 bytes = 64 contiguous bytes of each row per round) and
//     turns them in registers into A operands holding 1024 + q exactly in fp16;
//   - the round's X tile [BT x KR] is staged in LDS by the whole block (128-bit
//     loads, double-buffered), permuted into the order the codes unpack in,
//     together with its per-column sums;
//   - the group header is applied once per round and per accumulator through
//       sum_k (q - z) s x = s * (sum_k (1024 + q) x - (1024 + z) sum_k x)
//     ("the kernel reconstructs an approximate float from the integer and the
//     endpoints as it reads", "Quantization"), so the dequantized weight is
//     never rounded to fp16;
//   - per-row scales and zero points are staged in LDS, one packed pair per
//     row and round.
// Requires G % KR == 0 (KR = 128 k for 4-bit, 64 k for 8-bit).
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

namespace {

template <int BITS>
struct MfmaGeom {
    static constexpr int VALS = 128 / BITS;    // codes per 16-byte lane load
    static constexpr int KR = 4 * VALS;        // k per round (4 lane groups)
    static constexpr int KSTEPS = KR / 32;     // 16x16x32 MFMAs per round per column block
    static constexpr int SEGS = KR / 8;        // 16-byte X vectors per column per round
};

// Reorder one 8-value X vector into the order in which the codes unpack:
// 4-bit (q0,q4,q1,q5,q2,q6,q3,q7); 8-bit (q0,q2,q1,q3,q4,q6,q5,q7).
template <int BITS>
__device__ __forceinline__ uint4 permute8(uint4 in) {
    uint4 o;
    if constexpr (BITS == 4) {
        o.x = (in.x & 0xFFFFu) | (in.z << 16);
        o.y = (in.x >> 16) | (in.z & 0xFFFF0000u);
        o.z = (in.y & 0xFFFFu) | (in.w << 16);
        o.w = (in.y >> 16) | (in.w & 0xFFFF0000u);
    } else {
        o.x = (in.x & 0xFFFFu) | (in.y << 16);
        o.y = (in.x >> 16) | (in.y & 0xFFFF0000u);
        o.z = (in.z & 0xFFFFu) | (in.w << 16);
        o.w = (in.z >> 16) | (in.w & 0xFFFF0000u);
    }
    return o;
}

__device__ __forceinline__ float sum8(uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        s += half_bits_to_float((uint16_t)(w[i] & 0xFFFFu)) + half_bits_to_float((uint16_t)(w[i] >> 16));
    return s;
}

// A operand of k-step j from a lane's 16-byte chunk.
template <int BITS>
__device__ __forceinline__ h8_t a_operand(const uint4& cw, int j) {
    uint4 a;
    if constexpr (BITS == 4) {
        const uint32_t w = j == 0 ? cw.x : j == 1 ? cw.y : j == 2 ? cw.z : cw.w;
        a.x = nib_pair(w, 0);
        a.y = nib_pair(w, 1);
        a.z = nib_pair(w, 2);
        a.w = nib_pair(w, 3);
    } else {
        const uint32_t w0 = j == 0 ? cw.x : cw.z;
        const uint32_t w1 = j == 0 ? cw.y : cw.w;
        a.x = byte_pair(w0, 0);
        a.y = byte_pair(w0, 1);
        a.z = byte_pair(w1, 0);
        a.w = byte_pair(w1, 1);
    }
    return __builtin_bit_cast(h8_t, a);
}

template <int BITS, int BT>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(
    const uint16_t* __restrict__ X, const uint4* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros,
    uint16_t* __restrict__ Y, int64_t B, int64_t N, int64_t K, int32_t G) {
    typedef MfmaGeom<BITS> MG;
    constexpr int NCB = BT / 16;                      // 16-column blocks
    constexpr int XROW = MG::KR + 8;                  // padded LDS row (halfs)
    constexpr int NVEC = BT * MG::SEGS;               // X vectors per round
    constexpr int VPT = NVEC >= 256 ? NVEC / 256 : 1; // X vectors per thread

    __shared__ __align__(16) uint16_t xs[2][BT][XROW];
    __shared__ float xsum[2][BT];
    __shared__ __align__(16) uint32_t hdr[2][4][16];  // packed (scale, zero) per wave row

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int r16 = lane & 15;
    const int g4 = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 64 + wave * 16;
    const int64_t b0 = (int64_t)blockIdx.y * BT;
    const int64_t rowA = n0 + r16;
    const bool rowA_ok = rowA < N;
    const int64_t C = K / MG::VALS;
    const int64_t rounds = K / MG::KR;
    const int64_t ngrp = K / G;

    // X staging: vector v = tid + 256*u covers column v / SEGS, k-segment v % SEGS.
    auto x_load = [&](int64_t r, uint4* xr) {
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int v = tid + 256 * u;
            const int col = v / MG::SEGS, seg = v % MG::SEGS;
            uint4 val = make_uint4(0u, 0u, 0u, 0u);
            if (v < NVEC && b0 + col < B)
                val = *reinterpret_cast<const uint4*>(X + (b0 + col) * K + r * MG::KR + seg * 8);
            xr[u] = val;
        }
    };
    auto x_store = [&](int buf, const uint4* xr) {
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int v = tid + 256 * u;
            const int col = v / MG::SEGS, seg = v % MG::SEGS;
            float s = group_sum<MG::SEGS>(sum8(xr[u]));   // threads of one column are adjacent
            if (v < NVEC) {
                *reinterpret_cast<uint4*>(&xs[buf][col][seg * 8]) = permute8<BITS>(xr[u]);
                if (seg == 0) xsum[buf][col] = s;
            }
        }
    };
    auto hdr_load = [&](int64_t r) -> uint32_t {
        if (g4 != 0 || !rowA_ok) return 0u;
        const int64_t gi = rowA * ngrp + (r * MG::KR) / G;
        return (uint32_t)scales[gi] | ((uint32_t)zeros[gi] << 16);
    };

    f4_t tot[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) tot[cb] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // Prologue: round 0.
    uint4 cw = rowA_ok ? codes[rowA * C + g4] : make_uint4(0u, 0u, 0u, 0u);
    {
        uint4 xr[VPT];
        x_load(0, xr);
        x_store(0, xr);
        const uint32_t h = hdr_load(0);
        if (g4 == 0) hdr[0][wave][r16] = h;
    }
    __syncthreads();

    for (int64_t r = 0; r < rounds; ++r) {
        const int buf = (int)(r & 1);
        const bool more = r + 1 < rounds;
        uint4 cw_next = make_uint4(0u, 0u, 0u, 0u);
        uint4 xr[VPT];
        uint32_t h_next = 0u;
        if (more) {
            if (rowA_ok) cw_next = codes[rowA * C + (r + 1) * 4 + g4];
            x_load(r + 1, xr);
            h_next = hdr_load(r + 1);
        }

        f4_t acc[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[cb] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < MG::KSTEPS; ++j) {
            const h8_t a = a_operand<BITS>(cw, j);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const h8_t bop = __builtin_bit_cast(
                    h8_t, *reinterpret_cast<const uint4*>(&xs[buf][cb * 16 + r16][g4 * MG::VALS + 8 * j]));
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bop, acc[cb], 0, 0, 0);
            }
        }
        // Accumulator lane layout: rows 4*g4 + i, column r16 of each block.
        const uint4 hp = *reinterpret_cast<const uint4*>(&hdr[buf][wave][4 * g4]);
        const uint32_t hv[4] = {hp.x, hp.y, hp.z, hp.w};
        float sc[4], zc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sc[i] = half_bits_to_float((uint16_t)(hv[i] & 0xFFFFu));
            zc[i] = 1024.0f + half_bits_to_float((uint16_t)(hv[i] >> 16));
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const float xsv = xsum[buf][cb * 16 + r16];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                tot[cb][i] = __builtin_fmaf(sc[i], __builtin_fmaf(-zc[i], xsv, acc[cb][i]), tot[cb][i]);
        }

        if (more) {
            x_store(buf ^ 1, xr);
            if (g4 == 0) hdr[buf ^ 1][wave][r16] = h_next;
            cw = cw_next;
        }
        __syncthreads();
    }

#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int64_t col = b0 + cb * 16 + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t row = n0 + 4 * g4 + i;
            if (row < N && col < B) Y[col * N + row] = float_to_half_bits_rne(tot[cb][i]);
        }
    }
}

template <int BITS, int BT>
hipError_t launch_bt(const void* X, const void* codes, const void* scales, const void* zeros,
                     void* Y, int64_t B, int64_t K, int64_t N, int32_t G, hipStream_t stream) {
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((B + BT - 1) / BT));
    gemm_mfma_kernel<BITS, BT><<<grid, dim3(256), 0, stream>>>(
        static_cast<const uint16_t*>(X), static_cast<const uint4*>(codes),
        static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros),
        static_cast<uint16_t*>(Y), B, N, K, G);
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_bits(const void* X, const void* codes, const void* scales, const void* zeros,
                       void* Y, int64_t B, int64_t K, int64_t N, int32_t G, hipStream_t st) {
    if (B <= 16) return launch_bt<BITS, 16>(X, codes, scales, zeros, Y, B, K, N, G, st);
    if (B <= 32) return launch_bt<BITS, 32>(X, codes, scales, zeros, Y, B, K, N, G, st);
    return launch_bt<BITS, 64>(X, codes, scales, zeros, Y, B, K, N, G, st);
}

}  // namespace

bool mfma_supports(int64_t K, int32_t group, int32_t bits) {
    const int kr = bits == 4 ? MfmaGeom<4>::KR : MfmaGeom<8>::KR;
    return (bits == 4 || bits == 8) && group % kr == 0 && K % kr == 0;
}

hipError_t launch_gemm_mfma(const void* X, const void* codes, const void* scales,
                            const void* zeros, void* Y, int64_t B, int64_t K, int64_t N,
                            int32_t group, int32_t bits, int num_cus, hipStream_t stream) {
    (void)num_cus;
    if (bits == 4) return launch_bits<4>(X, codes, scales, zeros, Y, B, K, N, group, stream);
    return launch_bits<8>(X, codes, scales, zeros, Y, B, K, N, group, stream);
}

}  // namespace wq
