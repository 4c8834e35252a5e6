// Matrix-core product for small batches (B <= 16) that streams the packed
// weights in the load shape HBM serves best: Y[B,N] = X[B,K] * dequant(W)[N,K]^T.
//
// A decode step reads every weight once for the whole batch ("Quantization &
// inference optimisation", "Bandwidth, not compute"), so the time is the code
// stream's.  On this GPU a load-only kernel streams about 6.0-6.4 TB/s when
// each load instruction reads 256 bytes or more of each of at most four rows,
// but under 5.6 TB/s when it reads 64 or 128 bytes of each of 8 or 16 rows --
// the shape of a matrix-core operand, where 16 lanes hold 16 weight rows.  So
// this kernel loads in the first shape and rearranges in LDS:
//   - a block (8 waves, one per compute unit at a time) owns T tiles of 16
//     weight rows, for all of K; its waves split K into 512-k positions
//     (position p of every tile goes to wave (p - block) mod 8), so each wave
//     walks its positions across all the block's tiles;
//   - one item = one tile at one position: 16 rows x 256 bytes of codes, read
//     by four load instructions of 4 rows x 256 bytes (lane l: row 4i + l/16,
//     bytes 16(l%16)..), two items ahead of use in a register ring;
//   - the wave writes the item into its own LDS buffer and reads it back in
//     the matrix-core layout: lane (r16, g4) gets row r16, bytes 64r + 16g4 of
//     round r (128 k), exactly the chunk v_mfma_f32_16x16x32_f16 needs;
//   - the wave's X for its current position (16 batch rows x 512 k, fp16,
//     permuted into the order the codes unpack in) sits in its registers as
//     the A operands, and the round sums C1, C2 of X in its LDS;
//   - codes unpack exactly to fp16 1024 + q (even k) and 64 + q (odd k), the
//     MFMA accumulates from -C1, and the group header is applied per round in
//     fp32:  sum_k (q - z) s x = s * (sum_k u_k x_k - C1 - z * C2)
//     ("the kernel reconstructs an approximate float from the integer and the
//     endpoints as it reads", "Quantization");
//   - each item's total is added to the tile's running sum for this wave in
//     LDS; at the end the block adds the 8 waves' sums of every output in
//     wave order (deterministic) and writes Y in fp16.
// No scratch memory and no second kernel.  Requires 4-bit codes, group % 128
// == 0, K % 128 == 0, and the codes array under 4 GiB (buffer offsets).
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

namespace {

constexpr int SK_WAVES = 8;
constexpr int SK_TMAX = 8;                 // tiles per block at most
constexpr int SK_TROW = 256 + 16;          // LDS row of a wave's item buffer (bytes, padded)
constexpr int SK_RING = 3;                 // items in the register ring
constexpr int kBufWord3 = 0x00020000;      // raw, unswizzled gfx9 buffer
constexpr uint32_t kOob = 0xFFFFFFF0u;     // out-of-range buffer offset: reads zero, no traffic

struct SkArgs {
    const uint16_t* X;
    const uint8_t* codes;
    const uint16_t* scales;
    const uint16_t* zeros;
    uint16_t* Y;
    int64_t B, N, K;
    int64_t ntiles;
    int32_t G;
    int32_t T;          // tiles per block
};

// X vector reordered to the unpack order (0,4,1,5,2,6,3,7) of each 8 k.
__device__ __forceinline__ uint4 sk_order8(uint4 in) {
    uint4 o;
    o.x = __builtin_amdgcn_perm(in.z, in.x, 0x05040100u);
    o.y = __builtin_amdgcn_perm(in.z, in.x, 0x07060302u);
    o.z = __builtin_amdgcn_perm(in.w, in.y, 0x05040100u);
    o.w = __builtin_amdgcn_perm(in.w, in.y, 0x07060302u);
    return o;
}

// Offset-weighted (1024 per even k, 64 per odd k) and plain sums of one
// natural-order X vector; the products with 1, 64 and 1024 are exact.
__device__ __forceinline__ void sk_offset_sums(uint4 v, float& c1, float& c2) {
    const h2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    const h2_t wgt = {(_Float16)1024.0f, (_Float16)64.0f};
    float s = __builtin_amdgcn_fdot2(as_h2(v.x), one, 0.0f, false);
    s = __builtin_amdgcn_fdot2(as_h2(v.y), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(v.z), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(v.w), one, s, false);
    float w = __builtin_amdgcn_fdot2(as_h2(v.x), wgt, 0.0f, false);
    w = __builtin_amdgcn_fdot2(as_h2(v.y), wgt, w, false);
    w = __builtin_amdgcn_fdot2(as_h2(v.z), wgt, w, false);
    c1 = __builtin_amdgcn_fdot2(as_h2(v.w), wgt, w, false);
    c2 = s;
}

// B operand of k-step j of a round's chunk: the codes as exact fp16
// (1024 + q for even k, 64 + q for odd k), k order (0,4,1,5,2,6,3,7).
__device__ __forceinline__ h8_t sk_unpack(const uint4& cw, int j, uint32_t m_lo, uint32_t m_hi,
                                          uint32_t g_lo, uint32_t g_hi) {
    const uint32_t w = j == 0 ? cw.x : j == 1 ? cw.y : j == 2 ? cw.z : cw.w;
    const uint32_t w8 = w >> 8;
    uint4 b;
    b.x = (w & m_lo) | g_lo;
    b.y = (w & m_hi) | g_hi;
    b.z = (w8 & m_lo) | g_lo;
    b.w = (w8 & m_hi) | g_hi;
    return __builtin_bit_cast(h8_t, b);
}

__device__ __forceinline__ void sk_wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float sk_half(uint32_t w, int hi) {
    return hi ? (float)as_h2(w).y : (float)as_h2(w).x;
}

// HM: how headers are read.  1: one group per 128-k round with 8-byte
// aligned runs (G == 128, K % 512 == 0, header arrays 8-byte aligned): one
// 8-byte load of scales and one of zeros per item and lane.  0: any group that
// is a multiple of 128 k: one 2-byte load of each per round.
template <int HM>
__global__ __launch_bounds__(SK_WAVES * 64, 1) void gemm_sk_kernel(const SkArgs a) {
    __shared__ __align__(16) unsigned char trans[SK_WAVES][16 * SK_TROW];
    __shared__ __align__(16) float csum[SK_WAVES][2][4][16];      // [wave][-C1, C2][round][batch row]
    __shared__ __align__(16) float red[SK_TMAX][SK_WAVES][64 * 4]; // running item totals

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, g4 = lane >> 4;
    const int64_t tile0 = (int64_t)blockIdx.x * a.T;
    const int T = (int)((a.ntiles - tile0) < a.T ? (a.ntiles - tile0) : a.T);
    const int64_t K = a.K, N = a.N, B = a.B;
    const uint32_t row_bytes = (uint32_t)(K / 2);
    const int64_t rounds = K / 128;
    const int npos = (int)((K + 511) / 512);
    const int64_t ngrp = K / a.G;
    const int rpg = a.G / 128;

    // Zero the running sums of every tile and wave (read-modify-written below).
    for (int i = tid; i < SK_TMAX * SK_WAVES * 256; i += SK_WAVES * 64) (&red[0][0][0])[i] = 0.0f;
    __syncthreads();

    // Positions of this wave: first (wave + block) mod 8, then every 8th.
    const int pfirst = (int)((wave + blockIdx.x) % SK_WAVES);
    const int my_pos = pfirst < npos ? (npos - pfirst + SK_WAVES - 1) / SK_WAVES : 0;
    const int items = my_pos * T;

    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.codes), (short)0, (int)((uint64_t)N * row_bytes), kBufWord3);
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.X), (short)0, (int)(B * K * 2), kBufWord3);

    // Weight row of a tile row, clamped (rows past N reread the last row;
    // their outputs are never stored).
    auto wrow = [&](int t, int rr) -> uint32_t {
        const int64_t row = (tile0 + t) * 16 + rr;
        return (uint32_t)(row < N ? row : N - 1);
    };
    // Item k of this wave -> (position, tile), advanced incrementally.
    // Load cursor: codes and headers of item lk.
    int l_t = 0, l_j = 0, lk = 0;
    auto next_load = [&](uint4* cw, uint32_t* hw) {
        const bool live = lk < items;
        const int p = pfirst + SK_WAVES * l_j;
        // The last position may end before 512 k: its byte offset is clamped
        // to the row (the rounds past K meet zero X and add nothing).
        uint32_t col = (uint32_t)p * 256u + 16u * (uint32_t)(lane & 15);
        col = col < row_bytes ? col : row_bytes - 16u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t off = live ? wrow(l_t, 4 * i + (lane >> 4)) * row_bytes + col : kOob;
            typedef unsigned int v4u __attribute__((ext_vector_type(4)));
            const v4u v = __builtin_amdgcn_raw_buffer_load_b128(crs, (int)off, 0, 2);
            cw[i] = make_uint4(v.x, v.y, v.z, v.w);
        }
        const uint32_t hrow = wrow(l_t, r16);
        if constexpr (HM == 1) {
            const int64_t g = (int64_t)hrow * ngrp + 4 * p;
            const uint2 s2 = *reinterpret_cast<const uint2*>(a.scales + (live ? g : 0));
            const uint2 z2 = *reinterpret_cast<const uint2*>(a.zeros + (live ? g : 0));
            hw[0] = s2.x; hw[1] = s2.y; hw[2] = z2.x; hw[3] = z2.y;
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                int64_t rr = (int64_t)4 * p + r;
                rr = rr < rounds ? rr : rounds - 1;
                const int64_t g = (int64_t)hrow * ngrp + rr / rpg;
                const uint32_t s = a.scales[live ? g : 0];
                const uint32_t z = a.zeros[live ? g : 0];
                // Packed like the 8-byte form: words 0-1 scales, 2-3 zeros.
                if (r & 1) {
                    hw[r >> 1] |= s << 16;
                    hw[2 + (r >> 1)] |= z << 16;
                } else {
                    hw[r >> 1] = s;
                    hw[2 + (r >> 1)] = z;
                }
            }
        }
        if (++l_t == T) {
            l_t = 0;
            ++l_j;
        }
        ++lk;
    };

    uint4 ring[SK_RING][4];
    uint32_t hring[SK_RING][4];
    next_load(ring[0], hring[0]);
    next_load(ring[1], hring[1]);

    const uint32_t m_lo = vgpr_const(0x000F000Fu), m_hi = vgpr_const(0x00F000F0u);
    const uint32_t g_lo = vgpr_const(0x64006400u), g_hi = vgpr_const(0x54005400u);
    unsigned char* tb = trans[wave];
    h8_t xa[4][4];                          // A operands of the current position
    int cur_pos = -1;
    int c_t = 0, c_j = 0;                   // compute cursor

    // One item from ring slot `slot`.
    auto compute_item = [&](int slot) {
        const int p = pfirst + SK_WAVES * c_j;
        if (p != cur_pos) {
            // X of this position into registers, and its round sums into LDS.
            // Lane (r16, g4) holds batch row r16, k = 512p + 128r + 32g4 + 8v.
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float c1 = 0.0f, c2 = 0.0f;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int64_t k = (int64_t)512 * p + 128 * r + 32 * g4 + 8 * v;
                    const uint32_t off = (r16 < B && k < K) ? (uint32_t)((r16 * K + k) * 2) : kOob;
                    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
                    const v4u t = __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)off, 0, 0);
                    const uint4 x = make_uint4(t.x, t.y, t.z, t.w);
                    float d1, d2;
                    sk_offset_sums(x, d1, d2);
                    c1 += d1;
                    c2 += d2;
                    // xa[r][j] covers k = 32g4 + 8j of the round: vector v = j.
                    xa[r][v] = __builtin_bit_cast(h8_t, sk_order8(x));
                }
                c1 += __shfl_xor(c1, 16, 64);
                c2 += __shfl_xor(c2, 16, 64);
                c1 += __shfl_xor(c1, 32, 64);
                c2 += __shfl_xor(c2, 32, 64);
                if (g4 == 0) {
                    csum[wave][0][r][r16] = -c1;
                    csum[wave][1][r][r16] = c2;
                }
            }
            sk_wave_lds_sync();
            cur_pos = p;
        }
        // Item codes -> this wave's LDS buffer (4 rows x 256 bytes per load)
        // -> round chunks in the matrix-core layout.
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint4*>(tb + (4 * i + g4) * SK_TROW + 16 * r16) = ring[slot][i];
        sk_wave_lds_sync();
        uint4 ch[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ch[r] = *reinterpret_cast<const uint4*>(tb + r16 * SK_TROW + 64 * r + 16 * g4);
        // The tile's running sum is read now and written back after the math.
        f4_t* rs = reinterpret_cast<f4_t*>(&red[c_t][wave][4 * lane]);
        const f4_t old = *rs;
        // The four rounds are independent accumulation chains: step j of all
        // four goes out before step j + 1, so the matrix core never waits on
        // its own previous result.
        f4_t acc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = *reinterpret_cast<const f4_t*>(&csum[wave][0][r][4 * g4]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[r][j], sk_unpack(ch[r], j, m_lo, m_hi, g_lo, g_hi),
                                                                acc[r], 0, 0, 0);
        f4_t tot = old;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const f4_t cs2 = *reinterpret_cast<const f4_t*>(&csum[wave][1][r][4 * g4]);
            const float s = sk_half(hring[slot][r >> 1], r & 1);
            const float z = sk_half(hring[slot][2 + (r >> 1)], r & 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) tot[i] = __builtin_fmaf(s, __builtin_fmaf(-z, cs2[i], acc[r][i]), tot[i]);
        }
        *rs = tot;
        sk_wave_lds_sync();
        if (++c_t == T) {
            c_t = 0;
            ++c_j;
        }
    };

    // Items in groups of three (static ring slots); loads run two items ahead.
    for (int k = 0; k < items; k += SK_RING) {
#pragma unroll
        for (int d = 0; d < SK_RING; ++d) {
            next_load(ring[(d + 2) % SK_RING], hring[(d + 2) % SK_RING]);
            if (k + d < items) compute_item(d);
        }
    }
    __syncthreads();

    // Y = fp16(sum over the 8 waves, in wave order).  Output o of tile t:
    // batch row b = (o / 16) % 16, weight row 16 t + o % 16; its running sum
    // sits with lane (o % 16) + 16 (b / 4), element b % 4.
    for (int o = tid; o < T * 256; o += SK_WAVES * 64) {
        const int t = o >> 8, b = (o >> 4) & 15, rr = o & 15;
        const int64_t row = (tile0 + t) * 16 + rr;
        if (b >= B || row >= N) continue;
        const int idx = 4 * (rr + 16 * (b >> 2)) + (b & 3);
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < SK_WAVES; ++w) s += red[t][w][idx];
        a.Y[b * N + row] = float_to_half_bits_rne(s);
    }
}

}  // namespace

bool sk_supports(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits) {
    return bits == 4 && B >= 1 && B <= 16 && group % 128 == 0 && K % 128 == 0 && K >= 128 && N >= 1 &&
           (uint64_t)N * (uint64_t)(K / 2) <= 0xFFFFFF00ull && (uint64_t)B * (uint64_t)K * 2 <= 0xFFFFFF00ull;
}

hipError_t launch_gemm_sk(const void* X, const void* codes, const void* scales, const void* zeros, void* Y,
                          int64_t B, int64_t K, int64_t N, int32_t group, int num_cus, hipStream_t stream) {
    if (!sk_supports(B, K, N, group, 4)) return hipErrorInvalidValue;
    const int64_t ntiles = (N + 15) / 16;
    // About one block per compute unit, at most SK_TMAX tiles each.
    int64_t T = (ntiles + num_cus - 1) / num_cus;
    if (T > SK_TMAX) T = SK_TMAX;
    if (T < 1) T = 1;
    const int64_t blocks = (ntiles + T - 1) / T;
    SkArgs a{static_cast<const uint16_t*>(X), static_cast<const uint8_t*>(codes),
             static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros),
             static_cast<uint16_t*>(Y), B, N, K, ntiles, group, (int32_t)T};
    const bool hv = group == 128 && K % 512 == 0 && (K / 128) % 4 == 0 &&
                    reinterpret_cast<uintptr_t>(scales) % 8 == 0 && reinterpret_cast<uintptr_t>(zeros) % 8 == 0;
    if (hv)
        gemm_sk_kernel<1><<<dim3((unsigned)blocks), dim3(SK_WAVES * 64), 0, stream>>>(a);
    else
        gemm_sk_kernel<0><<<dim3((unsigned)blocks), dim3(SK_WAVES * 64), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace wq
