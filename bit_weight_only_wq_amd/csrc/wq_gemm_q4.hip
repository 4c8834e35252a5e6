// Small-batch product (B <= 4) on the matrix cores' 4 x 4 x 4 blocks:
// Y[B,N] = X[B,K] * dequant(W)[N,K]^T.
//
// At decode batch sizes the product is a stream of the packed weights ("Quantization
// & inference optimisation", "Bandwidth, not compute": 2B/w FLOP per byte), and
// HBM here serves that stream fastest when each load instruction reads at least
// 256 bytes of each of at most four rows.  v_mfma_f32_4x4x4_16b_f16 takes that
// layout without any rearranging: it is 16 independent 4 x 4 x 4 products, block
// b on lanes 4b..4b+3, lane 4b + j holding row j of A and column j of B (four k
// each) and column j of the block's 4 x 4 result.  So:
//   - a wave owns a quad of 4 weight rows and walks K in 512-k windows; one
//     load instruction reads 256 bytes of each of the quad's rows, lane 4b + j
//     taking row j's bytes 16b..16b+15 (32 codes, k = 512v + 32b ..); every
//     4 x 4 block therefore sees the same 32 k of the 4 rows, in 8 steps of 4 k;
//   - the A operand of lane 4b + j is batch row j of X at those k (zero for
//     j >= B), read from LDS, where X sits for the kernel's life (only its B
//     rows), permuted into the order the codes unpack in, beside the sums C1,
//     C2 of every 32-k chunk;
//   - codes unpack exactly to fp16 1024 + q (even k) and 64 + q (odd k); the
//     block accumulates from -C1 and the chunk's group header is applied once
//     in fp32 ("the kernel reconstructs an approximate float from the integer
//     and the endpoints as it reads", "Quantization"):
//         sum_k (q - z) s x = s * (sum_k u_k x_k - C1 - z * C2);
//   - the quad's group headers (4 adjacent rows: one contiguous run of scales
//     and one of zeros) are read once per quad with 8-byte loads, a quad ahead,
//     and kept in the wave's LDS as (scale, zero) word pairs;
//   - after the last window the 16 blocks' sums of each row are added across
//     lanes and the quad's outputs are written in fp16;
//   - waves start their walks at different windows, so the chip's loads do not
//     all fall on the same columns at once;
//   - the grid is persistent (16 waves per compute unit); every load runs
//     eight items ahead, and loads past the end use an out-of-range buffer
//     offset (no memory traffic).
// No scratch memory.  Requires 4-bit codes, K % 32 == 0, group % 32 == 0, at
// most 128 groups per row, and 8-byte aligned header arrays.
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

namespace {

constexpr int Q4_THREADS = 1024;           // 16 waves per block, one block per compute unit
constexpr int Q4_WAVES = Q4_THREADS / 64;
constexpr int Q4_RING = 8;                 // items in flight per wave
constexpr int kQ4BufWord3 = 0x00020000;    // raw, unswizzled gfx9 buffer
constexpr uint32_t kQ4Oob = 0xFFFFFFF0u;   // out-of-range buffer offset
constexpr int Q4_HMAX = 128;               // groups per row the header buffer holds
constexpr int Q4_HWORDS = 2;               // 8-byte header loads per lane and array
constexpr int Q4_CSTRIDE = 12;             // floats per chunk-sum entry (8 used): conflict-free reads

typedef _Float16 h4_t __attribute__((ext_vector_type(4)));

struct Q4Args {
    const uint16_t* X;
    const uint8_t* codes;
    const uint16_t* scales;
    const uint16_t* zeros;
    uint16_t* Y;
    int64_t B, N, K;
    int32_t nwin;       // 512-k windows (the last may be partial)
    int32_t ngrp;       // groups per row
    int64_t nquads;     // quads of 4 rows
    uint32_t gmagic;    // ceil(2^32 / (group / 32)): chunk -> group by multiply-high (0: group 32)
};

// LDS layout:
//   X:  [nwin][4 reads][16 blocks][NB rows] of 16 bytes: read r of block b,
//       row j holds X[j][512 v + 32 b + 8 r ..] in the unpack order
//       (0,4,1,5,2,6,3,7);
//   C:  [nwin][16 blocks] entries of Q4_CSTRIDE floats: -C1[e], C2[e] of the
//       block's 32 k for batch rows e = 0..3 (zero for e >= B);
//   H:  per wave, 4 * Q4_HMAX words: (scale | zero << 16) of the quad's rows,
//       row-major (row * ngrp + group);
//   Z:  16 zero bytes, the A operand of lanes whose batch row j >= B.
template <int NB>
size_t q4_lds_bytes(int nwin) {
    return (size_t)nwin * 4 * 16 * NB * 16 + (size_t)nwin * 16 * Q4_CSTRIDE * sizeof(float) +
           (size_t)Q4_WAVES * 4 * Q4_HMAX * sizeof(uint32_t) + 16;
}

__device__ __forceinline__ uint4 q4_order8(uint4 in) {
    uint4 o;
    o.x = __builtin_amdgcn_perm(in.z, in.x, 0x05040100u);
    o.y = __builtin_amdgcn_perm(in.z, in.x, 0x07060302u);
    o.z = __builtin_amdgcn_perm(in.w, in.y, 0x05040100u);
    o.w = __builtin_amdgcn_perm(in.w, in.y, 0x07060302u);
    return o;
}

template <int NB>
__global__ __launch_bounds__(Q4_THREADS) void gemm_q4_kernel(const Q4Args a) {
    extern __shared__ __align__(16) unsigned char q4_smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int j = lane & 3;              // row of the quad (B operand), batch row (A operand)
    const int blk = lane >> 2;           // 4 x 4 block: 32-k chunk of the window
    const int64_t N = a.N, K = a.K, B = a.B;
    const int nwin = a.nwin;
    const int ngrp = a.ngrp;
    const uint32_t row_bytes = (uint32_t)(K / 2);
    const uint32_t xbytes = (uint32_t)nwin * 4 * 16 * NB * 16;
    const uint32_t cbytes = (uint32_t)nwin * 16 * Q4_CSTRIDE * 4;
    unsigned char* xl = q4_smem;
    float* cl = reinterpret_cast<float*>(q4_smem + xbytes);
    // (The zero slot is written before the barrier that ends X staging.)
    uint32_t* hb = reinterpret_cast<uint32_t*>(q4_smem + xbytes + cbytes) + (tid >> 6) * 4 * Q4_HMAX;
    const uint32_t zslot = xbytes + cbytes + (uint32_t)(Q4_WAVES * 4 * Q4_HMAX * 4);   // Z's byte offset
    if (tid < 4) reinterpret_cast<uint32_t*>(q4_smem + zslot)[tid] = 0u;

    const int64_t gw = (int64_t)blockIdx.x * Q4_WAVES + (tid >> 6);
    const int64_t nw = (int64_t)gridDim.x * Q4_WAVES;
    const int64_t my_quads = gw < a.nquads ? (a.nquads - gw + nw - 1) / nw : 0;
    const int items = (int)(my_quads * nwin);          // < 2^31: N * K / 2 < 2^32 bytes
    const int v0 = (int)(gw % nwin);     // first window of every walk of this wave

    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.codes), (short)0, (int)((uint64_t)N * row_bytes), kQ4BufWord3);

    // ---- load cursor ------------------------------------------------------------
    // Code chunk of item (quad lq, window step lw): row lq*4 + j (clamped to
    // N - 1), bytes 256 v + 16 blk with v = (v0 + lw) mod nwin.
    int64_t lq = gw;
    int lw = 0, lv = v0;
    int lk = 0;
    auto row_off = [&](int64_t q) -> uint32_t {
        const int64_t row = q * 4 + j;
        return (uint32_t)(row < N ? row : N - 1) * row_bytes;
    };
    uint32_t lrow = row_off(lq);
    const uint32_t blk_col = 16u * (uint32_t)blk;
    auto next_load = [&](uint4& cw) {
        const uint32_t col = (uint32_t)lv * 256u + blk_col;
        const uint32_t off = (lk < items && col < row_bytes) ? lrow + col : kQ4Oob;
        typedef unsigned int v4u __attribute__((ext_vector_type(4)));
        const v4u t = __builtin_amdgcn_raw_buffer_load_b128(crs, (int)off, 0, 2);
        cw = make_uint4(t.x, t.y, t.z, t.w);
        ++lk;
        if (++lv == nwin) lv = 0;
        if (++lw == nwin) {
            lw = 0;
            lq += nw;
            lrow = row_off(lq);
        }
    };

    // ---- quad headers -------------------------------------------------------------
    // The quad's scales (then zeros) are one run of 4 * ngrp halves, 8-byte
    // aligned; lane l reads 4 halves at 4 (l + 64 w) of each.
    const int hrun = 4 * ngrp;
    const int64_t run_end = N * (int64_t)ngrp;
    uint2 hreg[2][Q4_HWORDS];
    auto load_hdr = [&](int64_t q) {
        const int64_t base = (q < a.nquads ? q : 0) * hrun;
#pragma unroll
        for (int w = 0; w < Q4_HWORDS; ++w) {
            const int64_t h = base + 4 * (lane + 64 * w);
            if (4 * (lane + 64 * w) >= hrun) {
                // Past the run: never written to LDS; any valid address.
                hreg[0][w] = *reinterpret_cast<const uint2*>(a.scales + base);
                hreg[1][w] = *reinterpret_cast<const uint2*>(a.zeros + base);
            } else if (h + 4 <= run_end) {
                hreg[0][w] = *reinterpret_cast<const uint2*>(a.scales + h);
                hreg[1][w] = *reinterpret_cast<const uint2*>(a.zeros + h);
            } else {
                // A piece that runs past the last row (partial last quad with a
                // group count that is not a multiple of 4): half by half.
                uint32_t sv[4], zv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t hi = h + i < run_end ? h + i : run_end - 1;
                    sv[i] = a.scales[hi];
                    zv[i] = a.zeros[hi];
                }
                hreg[0][w] = make_uint2(sv[0] | (sv[1] << 16), sv[2] | (sv[3] << 16));
                hreg[1][w] = make_uint2(zv[0] | (zv[1] << 16), zv[2] | (zv[3] << 16));
            }
        }
    };
    load_hdr(gw);

    uint4 ring[Q4_RING];
#pragma unroll
    for (int d = 0; d < Q4_RING; ++d) next_load(ring[d]);

    // ---- X and its chunk sums -> LDS (whole block, once) ----------------------
    // Slot s = ((v * 16 + b) * 4 + r) * 4 + jj: the 16 slots of a (window,
    // block) are adjacent lanes, so a chunk's sums over its four reads r are a
    // reduction over lanes 4 apart.  Each thread's loads of a round of 4 slots
    // go out together.
    {
        const int nslots = nwin * 16 * 16;
        const h2_t one = {(_Float16)1.0f, (_Float16)1.0f};
        const h2_t wgt = {(_Float16)1024.0f, (_Float16)64.0f};
        for (int s0 = 0; s0 < nslots; s0 += 4 * Q4_THREADS) {
            uint4 xs[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int s = s0 + u * Q4_THREADS + tid;
                const int jj = s & 3, r = (s >> 2) & 3, b = (s >> 4) & 15, v = s >> 8;
                const int64_t k = (int64_t)v * 512 + 32 * b + 8 * r;
                xs[u] = make_uint4(0u, 0u, 0u, 0u);
                if (s < nslots && jj < NB && jj < B && k < K)
                    xs[u] = *reinterpret_cast<const uint4*>(a.X + jj * K + k);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int s = s0 + u * Q4_THREADS + tid;
                const bool ok = s < nslots;
                const int jj = s & 3, r = (s >> 2) & 3, b = (s >> 4) & 15, v = s >> 8;
                const uint4 x = xs[u];
                float c2 = __builtin_amdgcn_fdot2(as_h2(x.x), one, 0.0f, false);
                c2 = __builtin_amdgcn_fdot2(as_h2(x.y), one, c2, false);
                c2 = __builtin_amdgcn_fdot2(as_h2(x.z), one, c2, false);
                c2 = __builtin_amdgcn_fdot2(as_h2(x.w), one, c2, false);
                float c1 = __builtin_amdgcn_fdot2(as_h2(x.x), wgt, 0.0f, false);
                c1 = __builtin_amdgcn_fdot2(as_h2(x.y), wgt, c1, false);
                c1 = __builtin_amdgcn_fdot2(as_h2(x.z), wgt, c1, false);
                c1 = __builtin_amdgcn_fdot2(as_h2(x.w), wgt, c1, false);
                c1 += __shfl_xor(c1, 4, 64);
                c2 += __shfl_xor(c2, 4, 64);
                c1 += __shfl_xor(c1, 8, 64);
                c2 += __shfl_xor(c2, 8, 64);
                if (ok) {
                    if (jj < NB)
                        *reinterpret_cast<uint4*>(xl + ((((size_t)v * 4 + r) * 16 + b) * NB + jj) * 16) =
                            q4_order8(x);
                    if (r == 0) {
                        float* c = cl + ((size_t)v * 16 + b) * Q4_CSTRIDE;
                        c[jj] = -c1;
                        c[4 + jj] = c2;
                    }
                }
            }
        }
    }
    __syncthreads();

    const uint32_t m_lo = vgpr_const(0x000F000Fu), m_hi = vgpr_const(0x00F000F0u);
    const uint32_t g_lo = vgpr_const(0x64006400u), g_hi = vgpr_const(0x54005400u);

    f4_t tot = {0.0f, 0.0f, 0.0f, 0.0f};
    int64_t cq = gw;                     // compute cursor
    int cw_step = 0, cv = v0;
    // LDS byte offsets of this lane's X slot and chunk sums at window cv.  A
    // lane whose batch row is past the stored rows reads the zero slot: its
    // window and read strides are 0, so every read is unconditional.
    const bool xrow = NB == 4 || j < NB;
    const uint32_t x_lane = xrow ? (uint32_t)((blk * NB + j) * 16) : zslot;
    const uint32_t x_win = xrow ? 4u * 16u * NB * 16u : 0u;      // bytes per window
    const uint32_t x_read = xrow ? 16u * NB * 16u : 0u;          // bytes per read r
    const uint32_t c_lane = xbytes + (uint32_t)(blk * Q4_CSTRIDE * 4);
    const uint32_t c_win = 16u * Q4_CSTRIDE * 4u;

    auto compute = [&](const uint4& cw) {
        if (cw_step == 0) {
            // A new quad: its headers (loaded a quad ago) into the wave's LDS
            // words, then the next quad's headers in flight.
#pragma unroll
            for (int w = 0; w < Q4_HWORDS; ++w) {
                if (4 * (lane + 64 * w) < hrun) {
                    const uint2 s = hreg[0][w], z = hreg[1][w];
                    *reinterpret_cast<uint4*>(hb + 4 * (lane + 64 * w)) =
                        make_uint4(__builtin_amdgcn_perm(z.x, s.x, 0x05040100u),
                                   __builtin_amdgcn_perm(z.x, s.x, 0x07060302u),
                                   __builtin_amdgcn_perm(z.y, s.y, 0x05040100u),
                                   __builtin_amdgcn_perm(z.y, s.y, 0x07060302u));
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            load_hdr(cq + nw);
        }
        // Group of this lane's chunk: (16 v + blk) / (group / 32).
        const uint32_t chunk = 16u * (uint32_t)cv + (uint32_t)blk;
        uint32_t g = a.gmagic ? __umulhi(chunk, a.gmagic) : chunk;
        g = g < (uint32_t)ngrp ? g : (uint32_t)ngrp - 1;
        const uint32_t hw = hb[j * ngrp + (int)g];
        const float s = half_bits_to_float((uint16_t)(hw & 0xFFFFu));
        const float z = half_bits_to_float((uint16_t)(hw >> 16));
        // All LDS reads of the item first: the four X vectors, the chunk sums.
        const uint32_t xa0 = (uint32_t)cv * x_win + x_lane;
        uint4 xv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) xv[r] = *reinterpret_cast<const uint4*>(q4_smem + xa0 + (uint32_t)r * x_read);
        const uint32_t ca = (uint32_t)cv * c_win + c_lane;
        const f4_t nc1 = *reinterpret_cast<const f4_t*>(q4_smem + ca);
        const f4_t c2 = *reinterpret_cast<const f4_t*>(q4_smem + ca + 16);
        const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
        // Two chains (even and odd steps) keep the matrix core busy.
        f4_t acc0 = nc1, acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t w8 = w[r] >> 8;
            // Step (r, 0): k (0,4,1,5) of the word's 8; step (r, 1): (2,6,3,7).
            const uint2 b0 = make_uint2((w[r] & m_lo) | g_lo, (w[r] & m_hi) | g_hi);
            const uint2 b1 = make_uint2((w8 & m_lo) | g_lo, (w8 & m_hi) | g_hi);
            acc0 = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(h4_t, make_uint2(xv[r].x, xv[r].y)),
                                                      __builtin_bit_cast(h4_t, b0), acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(h4_t, make_uint2(xv[r].z, xv[r].w)),
                                                      __builtin_bit_cast(h4_t, b1), acc1, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < NB; ++e) tot[e] = __builtin_fmaf(s, __builtin_fmaf(-z, c2[e], acc0[e] + acc1[e]), tot[e]);
        if (++cv == nwin) cv = 0;
        if (++cw_step == nwin) {
            // Quad done: add the 16 blocks' sums of each row (lanes 4 apart)
            // and write the quad's outputs.
#pragma unroll
            for (int e = 0; e < NB; ++e) {
                float t = tot[e];
                t += __shfl_xor(t, 4, 64);
                t += __shfl_xor(t, 8, 64);
                t += __shfl_xor(t, 16, 64);
                t += __shfl_xor(t, 32, 64);
                tot[e] = t;
            }
            const int64_t row = cq * 4 + j;
            if (blk == 0 && row < N) {
#pragma unroll
                for (int e = 0; e < NB; ++e)
                    if (e < B) a.Y[e * N + row] = float_to_half_bits_rne(tot[e]);
            }
            tot = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
            cw_step = 0;
            cq += nw;
        }
    };

    for (int k = 0; k < items; k += Q4_RING) {
#pragma unroll
        for (int d = 0; d < Q4_RING; ++d) {
            if (k + d < items) compute(ring[d]);
            next_load(ring[d]);
        }
    }
}

constexpr size_t kQ4MaxLds = 160 * 1024;

template <int NB>
hipError_t launch_q4_nb(const Q4Args& a, int num_cus, hipStream_t stream) {
    const size_t lds = q4_lds_bytes<NB>(a.nwin);
    if (lds > kQ4MaxLds) return hipErrorInvalidValue;
    static thread_local size_t cached_lds = (size_t)-1;
    static thread_local int cached_per_cu = 1;
    if (cached_lds != lds) {
        int v = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, gemm_q4_kernel<NB>, Q4_THREADS, lds) != hipSuccess ||
            v <= 0)
            v = 1;
        cached_lds = lds;
        cached_per_cu = v;
    }
    int64_t blocks = (a.nquads + Q4_WAVES - 1) / Q4_WAVES;
    const int64_t cap = (int64_t)num_cus * cached_per_cu;
    if (blocks > cap) blocks = cap;
    gemm_q4_kernel<NB><<<dim3((unsigned)blocks), dim3(Q4_THREADS), lds, stream>>>(a);
    return hipGetLastError();
}

int q4_rows(int64_t B) { return B <= 1 ? 1 : B <= 2 ? 2 : 4; }

}  // namespace

bool q4_supports(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits) {
    if (bits != 4 || B < 1 || B > 4 || K % 32 != 0 || group % 32 != 0 || K < 32 || N < 1) return false;
    if (K / group > Q4_HMAX) return false;
    if ((uint64_t)N * (uint64_t)(K / 2) > 0xFFFFFF00ull) return false;
    const int nwin = (int)((K + 511) / 512);
    const int nb = q4_rows(B);
    const size_t lds = nb == 1 ? q4_lds_bytes<1>(nwin) : nb == 2 ? q4_lds_bytes<2>(nwin) : q4_lds_bytes<4>(nwin);
    return lds <= kQ4MaxLds;
}

hipError_t launch_gemm_q4(const void* X, const void* codes, const void* scales, const void* zeros, void* Y,
                          int64_t B, int64_t K, int64_t N, int32_t group, int num_cus, hipStream_t stream) {
    if (!q4_supports(B, K, N, group, 4) || reinterpret_cast<uintptr_t>(scales) % 8 != 0 ||
        reinterpret_cast<uintptr_t>(zeros) % 8 != 0)
        return hipErrorInvalidValue;
    const uint64_t rpg = (uint64_t)(group / 32);
    Q4Args a{static_cast<const uint16_t*>(X), static_cast<const uint8_t*>(codes),
             static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros),
             static_cast<uint16_t*>(Y), B, N, K, (int32_t)((K + 511) / 512), (int32_t)(K / group), (N + 3) / 4,
             rpg == 1 ? 0u : (uint32_t)(((1ull << 32) + rpg - 1) / rpg)};
    switch (q4_rows(B)) {
        case 1: return launch_q4_nb<1>(a, num_cus, stream);
        case 2: return launch_q4_nb<2>(a, num_cus, stream);
    }
    return launch_q4_nb<4>(a, num_cus, stream);
}

}  // namespace wq
