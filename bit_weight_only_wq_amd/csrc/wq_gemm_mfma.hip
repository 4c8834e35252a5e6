// Skinny GEMM on the matrix cores (gfx950 MFMA) for batches past the GEMV regime:
// Y[B,N] = X[B,K] * dequant(W)[N,K]^T with fp16 operands and fp32 accumulation.
//
// Once 2B/w approaches the ridge ("Quantization & inference optimisation",
// "Bandwidth, not compute") the product is a real dense contraction, so it
// runs on v_mfma_f32_16x16x32_f16:
//   - a block owns 64 weight rows (4 waves x 16 rows) and BT batch columns;
//   - K is walked in stages of KS values; within a stage every lane streams one
//     128-bit code chunk per 128-k round of its row (4 lanes x 16 bytes = 64
//     contiguous bytes of each row per round), prefetched one stage ahead, and
//     turns it in registers into A operands holding 1024 + q exactly in fp16;
//   - the stage's X tile [BT x KS] is staged in LDS by the whole block
//     (128-bit loads issued a stage ahead), permuted into the order the codes
//     unpack in, with its per-round column sums; one barrier per stage;
//   - the group header is applied per 128-k round and accumulator through
//       sum_k (q - z) s x = s * (sum_k (1024 + q) x - (1024 + z) sum_k x)
//     ("the kernel reconstructs an approximate float from the integer and the
//     endpoints as it reads", "Quantization"), so the dequantized weight is
//     never rounded to fp16;
//   - per-row scales and zero points of the stage are staged in LDS as floats.
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
};

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

// Sum of 8 fp16 values in fp32 (products with 1.0 are exact).
__device__ __forceinline__ float sum8(uint4 v) {
    const h2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    float s = __builtin_amdgcn_fdot2(as_h2(v.x), one, 0.0f, false);
    s = __builtin_amdgcn_fdot2(as_h2(v.y), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(v.z), one, s, false);
    return __builtin_amdgcn_fdot2(as_h2(v.w), one, s, false);
}

// A 32-bit constant held in a VGPR, so that each unpack step is one
// v_and_or_b32 (gfx9 VOP3 instructions take no literal operand).
__device__ __forceinline__ uint32_t vgpr_const(uint32_t v) {
    uint32_t r;
    asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
    return r;
}

// A operand of k-step j from a lane's 16-byte chunk: fp16 pairs 1024 + q.
template <int BITS>
__device__ __forceinline__ h8_t a_operand(const uint4& cw, int j, uint32_t mask) {
    constexpr uint32_t MAGIC = 0x64006400u;
    uint4 a;
    if constexpr (BITS == 4) {
        const uint32_t w = j == 0 ? cw.x : j == 1 ? cw.y : j == 2 ? cw.z : cw.w;
        a.x = (w & mask) | MAGIC;
        a.y = ((w >> 4) & mask) | MAGIC;
        a.z = ((w >> 8) & mask) | MAGIC;
        a.w = ((w >> 12) & mask) | MAGIC;
    } else {
        const uint32_t w0 = j == 0 ? cw.x : cw.z;
        const uint32_t w1 = j == 0 ? cw.y : cw.w;
        a.x = (w0 & mask) | MAGIC;
        a.y = ((w0 >> 8) & mask) | MAGIC;
        a.z = (w1 & mask) | MAGIC;
        a.w = ((w1 >> 8) & mask) | MAGIC;
    }
    return __builtin_bit_cast(h8_t, a);
}

// Grid: x = 64-row tiles, y = BT-column tiles, z = K splits.  Split z covers
// stages [z*SPS, (z+1)*SPS); with one split the block writes Y (fp16), with
// several it writes fp32 partials part[z][b][n] that split_reduce_kernel sums
// in split order (deterministic).
template <int BITS, int BT, int KS>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(
    const uint16_t* __restrict__ X, const uint4* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros,
    uint16_t* __restrict__ Y, float* __restrict__ part, int64_t B, int64_t N, int64_t K,
    int32_t G, int64_t SPS) {
    typedef MfmaGeom<BITS> MG;
    constexpr int NCB = BT / 16;                      // 16-column blocks
    constexpr int RPS = KS / MG::KR;                  // rounds per stage
    constexpr int XROW = KS + 8;                      // padded LDS row (halfs)
    constexpr int SEGS = KS / 8;                      // 16-byte X vectors per column
    constexpr int SEGR = MG::KR / 8;                  // ... per column and round
    constexpr int NVEC = BT * SEGS;                   // X vectors per stage
    constexpr int VPT = NVEC >= 256 ? NVEC / 256 : 1; // X vectors per thread
    static_assert(NVEC % 256 == 0 || NVEC < 256, "X stage must tile the block");

    __shared__ __align__(16) uint16_t xs[2][BT][XROW];
    __shared__ float xsum[2][RPS][BT];
    __shared__ __align__(16) float2 hdr[2][RPS][64];  // (scale, 1024 + zero) per tile row

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int r16 = lane & 15;
    const int g4 = lane >> 4;
    const int64_t nb0 = (int64_t)blockIdx.x * 64;     // block's first row
    const int64_t n0 = nb0 + wave * 16;               // wave's first row
    const int64_t b0 = (int64_t)blockIdx.y * BT;
    const int64_t rowA = n0 + r16;
    const uint4* rowc = codes + (rowA < N ? rowA : N - 1) * (K / MG::VALS);
    const int64_t rounds = K / MG::KR;
    const int64_t st0 = (int64_t)blockIdx.z * SPS;
    const int64_t all_stages = (rounds + RPS - 1) / RPS;
    const int64_t st_end = st0 + SPS < all_stages ? st0 + SPS : all_stages;
    const int64_t ngrp = K / G;
    const uint32_t cmask = vgpr_const(BITS == 4 ? 0x000F000Fu : 0x00FF00FFu);

    // ---- global -> register loads of one stage --------------------------------
    // Every load is unconditional with a clamped address (rows past N, columns
    // past B, rounds past the end reread valid data whose results are masked),
    // so the compiler can count outstanding loads exactly and wait only for the
    // ones a step needs.
    const uint32_t last_round = (uint32_t)(rounds - 1);
    const uint32_t rpg = (uint32_t)(G / MG::KR);      // rounds per group
    auto load_codes = [&](int64_t st, uint4* cw) {
#pragma unroll
        for (int r = 0; r < RPS; ++r) {
            uint32_t rr = (uint32_t)(st * RPS + r);
            rr = rr < last_round ? rr : last_round;
            cw[r] = rowc[(int64_t)rr * 4 + g4];
        }
    };
    auto load_x = [&](int64_t st, uint4* xr) {
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int v = (tid + 256 * u) % NVEC;
            const int col = v / SEGS, seg = v % SEGS;
            int64_t k = st * KS + seg * 8;
            k = k < K - 8 ? k : K - 8;
            const int64_t b = b0 + col < B ? b0 + col : B - 1;
            xr[u] = *reinterpret_cast<const uint4*>(X + b * K + k);
        }
    };
    // A round past the end keeps a zero scale, so the step that computes it
    // (on clamped, finite data) adds nothing.
    auto load_hdr = [&](int64_t st, uint32_t& hs, uint32_t& hz) {
        const int row = tid & 63, r = (tid >> 6) % RPS;
        const int64_t n = nb0 + row < N ? nb0 + row : N - 1;
        const uint32_t rr0 = (uint32_t)(st * RPS + r);
        const uint32_t rr = rr0 < last_round ? rr0 : last_round;
        const int64_t gi = n * ngrp + rr / rpg;
        hs = scales[gi];
        hz = zeros[gi];
        if (rr0 > last_round) hs = 0u;
    };
    // ---- register -> LDS stores of one stage ----------------------------------
    auto store_stage = [&](int buf, const uint4* xr, uint32_t hs, uint32_t hz) {
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int v = tid + 256 * u;
            const int col = v / SEGS, seg = v % SEGS;
            // Threads of one (column, round) are SEGR adjacent lanes.
            const float s = group_sum<SEGR>(sum8(xr[u]));
            if (v < NVEC) {
                *reinterpret_cast<uint4*>(&xs[buf][col][seg * 8]) = permute8<BITS>(xr[u]);
                if (seg % SEGR == 0) xsum[buf][seg / SEGR][col] = s;
            }
        }
        if (tid < 64 * RPS)
            hdr[buf][tid >> 6][tid & 63] =
                make_float2(half_bits_to_float((uint16_t)hs), 1024.0f + half_bits_to_float((uint16_t)hz));
    };

    f4_t tot[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) tot[cb] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // ---- compute one stage from registers (codes) and LDS (X, header) ----------
    // All rounds' MFMA chains are issued first, into separate accumulators, and
    // the header corrections follow, so the matrix-core latency of one round
    // overlaps the issue of the next instead of stalling each round.
    auto compute = [&](int64_t st, int buf, const uint4* cw) {
        float2 h[RPS][4];
#pragma unroll
        for (int r = 0; r < RPS; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) h[r][i] = hdr[buf][r][wave * 16 + 4 * g4 + i];  // (s, 1024 + z)
        float xsv[RPS][NCB];
#pragma unroll
        for (int r = 0; r < RPS; ++r)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) xsv[r][cb] = xsum[buf][r][cb * 16 + r16];
        f4_t acc[RPS][NCB];
#pragma unroll
        for (int r = 0; r < RPS; ++r) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) acc[r][cb] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < MG::KSTEPS; ++j) {
                const h8_t a = a_operand<BITS>(cw[r], j, cmask);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    const h8_t bop = __builtin_bit_cast(
                        h8_t, *reinterpret_cast<const uint4*>(
                                  &xs[buf][cb * 16 + r16][r * MG::KR + g4 * MG::VALS + 8 * j]));
                    acc[r][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bop, acc[r][cb], 0, 0, 0);
                }
            }
        }
        // Accumulator lane layout: rows 4*g4 + i, column r16 of each block.
#pragma unroll
        for (int r = 0; r < RPS; ++r)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    tot[cb][i] = __builtin_fmaf(h[r][i].x, __builtin_fmaf(-h[r][i].y, xsv[r][cb], acc[r][cb][i]),
                                                tot[cb][i]);
    };

    // ---- pipeline ----------------------------------------------------------------
    // Codes run two stages ahead in a ring of three register sets; X and the
    // header run one stage ahead through registers into the other LDS buffer.
    // Issue order per stage (X, header, then codes) keeps the wait for X from
    // also waiting on the codes just issued.
    uint4 c0[RPS], c1[RPS], c2[RPS], xr[VPT];
    uint32_t hs, hz;
    load_x(st0, xr);
    load_hdr(st0, hs, hz);
    load_codes(st0, c0);
    load_codes(st0 + 1, c1);
    store_stage(0, xr, hs, hz);
    __syncthreads();

    // Every step loads, computes and stores unconditionally (loads past the
    // end are clamped and their rounds carry a zero scale): branch-free steps
    // let the compiler wait only for the loads each step consumes.
    auto step = [&](int64_t st, int buf, const uint4* cur, uint4* ahead2) {
        load_x(st + 1, xr);
        load_hdr(st + 1, hs, hz);
        load_codes(st + 2, ahead2);
        compute(st, buf, cur);
        store_stage(buf ^ 1, xr, hs, hz);
        __syncthreads();
    };
    for (int64_t st = st0; st < st_end; st += 6) {
        step(st, 0, c0, c2);
        if (st + 1 >= st_end) break;
        step(st + 1, 1, c1, c0);
        if (st + 2 >= st_end) break;
        step(st + 2, 0, c2, c1);
        if (st + 3 >= st_end) break;
        step(st + 3, 1, c0, c2);
        if (st + 4 >= st_end) break;
        step(st + 4, 0, c1, c0);
        if (st + 5 >= st_end) break;
        step(st + 5, 1, c2, c1);
    }

    float* pz = part ? part + (int64_t)blockIdx.z * B * N : nullptr;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int64_t col = b0 + cb * 16 + r16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t row = n0 + 4 * g4 + i;
            if (row < N && col < B) {
                if (pz) pz[col * N + row] = tot[cb][i];
                else Y[col * N + row] = float_to_half_bits_rne(tot[cb][i]);
            }
        }
    }
}

// Y = fp16(sum over splits of part[z]), splits added in order 0, 1, 2, ...
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part,
                                                           uint16_t* __restrict__ Y,
                                                           int64_t count, int splits) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= count) return;
    float s = part[i];
    for (int z = 1; z < splits; ++z) s += part[(int64_t)z * count + i];
    Y[i] = float_to_half_bits_rne(s);
}

template <int BITS, int BT, int KS>
hipError_t launch_bt(const void* X, const void* codes, const void* scales, const void* zeros,
                     void* Y, int64_t B, int64_t K, int64_t N, int32_t G, int num_cus,
                     hipStream_t stream) {
    constexpr int RPS = KS / MfmaGeom<BITS>::KR;
    const int64_t tiles = ((N + 63) / 64) * ((B + BT - 1) / BT);
    const int64_t stages = (K / MfmaGeom<BITS>::KR + RPS - 1) / RPS;
    // Split K until about three blocks per compute unit are in flight, keeping
    // at least two stages per split so that loads overlap compute.
    int64_t want = (3 * (int64_t)num_cus + tiles - 1) / tiles;
    int64_t max_split = stages / 2 > 0 ? stages / 2 : 1;
    if (want > max_split) want = max_split;
    if (want < 1) want = 1;
    const int64_t sps = (stages + want - 1) / want;
    const int64_t splits = (stages + sps - 1) / sps;
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((B + BT - 1) / BT), (unsigned)splits);
    float* part = nullptr;
    if (splits > 1) {
        uint32_t* unused = nullptr;
        hipError_t e = workspace_get(stream, 0, (size_t)splits * B * N * sizeof(float), &unused, &part);
        if (e != hipSuccess) return e;
    }
    gemm_mfma_kernel<BITS, BT, KS><<<grid, dim3(256), 0, stream>>>(
        static_cast<const uint16_t*>(X), static_cast<const uint4*>(codes),
        static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros),
        static_cast<uint16_t*>(Y), part, B, N, K, G, sps);
    hipError_t e = hipGetLastError();
    if (splits > 1 && e == hipSuccess) {
        const int64_t count = B * N;
        split_reduce_kernel<<<dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream>>>(
            part, static_cast<uint16_t*>(Y), count, (int)splits);
        e = hipGetLastError();
    }
    return e;
}

template <int BITS>
hipError_t launch_bits(const void* X, const void* codes, const void* scales, const void* zeros,
                       void* Y, int64_t B, int64_t K, int64_t N, int32_t G, int cus,
                       hipStream_t st) {
    constexpr int KR = MfmaGeom<BITS>::KR;
    if (B <= 16) return launch_bt<BITS, 16, 2 * KR>(X, codes, scales, zeros, Y, B, K, N, G, cus, st);
    if (B <= 32) return launch_bt<BITS, 32, 2 * KR>(X, codes, scales, zeros, Y, B, K, N, G, cus, st);
    return launch_bt<BITS, 64, 2 * KR>(X, codes, scales, zeros, Y, B, K, N, G, cus, st);
}

}  // namespace

bool mfma_supports(int64_t K, int32_t group, int32_t bits) {
    const int kr = bits == 4 ? MfmaGeom<4>::KR : MfmaGeom<8>::KR;
    return (bits == 4 || bits == 8) && group % kr == 0 && K % kr == 0;
}

hipError_t launch_gemm_mfma(const void* X, const void* codes, const void* scales,
                            const void* zeros, void* Y, int64_t B, int64_t K, int64_t N,
                            int32_t group, int32_t bits, int num_cus, hipStream_t stream) {
    if (xr_supports(B, K, group, bits))
        return launch_gemm_xr(X, codes, scales, zeros, Y, B, K, N, group, bits, num_cus, stream);
    if (bits == 4) return launch_bits<4>(X, codes, scales, zeros, Y, B, K, N, group, num_cus, stream);
    return launch_bits<8>(X, codes, scales, zeros, Y, B, K, N, group, num_cus, stream);
}

}  // namespace wq
