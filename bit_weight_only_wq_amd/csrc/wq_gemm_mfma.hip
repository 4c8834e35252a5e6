// Tiled product on the matrix cores (gfx950 MFMA) for batches past 16:
// Y[B,N] = X[B,K] * dequant(W)[N,K]^T with fp16 operands and fp32 accumulation.
//
// Once 2B/w approaches the ridge ("Quantization & inference optimisation",
// "Bandwidth, not compute") the product is a real dense contraction, so it
// runs on v_mfma_f32_16x16x32_f16 with X as the A operand (16 batch rows) and
// the weights as the B operand (16 weight rows):
//   - a block owns 64*RB weight rows (4 waves x RB tiles of 16 rows) and BT
//     batch columns and walks K in stages of KS values; a wave's RB row tiles
//     share every X operand it reads from LDS;
//   - every lane streams one 128-bit code chunk per 128-k round of its weight
//     row (4 lanes x 16 bytes = 64 contiguous bytes of the row per round),
//     two stages ahead in a ring of registers;
//   - the stage's X tile [BT x KS] is staged in LDS by the whole block (loads
//     issued a stage ahead), permuted into the order the codes unpack in; the
//     stage's group headers of the block's 64 rows go to LDS beside it; one
//     barrier per stage;
//   - each chunk is dequantized in registers ("the kernel reconstructs an
//     approximate float from the integer and the endpoints as it reads",
//     "Quantization") to fp16 (q - z) * s / 2 and reused for all BT columns:
//       (w & 0x000F000F) | 0x60006000 = (512 + q0/2, 512 + q4/2), exact
//       (w & 0x00F000F0) | 0x50005000 = ( 32 + q1/2,  32 + q5/2), exact
//     minus (512 + z/2) or (32 + z/2), times s, rounded once; the factor 1/2
//     keeps every operand finite for any fp16 weights and is undone on the
//     fp32 result.  The k order of an operand is (0,4,1,5,2,6,3,7) within each
//     8 k (8-bit codes: (0,2,1,3) within each 4 k), and X is permuted to match.
// Requires G % KR == 0 (KR = 128 k for 4-bit, 64 k for 8-bit).
#include "wq_device.h"
#include "wq_launch.h"
#include "wq_mfma_dq.h"

namespace wq {

namespace {

using dq::DqConsts;
using dq::dequant;
using dq::permute8;

template <int BITS>
struct MfmaGeom {
    static constexpr int VALS = 128 / BITS;    // codes per 16-byte lane load
    static constexpr int KR = 4 * VALS;        // k per round (4 lane groups)
    static constexpr int KSTEPS = KR / 32;     // 16x16x32 MFMAs per round per column block
};

// Grid: x = (64*RB)-row tiles, y = BT-column tiles, z = K splits.  Split z covers
// stages [z*SPS, (z+1)*SPS) (SPS a multiple of 8); with one split the block writes Y (fp16), with
// several it writes fp32 partials part[z][b][n] that split_reduce_kernel sums
// in split order (deterministic).
template <int BITS, int BT, int KS, int RB, bool HV>
__global__ __launch_bounds__(256, (BT == 64 && RB == 2) ? 3 : 1) void gemm_mfma_kernel(
    const uint16_t* __restrict__ X, const uint4* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros,
    uint16_t* __restrict__ Y, float* __restrict__ part, int64_t B, int64_t N, int64_t K,
    int32_t G, int64_t SPS) {
    typedef MfmaGeom<BITS> MG;
    constexpr int NCB = BT / 16;                      // 16-column (batch) blocks
    constexpr int RPS = KS / MG::KR;                  // rounds per stage
    constexpr int XROW = KS + 8;                      // padded LDS row (halfs)
    constexpr int SEGS = KS / 8;                      // 16-byte X vectors per column
    constexpr int NVEC = BT * SEGS;                   // X vectors per stage
    constexpr int VPT = NVEC >= 256 ? NVEC / 256 : 1; // X vectors per thread
    static_assert(NVEC % 256 == 0 || NVEC < 256, "X stage must tile the block");

    __shared__ __align__(16) uint16_t xs[2][BT][XROW];
    constexpr int BR = 64 * RB;                       // block rows
    __shared__ uint32_t hdr[2][RPS][BR];   // (scale | zero << 16) fp16 bits per block row

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int r16 = lane & 15;
    const int g4 = lane >> 4;
    const int64_t nb0 = (int64_t)blockIdx.x * BR;     // block's first row
    const int64_t n0 = nb0 + wave * 16 * RB;          // wave's first row
    const int64_t b0 = (int64_t)blockIdx.y * BT;
    // This lane's weight row in each of the wave's row tiles (B operand).
    const uint4* rowc[RB];
#pragma unroll
    for (int t = 0; t < RB; ++t) {
        const int64_t rowB = n0 + 16 * t + r16;
        rowc[t] = codes + (rowB < N ? rowB : N - 1) * (K / MG::VALS);
    }
    const int64_t rounds = K / MG::KR;
    const int64_t st0 = (int64_t)blockIdx.z * SPS;
    const int64_t all_stages = (rounds + RPS - 1) / RPS;
    const int64_t st_end = st0 + SPS < all_stages ? st0 + SPS : all_stages;
    const int64_t ngrp = K / G;
    const DqConsts cst = BITS == 4
        ? DqConsts{vgpr_const(0x000F000Fu), vgpr_const(0x00F000F0u), vgpr_const(0x60006000u), vgpr_const(0x50005000u)}
        : DqConsts{vgpr_const(0x00FF00FFu), 0u, vgpr_const(0x60006000u), 0u};
    const h2_t zmul = {(_Float16)0.5f, (_Float16)0.5f};
    const h2_t zadd = {(_Float16)512.0f, (_Float16)32.0f};

    // ---- global -> register loads of one stage --------------------------------
    // Every load is unconditional with a clamped address (rows past N, columns
    // past B, rounds past the end reread valid data); X columns past B and k
    // past K are zeroed at the LDS store, so clamped rounds add nothing.
    const uint32_t last_round = (uint32_t)(rounds - 1);
    const uint32_t rpg = (uint32_t)(G / MG::KR);      // rounds per group
    auto load_codes = [&](int64_t st, uint4* cw) {     // cw[r * RB + t]
#pragma unroll
        for (int r = 0; r < RPS; ++r) {
            uint32_t rr = (uint32_t)(st * RPS + r);
            rr = rr < last_round ? rr : last_round;
#pragma unroll
            for (int t = 0; t < RB; ++t) cw[r * RB + t] = rowc[t][(int64_t)rr * 4 + g4];
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
    // Headers, HV (one group per round, 8 | groups per row, aligned arrays):
    // each lane loads the 8 groups of a turn (8 rounds) of its own rows as
    // two 128-bit loads per row tile, one turn ahead.  Otherwise the block
    // stages each stage's headers in LDS.
    int64_t hrow[RB];
#pragma unroll
    for (int t = 0; t < RB; ++t) {
        const int64_t rowB = n0 + 16 * t + r16;
        hrow[t] = (rowB < N ? rowB : N - 1) * ngrp;
    }
    uint4 hsc[RB], hzc[RB], hsn[RB], hzn[RB];
    auto load_hdr_turn = [&](int64_t round_start) {
        int64_t ga = round_start;
        ga = ga + 8 <= rounds ? ga : rounds - 8;
#pragma unroll
        for (int t = 0; t < RB; ++t) {
            hsn[t] = *reinterpret_cast<const uint4*>(scales + hrow[t] + ga);
            hzn[t] = *reinterpret_cast<const uint4*>(zeros + hrow[t] + ga);
        }
    };
    auto load_hdr = [&](int64_t st, uint32_t& hs, uint32_t& hz) {
        if constexpr (HV) return;
        const int row = tid % BR, r = (tid / BR) % RPS;
        const int64_t n = nb0 + row < N ? nb0 + row : N - 1;
        uint32_t rr = (uint32_t)(st * RPS + r);
        rr = rr < last_round ? rr : last_round;
        const int64_t gi = n * ngrp + rr / rpg;
        hs = scales[gi];
        hz = zeros[gi];
    };
    // ---- register -> LDS stores of one stage ----------------------------------
    auto store_stage = [&](int64_t st, int buf, const uint4* xr, uint32_t hs, uint32_t hz) {
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int v = tid + 256 * u;
            const int col = v / SEGS, seg = v % SEGS;
            const int64_t k = st * KS + seg * 8;
            // Zero by an opaque mask, not a select: a select of loaded data
            // lets the compiler move the load into a branch at this point,
            // after the code loads of later stages, and wait for all of them.
            uint32_t m = (b0 + col < B && k < K && st < st_end) ? 0xFFFFFFFFu : 0u;
            asm volatile("" : "+v"(m));
            const uint4 x = {xr[u].x & m, xr[u].y & m, xr[u].z & m, xr[u].w & m};
            if (NVEC % 256 == 0 || v < NVEC)
                *reinterpret_cast<uint4*>(&xs[buf][col][seg * 8]) = permute8<BITS>(x);
        }
        if (!HV && tid < BR * RPS) hdr[buf][tid / BR][tid % BR] = hs | (hz << 16);
    };

    f4_t acc[RB][NCB];
#pragma unroll
    for (int t = 0; t < RB; ++t)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[t][cb] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // ---- compute one stage from registers (codes) and LDS (X, header) ----------
    // Each k-step's dequantized codes feed all NCB column blocks, and each X
    // operand read from LDS feeds all RB row tiles.
    // kt: this stage's position in its turn of 8 rounds (HV header index).
    auto compute = [&](int buf, const uint4* cw, int kt) {
#pragma unroll
        for (int r = 0; r < RPS; ++r) {
            h2_t nz[RB], ss[RB];
#pragma unroll
            for (int t = 0; t < RB; ++t) {
                uint32_t zb, sb;
                if constexpr (HV) {
                    const int i = (kt * RPS + r) & 7;
                    const uint32_t ws = i < 4 ? (i < 2 ? hsc[t].x : hsc[t].y) : (i < 6 ? hsc[t].z : hsc[t].w);
                    const uint32_t wz = i < 4 ? (i < 2 ? hzc[t].x : hzc[t].y) : (i < 6 ? hzc[t].z : hzc[t].w);
                    const uint32_t sel = (i & 1) ? 0x07060706u : 0x05040504u;   // half i&1, twice
                    sb = __builtin_amdgcn_perm(ws, ws, sel);
                    zb = __builtin_amdgcn_perm(wz, wz, sel);
                } else {
                    const uint32_t h = hdr[buf][r][wave * 16 * RB + 16 * t + r16];
                    zb = (h >> 16) | (h & 0xFFFF0000u);
                    sb = (h & 0xFFFFu) | (h << 16);
                }
                nz[t] = as_h2(zb) * zmul + zadd;     // (512 + z/2, 32 + z/2)
                ss[t] = as_h2(sb);
            }
#pragma unroll
            for (int j = 0; j < MG::KSTEPS; ++j) {
                h8_t bop[RB];
#pragma unroll
                for (int t = 0; t < RB; ++t) bop[t] = dequant<BITS>(cw[r * RB + t], j, cst, nz[t], ss[t]);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    const h8_t aop = __builtin_bit_cast(
                        h8_t, *reinterpret_cast<const uint4*>(
                                  &xs[buf][cb * 16 + r16][r * MG::KR + g4 * MG::VALS + 8 * j]));
#pragma unroll
                    for (int t = 0; t < RB; ++t)
                        acc[t][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop[t], acc[t][cb], 0, 0, 0);
                }
            }
        }
    };

    // ---- pipeline ----------------------------------------------------------------
    // Codes run two stages ahead in a ring of four register sets; X (and, in
    // the LDS header mode, the header) run one stage ahead through registers
    // into the other LDS buffer; HV headers run one 8-round turn ahead.
    uint4 cr[4][RPS * RB], xr[VPT];
    uint32_t hs = 0u, hz = 0u;
    if constexpr (HV) load_hdr_turn(st0 * RPS);
    load_x(st0, xr);
    load_hdr(st0, hs, hz);
    load_codes(st0, cr[0]);
    load_codes(st0 + 1, cr[1]);
    store_stage(st0, 0, xr, hs, hz);
    __syncthreads();

    constexpr int STT = 8 / RPS;                      // stages per header turn
    // The stage count is padded to whole 8-step bodies, so the loop has no
    // exits inside it; padded stages meet zero X and add nothing.
    for (int64_t st = st0; st < st_end; st += 8) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if constexpr (HV) {
                if (k % STT == 0) {
#pragma unroll
                    for (int t = 0; t < RB; ++t) {
                        hsc[t] = hsn[t];
                        hzc[t] = hzn[t];
                    }
                    load_hdr_turn((st + k) * RPS + 8);
                }
            }
            load_x(st + k + 1, xr);
            load_hdr(st + k + 1, hs, hz);
            load_codes(st + k + 2, cr[(k + 2) & 3]);
            // Keep the next stage's loads ahead of this stage's math: left to
            // itself the scheduler sinks them to their use and the X tile's
            // latency is paid in full every stage.
            __builtin_amdgcn_sched_barrier(0);
            compute(k & 1, cr[k & 3], k % STT);
            store_stage(st + k + 1, (k & 1) ^ 1, xr, hs, hz);
            // The next stage's X (and headers) are in LDS once this block's
            // LDS writes are done; the code loads stay in flight (a full
            // workgroup barrier would wait for them too, every stage).
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0) only
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
    }

    // Accumulator lane layout: batch rows 4*g4 + i of column block cb, weight
    // row r16 of tile t; the dequantized operand carried a factor 1/2.
    float* pz = part ? part + (int64_t)blockIdx.z * B * N : nullptr;
#pragma unroll
    for (int t = 0; t < RB; ++t) {
        const int64_t row = n0 + 16 * t + r16;
        if (row >= N) continue;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t col = b0 + cb * 16 + 4 * g4 + i;
                if (col < B) {
                    const float v = 2.0f * acc[t][cb][i];
                    if (pz) pz[col * N + row] = v;
                    else Y[col * N + row] = float_to_half_bits_rne(v);
                }
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

// The same sums four outputs per thread (count % 4 == 0, Y 8-byte aligned):
// 16-byte partial loads and one 8-byte store.
__global__ __launch_bounds__(256) void split_reduce4_kernel(const float4* __restrict__ part,
                                                            uint2* __restrict__ Y,
                                                            int64_t count4, int splits) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= count4) return;
    float4 s = part[i];
    for (int z = 1; z < splits; ++z) {
        const float4 v = part[(int64_t)z * count4 + i];
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    Y[i] = make_uint2((uint32_t)float_to_half_bits_rne(s.x) | ((uint32_t)float_to_half_bits_rne(s.y) << 16),
                      (uint32_t)float_to_half_bits_rne(s.z) | ((uint32_t)float_to_half_bits_rne(s.w) << 16));
}

template <int BITS, int BT, int KS, int RB>
hipError_t launch_bt(const void* X, const void* codes, const void* scales, const void* zeros,
                     void* Y, int64_t B, int64_t K, int64_t N, int32_t G, int num_cus,
                     const Scratch& ws, hipStream_t stream) {
    constexpr int RPS = KS / MfmaGeom<BITS>::KR;
    constexpr int BR = 64 * RB;
    const int64_t tiles = ((N + BR - 1) / BR) * ((B + BT - 1) / BT);
    const int64_t stages = (K / MfmaGeom<BITS>::KR + RPS - 1) / RPS;
    // Split K until about three blocks per compute unit are in flight (two
    // measured 11-13 % slower on the 7B-class down projection at B = 32 and
    // 64, 6 % at B = 128 on 8192 x 8192), keeping at least two stages per
    // split so that loads overlap compute; the fp32 partials of the splits go
    // to the caller's scratch (one split without).
    int64_t want = (3 * (int64_t)num_cus + tiles - 1) / tiles;
    int64_t max_split = stages / 2 > 0 ? stages / 2 : 1;
    if (want > max_split) want = max_split;
    if (want < 1) want = 1;
    if (!ws.sizing() && !ws.ptr) want = 1;
    int64_t sps = (stages + want - 1) / want;
    sps = (sps + 7) / 8 * 8;                          // whole 8-step loop bodies
    const int64_t splits = (stages + sps - 1) / sps;
    if (ws.sizing()) {
        ws.want(splits > 1 ? (size_t)splits * B * N * sizeof(float) : 0);
        return hipSuccess;
    }
    const dim3 grid((unsigned)((N + BR - 1) / BR), (unsigned)((B + BT - 1) / BT), (unsigned)splits);
    float* part = splits > 1 ? static_cast<float*>(ws.ptr) : nullptr;
    const bool hv = G == MfmaGeom<BITS>::KR && (K / G) % 8 == 0 &&
                    reinterpret_cast<uintptr_t>(scales) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(zeros) % 16 == 0;
    if (hv)
        gemm_mfma_kernel<BITS, BT, KS, RB, true><<<grid, dim3(256), 0, stream>>>(
            static_cast<const uint16_t*>(X), static_cast<const uint4*>(codes),
            static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros),
            static_cast<uint16_t*>(Y), part, B, N, K, G, sps);
    else
        gemm_mfma_kernel<BITS, BT, KS, RB, false><<<grid, dim3(256), 0, stream>>>(
            static_cast<const uint16_t*>(X), static_cast<const uint4*>(codes),
            static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros),
            static_cast<uint16_t*>(Y), part, B, N, K, G, sps);
    hipError_t e = hipGetLastError();
    if (splits > 1 && e == hipSuccess) {
        const int64_t count = B * N;
        if (count % 4 == 0 && reinterpret_cast<uintptr_t>(Y) % 8 == 0) {
            const int64_t count4 = count / 4;
            split_reduce4_kernel<<<dim3((unsigned)((count4 + 255) / 256)), dim3(256), 0, stream>>>(
                reinterpret_cast<const float4*>(part), static_cast<uint2*>(Y), count4, (int)splits);
        } else {
            split_reduce_kernel<<<dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream>>>(
                part, static_cast<uint16_t*>(Y), count, (int)splits);
        }
        e = hipGetLastError();
    }
    return e;
}

// Tall matrices give every compute unit enough 128-row tiles: two row tiles
// per wave halve the LDS reads per weight.  Shorter ones keep 64-row tiles.
// Past 16 columns every variant stages one 128-k round per step, which keeps
// enough K-splits for short matrices (measured on the 7B-class shapes).
template <int BITS>
hipError_t launch_bits(const void* X, const void* codes, const void* scales, const void* zeros,
                       void* Y, int64_t B, int64_t K, int64_t N, int32_t G, int cus,
                       const Scratch& ws, hipStream_t st) {
    constexpr int KR = MfmaGeom<BITS>::KR;
    const bool tall = N >= 64 * (int64_t)cus;
    if (B <= 16) return launch_bt<BITS, 16, 2 * KR, 1>(X, codes, scales, zeros, Y, B, K, N, G, cus, ws, st);
    if (B <= 32) {
        if (tall) return launch_bt<BITS, 32, KR, 2>(X, codes, scales, zeros, Y, B, K, N, G, cus, ws, st);
        return launch_bt<BITS, 32, KR, 1>(X, codes, scales, zeros, Y, B, K, N, G, cus, ws, st);
    }
    // Past 32 columns, 128-row tiles also pay when they alone give one to two
    // blocks per CU (B = 256 on 8192 x 8192 and 11008 x 4096: 7-10 % faster;
    // B = 512 on 8192 x 8192 and 4096 x 4096: 3-6 %; fewer or more tiles than
    // that measured equal or slower).
    const int64_t tiles128 = ((N + 127) / 128) * ((B + 63) / 64);
    if (tall || (tiles128 >= cus && tiles128 <= 2 * (int64_t)cus))
        return launch_bt<BITS, 64, KR, 2>(X, codes, scales, zeros, Y, B, K, N, G, cus, ws, st);
    return launch_bt<BITS, 64, KR, 1>(X, codes, scales, zeros, Y, B, K, N, G, cus, ws, st);
}

}  // namespace

bool mfma_supports(int64_t K, int32_t group, int32_t bits) {
    const int kr = bits == 4 ? MfmaGeom<4>::KR : MfmaGeom<8>::KR;
    return (bits == 4 || bits == 8) && group % kr == 0 && K % kr == 0;
}

static bool aligned_to(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

bool q4_takes(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits, const void* scales,
              const void* zeros) {
    return q4_supports(B, K, N, group, bits) && N >= 1024 && aligned_to(scales, 8) && aligned_to(zeros, 8);
}

// The quad-stream kernel takes B <= 4 on tall matrices (past 4 batch rows
// the 16-row kernels do more work per code byte for less).
bool qs_takes(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits, const void* scales,
              const void* zeros) {
    return B <= 4 && qs_supports(B, K, N, group, bits) && N >= 1024 && aligned_to(scales, 16) &&
           aligned_to(zeros, 16);
}

// The tile-stream kernel takes B <= 16 on matrices of at least 2048 rows
// (where the quad and K-split-wave kernels do not).
bool ts_takes(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits, const void* scales,
              const void* zeros) {
    return ts_supports(B, K, N, group, bits) && N >= 2048 && aligned_to(scales, 8) && aligned_to(zeros, 8);
}

bool mfma_path_takes(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits, const void* scales,
                     const void* zeros) {
    return qs_takes(B, K, N, group, bits, scales, zeros) || q4_takes(B, K, N, group, bits, scales, zeros) ||
           mfma_supports(K, group, bits);
}

hipError_t launch_gemm_mfma(const void* X, const void* codes, const void* scales,
                            const void* zeros, void* Y, int64_t B, int64_t K, int64_t N,
                            int32_t group, int32_t bits, int num_cus, const Scratch& ws,
                            hipStream_t stream) {
    // Tall matrices at B <= 4 take the quad-stream kernel (groups of 64 and
    // more) or the quad-row kernel; from B = 5 to 64, matrices of at least
    // 1.8 16-row tiles per compute unit take the K-split-wave kernel, and
    // up to B = 16 the others take the tile-stream kernel or (with header
    // arrays it cannot stage) the streaming 16-row kernel; none of them needs
    // scratch.
    if (qs_takes(B, K, N, group, bits, scales, zeros)) {
        if (ws.sizing()) return hipSuccess;
        return launch_gemm_qs(X, codes, scales, zeros, Y, B, K, N, group, num_cus, stream);
    }
    if (q4_takes(B, K, N, group, bits, scales, zeros)) {
        if (ws.sizing()) return hipSuccess;
        return launch_gemm_q4(X, codes, scales, zeros, Y, B, K, N, group, num_cus, stream);
    }
    if (kw_takes(B, K, N, group, bits, false, X, scales, zeros, num_cus)) {
        if (ws.sizing()) return hipSuccess;
        return launch_gemm_kw(X, codes, scales, zeros, Y, B, K, N, group, bits, false, num_cus, stream);
    }
    if (ts_takes(B, K, N, group, bits, scales, zeros)) {
        if (ws.sizing()) return hipSuccess;
        return launch_gemm_ts(X, codes, scales, zeros, Y, B, K, N, group, num_cus, stream);
    }
    if (sk_supports(B, K, N, group, bits) && (N + 15) / 16 >= (int64_t)num_cus / 2) {
        if (ws.sizing()) return hipSuccess;
        return launch_gemm_sk(X, codes, scales, zeros, Y, B, K, N, group, num_cus, stream);
    }
    // The X-resident kernel takes its shapes, but without scratch only when
    // one K-slice holds all of X (its slices meet in fp32 partials).
    const bool no_scratch = !ws.sizing() && !ws.ptr;
    if (xr_supports(B, K, group, bits) && (!no_scratch || xr_single_slice(B, K, bits))) {
        const XrProduct p{X, codes, scales, zeros, Y, K, N, group};
        return launch_gemm_xr_many(&p, 1, B, bits, num_cus, ws, stream);
    }
    if (bits == 4) return launch_bits<4>(X, codes, scales, zeros, Y, B, K, N, group, num_cus, ws, stream);
    return launch_bits<8>(X, codes, scales, zeros, Y, B, K, N, group, num_cus, ws, stream);
}

}  // namespace wq
