// Small-batch decode GEMV (gfx950, VALU): Y[B,N] = X[B,K] * dequant(W)[N,K]^T.
//
// The decode step is bandwidth-bound at small batch ("Quantization & inference
// optimisation", "Bandwidth, not compute": 2B/w FLOP per byte), so this path is
// built to stream the packed weights once at full HBM rate:
//   - each thread owns a fixed set of 16-byte code chunks of every row it
//     visits (chunk c, c+TG, c+2TG, ... of the row), read with one 128-bit
//     load each; TG consecutive threads cover a row, so a wave's loads are
//     contiguous;
//   - the matching X values live in LDS for the whole kernel, already
//     permuted into the order the codes unpack in, so X is read from HBM once
//     per block;
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

// X positions (within a chunk) of fp16 pair p of word j, in unpack order.
// 4-bit: pairs (q0,q4) (q1,q5) (q2,q6) (q3,q7) of each 8-code word.
// 8-bit: pairs (q0,q2) (q1,q3) of each 4-code word.
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

// Wave-scope ordering of LDS accesses made by the lanes of one wave.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Buffer resource word 3 for raw (unformatted, unswizzled) gfx9 buffers.
constexpr int kBufferWord3 = 0x00020000;

// 128-bit streaming load through a buffer resource (nt cache policy).
__device__ __forceinline__ uint4 load_stream_buf(__amdgpu_buffer_rsrc_t rsrc, uint32_t off) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u t = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)off, 0, 2);
    return make_uint4(t.x, t.y, t.z, t.w);
}

// Sum over aligned groups of W lanes (W in {16, 32, 64}), complete in the last
// lane of each group: row sums by DPP within 16 lanes, then row broadcasts
// (lane 15 of a row into the next row, lane 31 into rows 2 and 3) instead of
// cross-row shuffles through LDS.
template <int W>
__device__ __forceinline__ float group_total_last(float v) {
    v = group_sum<16>(v);
    if constexpr (W >= 32)
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
    if constexpr (W >= 64)
        v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false));
    return v;
}

// X lives in LDS for the whole kernel as one record per (batch row, chunk):
//   QPC uint4   the chunk's fp16 X pairs in the order its codes unpack;
//   float2      (K0, xT): xT = sum of the chunk's X, and K0 the constant that
//               the unpack offsets contribute (1024 per unscaled code, 64 per
//               code unpacked times 16, after the 1/16 rescale);
//   float2      padding, so records are 80 (4-bit) or 48 (8-bit) bytes apart
//               and the 16-byte reads of consecutive threads avoid bank clashes.
// Then for a chunk, with pa accumulated from -K0 over the unscaled codes and
// pb over the scaled ones:  sum_k (q_k - z) x_k = pa + pb/16 - z * xT.
template <int BITS, int NB, int TG, int CPT>
__global__ __launch_bounds__(256) void gemv_kernel(
    const uint16_t* __restrict__ X, const uint4* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros,
    uint16_t* __restrict__ Y, int64_t B, int64_t N, int64_t K, int32_t G) {
    typedef ChunkGeom<BITS> CG;
    constexpr int QPC = CG::PAIRS / 4;          // uint4 of X pairs per chunk
    constexpr int REC = QPC + 1;                // uint4 per X record
    constexpr int RPB = 256 / TG;               // rows per block pass
    constexpr int WPR = TG > 64 ? TG / 64 : 1;  // waves per row
    constexpr uint32_t MAGIC = 0x64006400u;     // fp16 1024.0 in both halves
    extern __shared__ __align__(16) unsigned char smem[];
    // Per row slot, (scale, zero) of the row's groups as floats.  A row has at
    // most TG*CPT chunks, hence at most TG*CPT groups.
    __shared__ float2 hdr[RPB * TG * CPT];
    __shared__ float red[(TG > 64) ? 4 * NB : 1];

    const int tid = threadIdx.x;
    const int rs = tid / TG;           // row slot in the pass
    const int tl = tid % TG;           // thread within the row
    const int C = (int)(K / CG::VALS); // chunks per row
    const int64_t ngrp = K / G;        // groups per row
    const int cpg = G / CG::VALS;      // chunks per group
    const int64_t b0 = (int64_t)blockIdx.y * NB;
    const int nb = (int)((B - b0) < NB ? (B - b0) : NB);
    const int64_t passes = (N + RPB - 1) / RPB;
    float2* row_hdr = hdr + rs * (TG * CPT);
    uint4* xrec = reinterpret_cast<uint4*>(smem);
    const uint32_t m_lo = vgpr_const(BITS == 4 ? 0x000F000Fu : 0x00FF00FFu);
    const uint32_t m_hi = vgpr_const(0x00F000F0u);

    // This thread's chunks: clamped index, group and liveness (ragged rows).
    int cidx[CPT], gidx[CPT];
    bool cin[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int c = tl + TG * i;
        cin[i] = c < C;
        cidx[i] = c < C ? c : C - 1;
        gidx[i] = cidx[i] / cpg;
    }

    // Global loads of one pass: this thread's code chunks of row n, and the
    // header entries tl, tl+TG, ... of that row (coalesced 2-byte loads, kept
    // in separate registers so that nothing waits on them before use).
    // Branches are block-uniform; per-lane bounds clamp the address instead
    // (a clamped chunk is loaded but later weighted by a zero scale).
    int hidx[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int64_t g = tl + (int64_t)TG * i;
        hidx[i] = (int)(g < ngrp ? g : ngrp - 1);
    }
    // Every load is unconditional (passes past the end reread the last row,
    // chunks and header entries past the row's end reread its last ones), so
    // the compiler can count the loads in flight exactly and the next pass's
    // loads stay outstanding while the current pass computes.
    auto load_pass = [&](int64_t pass, uint4* w, uint32_t* hs, uint32_t* hz) {
        int64_t n = pass * RPB + rs;
        n = n < N ? n : N - 1;
        const uint4* rowc = codes + n * C;
        const uint16_t* rows = scales + n * ngrp;
        const uint16_t* rowz = zeros + n * ngrp;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            w[i] = load_stream(rowc + cidx[i]);
            hs[i] = rows[hidx[i]];
            hz[i] = rowz[hidx[i]];
        }
    };

    int64_t pass = blockIdx.x;
    uint4 wA[CPT], wB[CPT];
    uint32_t sA[CPT], sB[CPT], zA[CPT], zB[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        wA[i] = wB[i] = make_uint4(0u, 0u, 0u, 0u);
        sA[i] = sB[i] = zA[i] = zB[i] = 0u;
    }
    load_pass(pass, wA, sA, zA);        // first codes in flight before the X setup

    // ---- X records into LDS (whole block) ------------------------------------
    for (int e = tid; e < NB * C; e += 256) {
        const int b = e / C, c = e % C;
        uint16_t xv[CG::VALS];
        if (b < nb) {
            const uint4* src = reinterpret_cast<const uint4*>(X + (b0 + b) * K + (int64_t)c * CG::VALS);
#pragma unroll
            for (int v = 0; v < CG::VALS / 8; ++v) {
                uint4 u = src[v];
                uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    xv[8 * v + 2 * q] = (uint16_t)(ww[q] & 0xFFFFu);
                    xv[8 * v + 2 * q + 1] = (uint16_t)(ww[q] >> 16);
                }
            }
        } else {
#pragma unroll
            for (int v = 0; v < CG::VALS; ++v) xv[v] = 0;
        }
        uint32_t pr[CG::PAIRS];
        float sa = 0.0f, sb = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int p = 0; p < CG::PAIRS_PER_WORD; ++p) {
                int a, bb;
                pair_positions<BITS>(j, p, a, bb);
                pr[j * CG::PAIRS_PER_WORD + p] = (uint32_t)xv[a] | ((uint32_t)xv[bb] << 16);
                const float t = half_bits_to_float(xv[a]) + half_bits_to_float(xv[bb]);
                if (BITS == 4 && (p & 1)) sb += t;
                else sa += t;
            }
        uint4* rec = xrec + (size_t)e * REC;
#pragma unroll
        for (int r = 0; r < QPC; ++r)
            rec[r] = make_uint4(pr[4 * r], pr[4 * r + 1], pr[4 * r + 2], pr[4 * r + 3]);
        const float k0 = 1024.0f * sa + 64.0f * sb;
        rec[QPC] = make_uint4(__builtin_bit_cast(uint32_t, k0), __builtin_bit_cast(uint32_t, sa + sb), 0u, 0u);
    }
    __syncthreads();

    // One pass: stage the row's header in LDS, compute, reduce, store.
    auto compute_pass = [&](int64_t ps, const uint4* w, const uint32_t* hs, const uint32_t* hz) {
        const int64_t n = ps * RPB + rs;
        const bool row_ok = n < N;
#pragma unroll
        for (int i = 0; i < CPT; ++i)
            if ((int64_t)TG * i < ngrp)   // uniform; clamped lanes rewrite the last entry
                row_hdr[hidx[i]] = make_float2(half_bits_to_float((uint16_t)hs[i]),
                                               half_bits_to_float((uint16_t)hz[i]));
        if constexpr (TG > 64) __syncthreads();
        else wave_lds_sync();

        float acc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = 0.0f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const float2 sz = row_hdr[gidx[i]];
            const float s = (row_ok && cin[i]) ? sz.x : 0.0f;
            const uint32_t ww[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
            const uint4* rec[NB];
            float pa[NB], pb[NB], xt[NB];
            // The X records do not change between passes; an opaque copy of the
            // index keeps their LDS reads inside the pass loop instead of being
            // hoisted into registers (which would cost occupancy).
            // The dependency on acc also orders chunk i's X reads after chunk
            // i-1's math, which bounds the registers holding X in flight.
            int ci = cidx[i];
            asm volatile("" : "+v"(ci) : "v"(acc[0]));
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                rec[b] = xrec + (size_t)(b * C + ci) * REC;
                const uint4 kx = rec[b][QPC];
                pa[b] = -__builtin_bit_cast(float, kx.x);
                xt[b] = __builtin_bit_cast(float, kx.y);
                pb[b] = 0.0f;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t sh = ww[j] >> 8;
                if constexpr (BITS == 4) {
                    // (q0,q4) and (q2,q6) unpack as 1024+q, (q1,q5) and (q3,q7)
                    // as 1024+16q: one AND-OR each, one shift per word.
                    const h2_t q04 = as_h2((ww[j] & m_lo) | MAGIC);
                    const h2_t q15 = as_h2((ww[j] & m_hi) | MAGIC);
                    const h2_t q26 = as_h2((sh & m_lo) | MAGIC);
                    const h2_t q37 = as_h2((sh & m_hi) | MAGIC);
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        const uint4 xv = rec[b][j];
                        pa[b] = __builtin_amdgcn_fdot2(q04, as_h2(xv.x), pa[b], false);
                        pb[b] = __builtin_amdgcn_fdot2(q15, as_h2(xv.y), pb[b], false);
                        pa[b] = __builtin_amdgcn_fdot2(q26, as_h2(xv.z), pa[b], false);
                        pb[b] = __builtin_amdgcn_fdot2(q37, as_h2(xv.w), pb[b], false);
                    }
                } else {
                    const h2_t q02 = as_h2((ww[j] & m_lo) | MAGIC);
                    const h2_t q13 = as_h2((sh & m_lo) | MAGIC);
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        const uint4 xv = rec[b][j >> 1];
                        pa[b] = __builtin_amdgcn_fdot2(q02, as_h2((j & 1) ? xv.z : xv.x), pa[b], false);
                        pa[b] = __builtin_amdgcn_fdot2(q13, as_h2((j & 1) ? xv.w : xv.y), pa[b], false);
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float t = pa[b];
                if constexpr (BITS == 4) t = __builtin_fmaf(pb[b], 0.0625f, t);
                t = __builtin_fmaf(-sz.y, xt[b], t);
                acc[b] = __builtin_fmaf(s, t, acc[b]);
            }
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
            wave_lds_sync();
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
    };

    // ---- stream rows, two passes per iteration (ping-pong registers) --------
    const int64_t step = gridDim.x;
    while (pass < passes) {
        load_pass(pass + step, wB, sB, zB);
        compute_pass(pass, wA, sA, zA);
        pass += step;
        if (pass >= passes) break;
        load_pass(pass + step, wA, sA, zA);
        compute_pass(pass, wB, sB, zB);
        pass += step;
    }
}

// ---- one batch row ---------------------------------------------------------
// B = 1 with whole rows inside one wave (TG <= 64) and an even group count per
// row: the same arithmetic as gemv_kernel, with less work around it.
//   - the group headers of a row arrive as 32-bit words (two scales or two
//     zeros each, HL words per thread) instead of one 16-bit load per entry;
//   - with TG == 64 the row is uniform across the wave, so the code loads take
//     a scalar row base and a fixed per-lane offset;
//   - chunks past a row's end read an all-zero X record (index C) instead of
//     being masked in every pass, and the records hold -K0, so a chunk costs
//     its unpack, its dot products and three FMAs.
template <int BITS, int TG, int CPT, int HL>
__global__ __launch_bounds__(256) void gemv_row_kernel(
    const uint16_t* __restrict__ X, const uint4* __restrict__ codes,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros,
    uint16_t* __restrict__ Y, int64_t N, int64_t K, int32_t G) {
    typedef ChunkGeom<BITS> CG;
    constexpr int QPC = CG::PAIRS / 4;          // uint4 of X pairs per chunk
    constexpr int REC = QPC + 1;                // uint4 per X record
    constexpr int RPB = 256 / TG;               // rows per block pass
    constexpr uint32_t MAGIC = 0x64006400u;
    // LDS: C + 1 X records, then (scale, zero) of every group of the block's
    // RPB rows.
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x;
    const int tl = tid % TG;
    const int rs = TG == 64 ? __builtin_amdgcn_readfirstlane(tid / TG) : tid / TG;
    const int C = (int)(K / CG::VALS);
    const int ngrp = (int)(K / G);
    const int cpg = G / CG::VALS;
    const int S = ngrp / 2;                     // header words per array and row
    // Row and pass indices fit 32 bits (the launcher checks N), which keeps
    // their compares on the scalar unit.
    const int Nr = (int)N;
    const int passes = (Nr + RPB - 1) / RPB;
    uint4* xrec = reinterpret_cast<uint4*>(smem);
    const uint32_t m_lo = vgpr_const(BITS == 4 ? 0x000F000Fu : 0x00FF00FFu);
    const uint32_t m_hi = vgpr_const(0x00F000F0u);

    // Per chunk: byte offset in the row, LDS byte address of its X record,
    // and its group.
    uint32_t coff[CPT], xaddr[CPT], gix[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int c = tl + TG * i;
        const bool ok = c < C;
        const int cc = ok ? c : C - 1;
        coff[i] = (uint32_t)cc * 16u;
        xaddr[i] = (uint32_t)(ok ? c : C) * (uint32_t)(REC * 16);
        gix[i] = (uint32_t)(cc / cpg);
    }
    // Header word h of this thread: word w of the row's 2S words (scales
    // first, then zeros; threads past the end repeat the last word), its byte
    // offset from the row's first scale, and where its two values go in hdr.
    int64_t hoff[HL];
    int hst[HL];
#pragma unroll
    for (int h = 0; h < HL; ++h) {
        int w = tl + TG * h;
        w = w < 2 * S ? w : 2 * S - 1;
        const bool isz = w >= S;
        const int wm = isz ? w - S : w;
        hoff[h] = (isz ? (int64_t)(reinterpret_cast<const char*>(zeros) -
                                   reinterpret_cast<const char*>(scales))
                       : (int64_t)0) +
                  (int64_t)wm * 4;
        hst[h] = 4 * wm + (isz ? 1 : 0);
    }

    // Every load is issued unconditionally, so the next pass stays in flight
    // while the current one computes.  With TG == 64 a wave owns one row, and
    // its codes are read through a buffer resource: scalar base, per-lane
    // 32-bit offsets, and a record count of zero for rows past the end, which
    // then read zeros without touching memory.  Narrower groups (several rows
    // per wave) reread the last row instead.
    auto load_pass = [&](int pass, uint4* w, uint32_t* hw) {
        // The prefetched pass may lie up to a grid's worth past the last one:
        // its row is formed in 64 bits (no overflow for N near 2^31).
        const int64_t n64 = (int64_t)pass * RPB + rs;
        const bool live = n64 < (int64_t)Nr;
        const int n = live ? (int)n64 : Nr - 1;
        if constexpr (TG == 64) {
            const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint4*>(codes + (int64_t)n * C), (short)0, live ? C * 16 : 0, kBufferWord3);
#pragma unroll
            for (int i = 0; i < CPT; ++i) w[i] = load_stream_buf(rsrc, coff[i]);
        } else {
            const char* rowc = reinterpret_cast<const char*>(codes + (int64_t)n * C);
#pragma unroll
            for (int i = 0; i < CPT; ++i) w[i] = load_stream(reinterpret_cast<const uint4*>(rowc + coff[i]));
        }
        const char* rowh = reinterpret_cast<const char*>(scales + (int64_t)n * ngrp);
#pragma unroll
        for (int h = 0; h < HL; ++h) hw[h] = *reinterpret_cast<const uint32_t*>(rowh + hoff[h]);
    };

    int pass = blockIdx.x;
    uint4 wA[CPT], wB[CPT];
    uint32_t hA[HL], hB[HL];
#pragma unroll
    for (int i = 0; i < CPT; ++i) wA[i] = wB[i] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int h = 0; h < HL; ++h) hA[h] = hB[h] = 0u;
    load_pass(pass, wA, hA);

    // ---- X records in LDS, plus the zero record C ---------------------------
    for (int e = tid; e <= C; e += 256) {
        uint16_t xv[CG::VALS];
        if (e < C) {
            const uint4* src = reinterpret_cast<const uint4*>(X + (int64_t)e * CG::VALS);
#pragma unroll
            for (int v = 0; v < CG::VALS / 8; ++v) {
                const uint4 u = src[v];
                const uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    xv[8 * v + 2 * q] = (uint16_t)(ww[q] & 0xFFFFu);
                    xv[8 * v + 2 * q + 1] = (uint16_t)(ww[q] >> 16);
                }
            }
        } else {
#pragma unroll
            for (int v = 0; v < CG::VALS; ++v) xv[v] = 0;
        }
        uint32_t pr[CG::PAIRS];
        float sa = 0.0f, sb = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int p = 0; p < CG::PAIRS_PER_WORD; ++p) {
                int a, bb;
                pair_positions<BITS>(j, p, a, bb);
                pr[j * CG::PAIRS_PER_WORD + p] = (uint32_t)xv[a] | ((uint32_t)xv[bb] << 16);
                const float t = half_bits_to_float(xv[a]) + half_bits_to_float(xv[bb]);
                if (BITS == 4 && (p & 1)) sb += t;
                else sa += t;
            }
        uint4* rec = xrec + (size_t)e * REC;
#pragma unroll
        for (int r = 0; r < QPC; ++r)
            rec[r] = make_uint4(pr[4 * r], pr[4 * r + 1], pr[4 * r + 2], pr[4 * r + 3]);
        const float k0 = 1024.0f * sa + 64.0f * sb;
        rec[QPC] = make_uint4(__builtin_bit_cast(uint32_t, -k0), __builtin_bit_cast(uint32_t, sa + sb), 0u, 0u);
    }
    __syncthreads();

    float2* hrow = reinterpret_cast<float2*>(smem + (size_t)(C + 1) * REC * 16) + (size_t)rs * ngrp;
    float* hf = reinterpret_cast<float*>(hrow);
    auto compute_pass = [&](int ps, const uint4* w, const uint32_t* hw) {
        const int n = ps * RPB + rs;
#pragma unroll
        for (int h = 0; h < HL; ++h) {
            hf[hst[h]] = half_bits_to_float((uint16_t)(hw[h] & 0xFFFFu));
            hf[hst[h] + 2] = half_bits_to_float((uint16_t)(hw[h] >> 16));
        }
        wave_lds_sync();
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const float2 sz = hrow[gix[i]];
            // The address is made opaque in place: the record reads stay in
            // the pass loop, after the previous chunk's math (which bounds the
            // registers in flight), at no instruction cost.
            asm volatile("" : "+v"(xaddr[i]) : "v"(acc));
            const uint4* rec = reinterpret_cast<const uint4*>(smem + xaddr[i]);
            const uint4 kx = rec[QPC];
            float pa = __builtin_bit_cast(float, kx.x);
            const float xt = __builtin_bit_cast(float, kx.y);
            float pb = 0.0f;
            const uint32_t ww[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t sh = ww[j] >> 8;
                if constexpr (BITS == 4) {
                    const h2_t q04 = as_h2((ww[j] & m_lo) | MAGIC);
                    const h2_t q15 = as_h2((ww[j] & m_hi) | MAGIC);
                    const h2_t q26 = as_h2((sh & m_lo) | MAGIC);
                    const h2_t q37 = as_h2((sh & m_hi) | MAGIC);
                    const uint4 xv = rec[j];
                    pa = __builtin_amdgcn_fdot2(q04, as_h2(xv.x), pa, false);
                    pb = __builtin_amdgcn_fdot2(q15, as_h2(xv.y), pb, false);
                    pa = __builtin_amdgcn_fdot2(q26, as_h2(xv.z), pa, false);
                    pb = __builtin_amdgcn_fdot2(q37, as_h2(xv.w), pb, false);
                } else {
                    const h2_t q02 = as_h2((ww[j] & m_lo) | MAGIC);
                    const h2_t q13 = as_h2((sh & m_lo) | MAGIC);
                    const uint4 xv = rec[j >> 1];
                    pa = __builtin_amdgcn_fdot2(q02, as_h2((j & 1) ? xv.z : xv.x), pa, false);
                    pa = __builtin_amdgcn_fdot2(q13, as_h2((j & 1) ? xv.w : xv.y), pa, false);
                }
            }
            float t = pa;
            if constexpr (BITS == 4) t = __builtin_fmaf(pb, 0.0625f, t);
            t = __builtin_fmaf(-sz.y, xt, t);
            acc = __builtin_fmaf(sz.x, t, acc);
        }
        acc = group_total_last<TG>(acc);
        if (tl == TG - 1 && n < Nr) Y[n] = float_to_half_bits_rne(acc);
        wave_lds_sync();
    };

    // The scheduling barriers keep each pass's loads ahead of the previous
    // pass's math (the header staging would otherwise be hoisted above them
    // and wait for every load in flight).
    const int step = gridDim.x;
    while (pass < passes) {
        load_pass(pass + step, wB, hB);
        __builtin_amdgcn_sched_barrier(0);
        compute_pass(pass, wA, hA);
        pass += step;
        if (pass >= passes) break;
        load_pass(pass + step, wA, hA);
        __builtin_amdgcn_sched_barrier(0);
        compute_pass(pass, wB, hB);
        pass += step;
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

// LDS bytes of X per batch row and chunk: the permuted pairs plus one uint4
// holding the chunk constants.
size_t x_lds_per_chunk(int32_t bits) {
    return ((size_t)(64 / bits) / 4 + 1) * sizeof(uint4);
}

constexpr size_t kMaxXLds = 64 * 1024;

// Batch tile NB covers the batch up to 8 rows while its X fits in 64 KB of
// LDS; TG threads per row is the smallest power of two (16..256) that covers
// a row with at most 4 chunks per thread.
bool choose(int64_t B, int64_t K, int32_t bits, GemvChoice& ch) {
    const int vals = 128 / bits;
    if (K % vals != 0) return false;
    const int64_t C = K / vals;
    int nb = pow2_ceil(B < 8 ? B : 8);
    while (nb > 1 && (size_t)nb * C * x_lds_per_chunk(bits) > kMaxXLds) nb >>= 1;
    if ((size_t)nb * C * x_lds_per_chunk(bits) > kMaxXLds) return false;
    int tg = 16;
    while (tg < 256 && (int64_t)tg * 4 < C) tg <<= 1;
    const int64_t need = (C + tg - 1) / tg;
    if (need > 4) return false;
    const int cpt = pow2_ceil(need);
    while (nb * cpt > 8 && nb > 1) nb >>= 1;  // bounds the accumulators per thread
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
    typedef ChunkGeom<BITS> CG;
    const int64_t C = K / CG::VALS;
    const size_t lds = (size_t)NB * C * x_lds_per_chunk(BITS);
    // Persistent grid: as many blocks as fit on the chip at once, each looping
    // over row passes, so X is staged once per resident block.
    // Occupancy depends on the X record size; remember the last answer.
    static thread_local size_t cached_lds = (size_t)-1;
    static thread_local int cached_per_cu = 1;
    if (cached_lds != lds) {
        int v = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, gemv_kernel<BITS, NB, TG, CPT>, 256, lds) !=
                hipSuccess || v <= 0)
            v = 1;
        cached_lds = lds;
        cached_per_cu = v;
    }
    const int per_cu = cached_per_cu;
    const int64_t passes = (N + RPB - 1) / RPB;
    const int64_t cap = (int64_t)num_cus * per_cu;
    const dim3 grid((unsigned)(passes < cap ? passes : cap), (unsigned)((B + NB - 1) / NB));
    gemv_kernel<BITS, NB, TG, CPT><<<grid, dim3(256), lds, stream>>>(
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

// LDS of the one-row kernel: X records (C + 1 of them, the last zero) and
// the group headers of the 256 / TG rows of a block pass.
size_t row_lds_bytes(int64_t K, int32_t G, int32_t bits, int tg) {
    return (size_t)(K / (128 / bits) + 1) * x_lds_per_chunk(bits) +
           (size_t)(256 / tg) * (size_t)(K / G) * sizeof(float2);
}

template <int BITS, int TG, int CPT, int HL>
hipError_t launch_row(const void* X, const void* codes, const void* scales, const void* zeros,
                      void* Y, int64_t K, int64_t N, int32_t G, int num_cus, hipStream_t stream) {
    constexpr int RPB = 256 / TG;
    const size_t lds = row_lds_bytes(K, G, BITS, TG);
    static thread_local size_t cached_lds = (size_t)-1;
    static thread_local int cached_per_cu = 1;
    if (cached_lds != lds) {
        int v = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, gemv_row_kernel<BITS, TG, CPT, HL>, 256, lds) !=
                hipSuccess || v <= 0)
            v = 1;
        cached_lds = lds;
        cached_per_cu = v;
    }
    const int64_t passes = (N + RPB - 1) / RPB;
    const int64_t cap = (int64_t)num_cus * cached_per_cu;
    gemv_row_kernel<BITS, TG, CPT, HL><<<dim3((unsigned)(passes < cap ? passes : cap)), dim3(256), lds, stream>>>(
        static_cast<const uint16_t*>(X), static_cast<const uint4*>(codes),
        static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros),
        static_cast<uint16_t*>(Y), N, K, G);
    return hipGetLastError();
}

template <int BITS, int TG, int CPT>
hipError_t row_by_hl(int hl, const void* X, const void* codes, const void* scales, const void* zeros,
                     void* Y, int64_t K, int64_t N, int32_t G, int cus, hipStream_t st) {
    if (hl == 1) return launch_row<BITS, TG, CPT, 1>(X, codes, scales, zeros, Y, K, N, G, cus, st);
    if constexpr (CPT >= 2)
        if (hl == 2) return launch_row<BITS, TG, CPT, 2>(X, codes, scales, zeros, Y, K, N, G, cus, st);
    if constexpr (CPT >= 4)
        if (hl == 4) return launch_row<BITS, TG, CPT, 4>(X, codes, scales, zeros, Y, K, N, G, cus, st);
    return hipErrorInvalidValue;
}

template <int BITS, int TG>
hipError_t row_by_cpt(int cpt, int hl, const void* X, const void* codes, const void* scales,
                      const void* zeros, void* Y, int64_t K, int64_t N, int32_t G, int cus,
                      hipStream_t st) {
    switch (cpt) {
        case 1: return row_by_hl<BITS, TG, 1>(hl, X, codes, scales, zeros, Y, K, N, G, cus, st);
        case 2: return row_by_hl<BITS, TG, 2>(hl, X, codes, scales, zeros, Y, K, N, G, cus, st);
        case 4: return row_by_hl<BITS, TG, 4>(hl, X, codes, scales, zeros, Y, K, N, G, cus, st);
    }
    return hipErrorInvalidValue;
}

// The one-row kernel applies when a row fits one wave, its group count is
// even and the header arrays allow 32-bit loads.  HL = header words per thread.
bool row_path(int64_t B, int64_t K, int64_t N, int32_t G, const GemvChoice& ch,
              const void* scales, const void* zeros, int& hl) {
    if (B != 1 || ch.tg > 64 || N >= ((int64_t)1 << 31) - 256) return false;
    const int64_t ngrp = K / G;
    if (ngrp % 2 != 0 || reinterpret_cast<uintptr_t>(scales) % 4 != 0 ||
        reinterpret_cast<uintptr_t>(zeros) % 4 != 0)
        return false;
    const int64_t need = (ngrp + ch.tg - 1) / ch.tg;   // 2 * (ngrp / 2) words over TG threads
    hl = need <= 1 ? 1 : need <= 2 ? 2 : 4;
    return hl <= ch.cpt;
}

}  // namespace

bool gemv_supports(int64_t K, int32_t bits) {
    GemvChoice ch;
    return choose(1, K, bits, ch);
}

hipError_t launch_gemv(const void* X, const void* codes, const void* scales,
                       const void* zeros, void* Y, int64_t B, int64_t K, int64_t N,
                       int32_t group, int32_t bits, int num_cus, hipStream_t stream) {
    GemvChoice ch;
    if (!choose(B, K, bits, ch)) return hipErrorInvalidValue;
    int hl = 0;
    if (row_path(B, K, N, group, ch, scales, zeros, hl)) {
        const int cus = num_cus;
        if (bits == 4) {
            switch (ch.tg) {
                case 16: return row_by_cpt<4, 16>(ch.cpt, hl, X, codes, scales, zeros, Y, K, N, group, cus, stream);
                case 32: return row_by_cpt<4, 32>(ch.cpt, hl, X, codes, scales, zeros, Y, K, N, group, cus, stream);
                case 64: return row_by_cpt<4, 64>(ch.cpt, hl, X, codes, scales, zeros, Y, K, N, group, cus, stream);
            }
        } else {
            switch (ch.tg) {
                case 16: return row_by_cpt<8, 16>(ch.cpt, hl, X, codes, scales, zeros, Y, K, N, group, cus, stream);
                case 32: return row_by_cpt<8, 32>(ch.cpt, hl, X, codes, scales, zeros, Y, K, N, group, cus, stream);
                case 64: return row_by_cpt<8, 64>(ch.cpt, hl, X, codes, scales, zeros, Y, K, N, group, cus, stream);
            }
        }
        return hipErrorInvalidValue;
    }
    if (bits == 4)
        return by_shape<4>(ch, X, codes, scales, zeros, Y, B, K, N, group, num_cus, stream);
    return by_shape<8>(ch, X, codes, scales, zeros, Y, B, K, N, group, num_cus, stream);
}

}  // namespace wq
