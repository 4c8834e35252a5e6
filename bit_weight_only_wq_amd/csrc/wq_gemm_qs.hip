// Small-batch product (B <= 4) on the matrix cores' 4 x 4 x 4 blocks:
// Y[B,N] = X[B,K] * dequant(W)[N,K]^T.
//
// At decode batch sizes the product is a stream of the packed weights
// ("Quantization & inference optimisation", "Bandwidth, not compute": 2B/w
// FLOP per byte), and what limits such a stream is how many bytes are in
// flight and how many instructions move them, not arithmetic.  So:
//   - an item is 4 weight rows (a quad) x 512 k: 4 x 256 bytes of codes, one
//     128-bit load per lane (lane 4b + j: row j, bytes 16b..16b+15 of the
//     256), the shape HBM serves at 6 TB/s and more; it is the only load in
//     the main loop, and every wave keeps 8 of them in flight in a ring of
//     registers (8 KB per wave, 64 KB per compute unit), so every wait in
//     the loop is a counted one;
//   - v_mfma_f32_4x4x4_16b_f16 takes that layout as it is: block b (lanes
//     4b..4b+3) multiplies the 32 k of chunk b, lane 4b + j holding row j of
//     the codes (B operand) and batch row j of X (A operand);
//   - a wave keeps the same one, two or four 512-k positions of K for the
//     whole kernel, so its X operands and their chunk sums live in registers,
//     loaded once; the P waves of a row stream split K between them and walk
//     the stream's quads together;
//   - the group headers of all the block's quads are copied into LDS once, at
//     the start (contiguous 16-byte loads straight into LDS), while the first
//     code loads are already in flight;
//   - codes unpack exactly to fp16 1024 + q (even k) and 64 + q (odd k); each
//     block's accumulation starts at -C1 (the offsets' weighted X sum) and the
//     chunk's group header is applied once per item in fp32 ("the kernel
//     reconstructs an approximate float from the integer and the endpoints as
//     it reads", "Quantization"):
//         sum_k (q - z) s x = s * (sum_k u_k x_k - C1 - z * C2);
//   - after a quad's positions, the 16 blocks' sums of each (batch row, weight
//     row) are added across lanes (two half swaps and two row rotations) and
//     the wave's 16 sums go to LDS; after the last quad the block
//     adds the P waves' sums of every output in wave order (deterministic)
//     and writes Y.  The loop has no barrier.
// Loads past a row's end or the stream's end fall outside the buffer and
// return zero without touching memory.  No scratch memory.  Requires 4-bit
// codes, K % 32 == 0, group % 64 == 0, an even group count per row, 16-byte
// aligned header arrays and K <= 16384.
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

namespace {

constexpr int QS_MAX_LDS = 160 * 1024;
constexpr int kQsBufWord3 = 0x00020000;     // raw, unswizzled gfx9 buffer
constexpr uint32_t kQsFar = 0x80000000u;    // a per-lane offset past every buffer this kernel reads

typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef unsigned int qs_v4u __attribute__((ext_vector_type(4)));

struct QsArgs {
    const uint16_t* X;
    const uint8_t* codes;
    const uint16_t* scales;
    const uint16_t* zeros;
    uint16_t* Y;
    int32_t B, N, K, G;
    int32_t ngrp;          // groups per row
    int32_t npos;          // 512-k positions (the last may be partial)
    int32_t P, R;          // waves per row stream, row streams per block
    int32_t nquads;        // quads of 4 rows
    int32_t S;             // row streams in the grid
    int32_t QB;            // quads per stream at most
    uint32_t row_bytes;    // K / 2
    uint32_t code_bytes;   // N * K / 2
    uint32_t hdr_bytes;    // N * ngrp * 2
    uint32_t hdr_half;     // LDS bytes of the staged scales (the zeros follow; whole kilobytes)
};

// LDS: the staged scales, [R][QB][4 rows][ngrp] halves, then the zeros in the
// same layout (each rounded up to whole kilobytes: a staging load fills
// one), then the waves' per-quad sums, [R][QB][P][16] floats.
size_t qs_hdr_half(int R, int QB, int ngrp) {
    const size_t b = (size_t)R * QB * 8 * ngrp;
    return (b + 1023) / 1024 * 1024;
}
size_t qs_red_lds(int R, int QB, int P) { return (size_t)R * QB * P * 16 * sizeof(float); }

__device__ __forceinline__ uint4 qs_order8(uint4 in) {
    uint4 o;
    o.x = __builtin_amdgcn_perm(in.z, in.x, 0x05040100u);   // x0 | x4 << 16
    o.y = __builtin_amdgcn_perm(in.z, in.x, 0x07060302u);   // x1 | x5 << 16
    o.z = __builtin_amdgcn_perm(in.w, in.y, 0x05040100u);   // x2 | x6 << 16
    o.w = __builtin_amdgcn_perm(in.w, in.y, 0x07060302u);   // x3 | x7 << 16
    return o;
}

template <int CTRL>
__device__ __forceinline__ float qs_dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Value of lane 4 * (lane / 4) + E (quad_perm [E, E, E, E]).
template <int E>
__device__ __forceinline__ float qs_quad_bcast(float v) {
    return qs_dpp<E | (E << 2) | (E << 4) | (E << 6)>(v);
}

// Half swaps between two registers (v_permlane32_swap / v_permlane16_swap),
// written as instructions: the compiler's builtins for them return wrong
// values here when both results feed one expression.  The s_nop pairs give
// the wait states a VALU result needs before and after a permlane.
//   swap32: a' = [a lanes 0-31 | b lanes 0-31], b' = [a lanes 32-63 | b lanes 32-63]
//   swap16 (per half): a' = [a 0-15, b 0-15], b' = [a 16-31, b 16-31]
__device__ __forceinline__ void qs_swap32(float& a, float& b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void qs_swap16(float& a, float& b) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}

// Sum of t[e] (e = 0..3) over the 16 blocks of each batch row e and weight
// row j.  Lane l ends with the total of e = l / 16, j = l % 4 (the same on the
// four lanes l % 16 = j, j + 4, j + 8, j + 12).
__device__ __forceinline__ float qs_block_sum(const f4_t t) {
    // Halves: lanes 0-31 keep e = 0 (resp. 1), lanes 32-63 e = 2 (3), each
    // summed over lanes l and l ^ 32 (blocks b and b ^ 8).
    float a0 = t[0], a2 = t[2], a1 = t[1], a3 = t[3];
    qs_swap32(a0, a2);
    qs_swap32(a1, a3);
    float w0 = a0 + a2, w1 = a1 + a3;
    // Quarters: lanes 0-15 keep e = 0, 16-31 e = 1, 32-47 e = 2, 48-63 e = 3.
    qs_swap16(w0, w1);
    float u = w0 + w1;
    // The four blocks of each 16-lane row: rotate by 4 and by 8 lanes.
    u += qs_dpp<0x124>(u);   // row_ror:4
    u += qs_dpp<0x128>(u);   // row_ror:8
    return u;
}

// Quads of a row stream: the stream's QB consecutive quads.  Quad q of
// stream st, and how many quads the stream has.
#ifndef QS_INTERLEAVE
#define QS_INTERLEAVE 1
#endif
__device__ __forceinline__ uint32_t qs_quad(const QsArgs& a, int st, int q) {
    return QS_INTERLEAVE ? (uint32_t)(st + q * a.S) : (uint32_t)(st * a.QB + q);
}
__device__ __forceinline__ int qs_nq(const QsArgs& a, int st) {
    if (QS_INTERLEAVE) return st < a.nquads ? (a.nquads - st + a.S - 1) / a.S : 0;
    const int left = a.nquads - st * a.QB;
    return left < 0 ? 0 : left < a.QB ? left : a.QB;
}

// The block meets with its LDS writes done (loads stay in flight).
__device__ __forceinline__ void qs_meet() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0) only
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// NE: batch rows whose outputs are computed (1, 2 or 4).  NPW: positions per
// wave (1, 2 or 4).  W: waves per block, D: items in flight per wave (W * D
// KB per compute unit).
template <int NE, int NPW, int W, int D>
__global__ __launch_bounds__(W * 64, 1) void gemm_qs_kernel(const QsArgs a) {
    extern __shared__ __align__(16) unsigned char qs_lds[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = a.R * a.P;
    const int j = lane & 3;              // weight row of the quad (B operand), batch row (A operand)
    const int blk = lane >> 2;           // 4 x 4 block: 32-k chunk of the position
    const int rs = wave / a.P;           // row stream of the block
    const int pw = wave - rs * a.P;      // wave within the stream
    const int stream = blockIdx.x * a.R + rs;
    const int nq = qs_nq(a, stream);                 // <= QB
    const int items = nq * NPW;
    const uint32_t run = 8u * (uint32_t)a.ngrp;         // header bytes of one quad and array
    unsigned char* const hdr = qs_lds;
    float* const red_all = reinterpret_cast<float*>(qs_lds + 2u * a.hdr_half);

    // ---- 1. the block's group headers -> LDS (loads straight into LDS) --------
    // Staging load c fills LDS bytes [1024 c, 1024 c + 1024) of the scales'
    // (then the zeros') area: lane l the 16 bytes at 1024 c + 16 l, which are
    // bytes w of quad q of stream r, read from that quad's 4 rows (nothing
    // past the block's quads or the matrix).
    {
        const uint32_t per_arr = a.hdr_half / 1024u;
        const uint32_t nruns = (uint32_t)a.R * (uint32_t)a.QB;
        for (uint32_t c = (uint32_t)wave; c < 2u * per_arr; c += (uint32_t)nwaves) {
            const bool zarr = c >= per_arr;
            const uint32_t o = 1024u * (zarr ? c - per_arr : c) + 16u * (uint32_t)lane;
            const uint32_t ri = o / run, w = o - ri * run;
            const uint32_t rr = ri / (uint32_t)a.QB, q = ri - rr * (uint32_t)a.QB;
            const uint32_t quad = qs_quad(a, blockIdx.x * a.R + (int)rr, (int)q);
            const uint32_t src = (ri < nruns && quad < (uint32_t)a.nquads) ? quad * run + w : kQsFar;
            const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(zarr ? a.zeros : a.scales), (short)0, (int)a.hdr_bytes, kQsBufWord3);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(hdr + 1024u * c), 16, (int)src, 0, 0, 0);
        }
    }

    // The phases' loads stay in this order (staging, X, ring): the waits
    // below count on it.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // ---- 2. X operands (registers) ---------------------------------------------
    // Lane 4b + j holds batch row j at k = 512 p + 32 b + 8 r (r = 0..3).
    // Rows past B and chunks past K read zeros.
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.X), (short)0, (int)((uint32_t)a.B * (uint32_t)a.K * 2u), kQsBufWord3);
    uint4 xa[NPW][4];
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
        const int p = pw + i * a.P;
        const int64_t k0 = (int64_t)p * 512 + 32 * blk;
        const bool live = p < a.npos && j < a.B && k0 < a.K;
        const uint32_t xo = live ? (uint32_t)(((int64_t)j * a.K + k0) * 2) : kQsFar;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const qs_v4u t = __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)(xo + 16u * r), 0, 0);
            xa[i][r] = make_uint4(t.x, t.y, t.z, t.w);
        }
    }

    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // ---- 3. the code ring ---------------------------------------------------------
    // Item it = (quad index it / NPW, position slot it % NPW); quad index q is
    // the stream's quad stream + q * S.  Each load's buffer starts at its quad
    // and ends at the matrix's end (no bytes for items past the stream's end),
    // so the range check, which covers the per-lane offset, turns every read
    // past the last row into a zero without memory traffic.
    uint32_t coff[NPW], hl[NPW];
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
        const int p = pw + i * a.P;
        // A chunk past the row's end reads the next row's bytes (X is zero
        // there); a position past the last one reads nothing.
        coff[i] = p < a.npos ? (uint32_t)j * a.row_bytes + (uint32_t)p * 256u + 16u * (uint32_t)blk : kQsFar;
        // LDS offset of this lane's scale within a quad's staged run.
        int g = (int)(((int64_t)p * 512 + 32 * blk) / a.G);
        g = g < a.ngrp ? g : a.ngrp - 1;
        hl[i] = (uint32_t)(2 * (j * a.ngrp + g));
    }
    const uint32_t quad_cb = 4u * a.row_bytes;
    auto load_item = [&](int it) -> uint4 {
        const uint32_t quad = qs_quad(a, stream, it / NPW);
        const bool live = it < items;
        const uint32_t base = live ? quad * quad_cb : 0u;
        const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(a.codes + base), (short)0, live ? (int)(a.code_bytes - base) : 0, kQsBufWord3);
        const qs_v4u t = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)coff[it % NPW], 0, 2);
        return make_uint4(t.x, t.y, t.z, t.w);
    };
    uint4 ring[D];
#pragma unroll
    for (int d = 0; d < D; ++d) ring[d] = load_item(d);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // ---- 4. X chunk sums, permuted operands; headers visible to all waves -----
    // -C1 and C2 of every batch row over chunk b come from the quad's four
    // lanes.  (Waiting for X and the staged headers leaves the ring's
    // loads, issued after them, in flight.)
    f4_t nc1[NPW], c2[NPW];
    {
        const h2_t one = {(_Float16)1.0f, (_Float16)1.0f};
        const h2_t wgt = {(_Float16)1024.0f, (_Float16)64.0f};
#pragma unroll
        for (int i = 0; i < NPW; ++i) {
                float d1 = 0.0f, d2 = 0.0f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint4 x = xa[i][r];
                    d2 = __builtin_amdgcn_fdot2(as_h2(x.x), one, d2, false);
                    d2 = __builtin_amdgcn_fdot2(as_h2(x.y), one, d2, false);
                    d2 = __builtin_amdgcn_fdot2(as_h2(x.z), one, d2, false);
                    d2 = __builtin_amdgcn_fdot2(as_h2(x.w), one, d2, false);
                    d1 = __builtin_amdgcn_fdot2(as_h2(x.x), wgt, d1, false);
                    d1 = __builtin_amdgcn_fdot2(as_h2(x.y), wgt, d1, false);
                    d1 = __builtin_amdgcn_fdot2(as_h2(x.z), wgt, d1, false);
                    d1 = __builtin_amdgcn_fdot2(as_h2(x.w), wgt, d1, false);
                    xa[i][r] = qs_order8(x);
                }
                nc1[i] = f4_t{-qs_quad_bcast<0>(d1), -qs_quad_bcast<1>(d1), -qs_quad_bcast<2>(d1),
                              -qs_quad_bcast<3>(d1)};
                c2[i] = f4_t{qs_quad_bcast<0>(d2), qs_quad_bcast<1>(d2), qs_quad_bcast<2>(d2),
                             qs_quad_bcast<3>(d2)};
        }
    }
    // The staging loads were issued before the ring's D: once at most D
    // loads are outstanding, this wave's staging has landed in LDS.
    asm volatile("" ::: "memory");
    static_assert(D == 4 || D == 8 || D == 16, "ring depth");
    __builtin_amdgcn_s_waitcnt(D == 16 ? 0x4F70 : D == 8 ? 0x0F78 : 0x0F74);   // vmcnt(D): bits 3:0, 15:14
    qs_meet();

    // ---- 5. the stream -----------------------------------------------------------
    const uint32_t m_lo = vgpr_const(0x000F000Fu), m_hi = vgpr_const(0x00F000F0u);
    const uint32_t g_lo = vgpr_const(0x64006400u), g_hi = vgpr_const(0x54005400u);
    f4_t tot = {0.0f, 0.0f, 0.0f, 0.0f};
    const unsigned char* const shdr = hdr + (size_t)rs * a.QB * run;
    float* const red = red_all + (size_t)rs * a.QB * a.P * 16;

    // One item: unpack, multiply, apply the header (positions past K are
    // skipped).  After a quad's last position, its block sums go to LDS.
    auto compute = [&](int i, int it, const uint4& cw) {
        const int q = it / NPW;
        if (pw + i * a.P < a.npos) {
            const unsigned char* h = shdr + (size_t)q * run + hl[i];
            const float s = half_bits_to_float(*reinterpret_cast<const uint16_t*>(h));
            const float z = half_bits_to_float(*reinterpret_cast<const uint16_t*>(h + a.hdr_half));
            const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
            // B operands of the four words: steps (r, 0) take k (0,4,1,5) of
            // word r, steps (r, 1) take (2,6,3,7).
            uint2 b0[4], b1[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t w8 = w[r] >> 8;
                b0[r] = make_uint2((w[r] & m_lo) | g_lo, (w[r] & m_hi) | g_hi);
                b1[r] = make_uint2((w8 & m_lo) | g_lo, (w8 & m_hi) | g_hi);
            }
            // Two accumulation chains (even, odd steps) keep the matrix core busy.
            f4_t acc0 = nc1[i];
            f4_t acc1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint4 x = xa[i][r];
                acc0 = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(h4_t, make_uint2(x.x, x.y)),
                                                          __builtin_bit_cast(h4_t, b0[r]), acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(h4_t, make_uint2(x.z, x.w)),
                                                          __builtin_bit_cast(h4_t, b1[r]), acc1, 0, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                float t = acc0[e] + acc1[e];
                t = __builtin_fmaf(-z, c2[i][e], t);
                tot[e] = __builtin_fmaf(s, t, tot[e]);
            }
        }
        if (i == NPW - 1) {
            float* const dst = red + ((size_t)q * a.P + pw) * 16;
            const float u = qs_block_sum(tot);
            if ((lane & 12) == 0) dst[4 * (lane >> 4) + j] = u;
            tot = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };

    for (int it0 = 0; it0 < items; it0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int it = it0 + d;
            if (it < items) compute(d % NPW, it, ring[d]);
            ring[d] = load_item(it + D);
        }
    }
    qs_meet();

    // ---- 6. Y: the P waves' sums of every output, in wave order -------------
    const int per_stream = a.QB * 4 * a.B;
    for (int o = threadIdx.x; o < a.R * per_stream; o += nwaves * 64) {
        const int r = o / per_stream;
        const int rem = o - r * per_stream;
        const int b = rem % a.B;
        const int qj = rem / a.B;
        const int q = qj >> 2, jj = qj & 3;
        const int st_r = blockIdx.x * a.R + r;
        const int nq_r = qs_nq(a, st_r);
        const int64_t row = (int64_t)qs_quad(a, st_r, q) * 4 + jj;
        if (q >= nq_r || row >= a.N) continue;
        const float* src = red_all + (((size_t)r * a.QB + q) * a.P) * 16 + 4 * b + jj;
        float t = 0.0f;
        for (int w = 0; w < a.P; ++w) t += src[(size_t)w * 16];
        a.Y[(int64_t)b * a.N + row] = float_to_half_bits_rne(t);
    }
    // Loads issued past the end: let them land before the block ends.
    __builtin_amdgcn_s_waitcnt(0);
}

struct QsPlan {
    int waves, depth, npw, P, R, blocks, QB;
    size_t half, lds;
};

// 8 waves with 8 items in flight each: 64 loads of 1 KB per compute unit.
// (A read-only copy of this loop streams faster with 64 KB in flight than
// with 128 KB, the more so as a wave's share of the matrix is only a few
// dozen items: a deeper ring takes longer to fill and to drain.)
constexpr int QS_W = 8, QS_D = 8;

// Positions per wave, waves per stream, streams per block and the grid;
// false when the shape does not fit.
bool qs_plan(int64_t B, int64_t K, int64_t N, int num_cus, QsPlan& pl) {
    const int W = QS_W;
    const int64_t npos = (K + 511) / 512;
    int npw = 1;
    while (npw < 4 && npos > (int64_t)W * npw) npw <<= 1;
    if (npos > (int64_t)W * npw) return false;
    const int P = (int)((npos + npw - 1) / npw);
    const int R = W / P;
    const int64_t nquads = (N + 3) / 4;
    int64_t blocks = (nquads + R - 1) / R;
    if (blocks > num_cus) blocks = num_cus;
    pl = QsPlan{R * P, QS_D, npw, P, R, (int)blocks, 0, 0, 0};
    return true;
}

// Grow the grid until the staged headers and the per-quad sums fit in LDS.
bool qs_fit(int64_t N, int32_t ngrp, QsPlan& pl) {
    const int64_t nquads = (N + 3) / 4;
    int64_t blocks = pl.blocks;
    for (;;) {
        const int64_t S = blocks * pl.R;
        const int QB = (int)((nquads + S - 1) / S);
        const size_t half = qs_hdr_half(pl.R, QB, ngrp);
        const size_t lds = 2 * half + qs_red_lds(pl.R, QB, pl.P);
        if (lds <= (size_t)QS_MAX_LDS) {
            pl.blocks = (int)blocks;
            pl.QB = QB;
            pl.half = half;
            pl.lds = lds;
            return true;
        }
        if (blocks >= nquads) return false;
        blocks = blocks * 2 < nquads ? blocks * 2 : nquads;
    }
}

template <int NE, int NPW, int W, int D>
hipError_t launch_qs4(const QsArgs& a, const QsPlan& pl, hipStream_t stream) {
    gemm_qs_kernel<NE, NPW, W, D><<<dim3((unsigned)pl.blocks), dim3((unsigned)(pl.waves * 64)), pl.lds, stream>>>(a);
    return hipGetLastError();
}

template <int NE>
hipError_t launch_qs2(const QsArgs& a, const QsPlan& pl, hipStream_t stream) {
    switch (pl.npw) {
        case 1: return launch_qs4<NE, 1, QS_W, QS_D>(a, pl, stream);
        case 2: return launch_qs4<NE, 2, QS_W, QS_D>(a, pl, stream);
        case 4: return launch_qs4<NE, 4, QS_W, QS_D>(a, pl, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool qs_supports(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits) {
    if (bits != 4 || B < 1 || B > 4 || K < 32 || K % 32 != 0 || group < 64 || group % 64 != 0 || N < 1)
        return false;
    if (K % group != 0 || (K / group) % 2 != 0) return false;
    // 32-bit buffer offsets with room for the far offset: codes, headers and
    // X under 2 GiB.
    if ((uint64_t)N * (uint64_t)(K / 2) + 8ull * (uint64_t)K >= (uint64_t)kQsFar) return false;
    if ((uint64_t)N * (uint64_t)(K / group) * 2ull + 8ull * (uint64_t)K >= (uint64_t)kQsFar) return false;
    if ((uint64_t)B * (uint64_t)K * 2ull >= (uint64_t)kQsFar) return false;
    QsPlan pl;
    if (!qs_plan(B, K, N, 256, pl)) return false;
    return qs_fit(N, (int32_t)(K / group), pl);
}

hipError_t launch_gemm_qs(const void* X, const void* codes, const void* scales, const void* zeros, void* Y,
                          int64_t B, int64_t K, int64_t N, int32_t group, int num_cus, hipStream_t stream) {
    if (!qs_supports(B, K, N, group, 4) || reinterpret_cast<uintptr_t>(scales) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(zeros) % 16 != 0)
        return hipErrorInvalidValue;
    const int32_t ngrp = (int32_t)(K / group);
    QsPlan pl;
    if (!qs_plan(B, K, N, num_cus, pl) || !qs_fit(N, ngrp, pl)) return hipErrorInvalidValue;
    QsArgs a{static_cast<const uint16_t*>(X), static_cast<const uint8_t*>(codes),
             static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros),
             static_cast<uint16_t*>(Y), (int32_t)B, (int32_t)N, (int32_t)K, group, ngrp,
             (int32_t)((K + 511) / 512), pl.P, pl.R, (int32_t)((N + 3) / 4), pl.blocks * pl.R, pl.QB,
             (uint32_t)(K / 2), (uint32_t)((uint64_t)N * (uint64_t)(K / 2)),
             (uint32_t)((uint64_t)N * (uint64_t)ngrp * 2ull), (uint32_t)pl.half};
    if (B == 1) return launch_qs2<1>(a, pl, stream);
    if (B == 2) return launch_qs2<2>(a, pl, stream);
    return launch_qs2<4>(a, pl, stream);
}

}  // namespace wq
