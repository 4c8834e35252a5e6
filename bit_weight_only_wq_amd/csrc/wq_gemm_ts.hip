// Small-batch product (5 <= B <= 16 on matrices of fewer than 1.8 16-row
// tiles per compute unit) on the matrix cores' 16 x 16 x 32 blocks:
// Y[B,N] = X[B,K] * dequant(W)[N,K]^T.
//
// The decode product streams the packed weights once for the whole batch
// ("Quantization & inference optimisation", "Bandwidth, not compute"; "Serving
// many users at once", "Batching: one read, many users"), so the design is the
// quad-stream kernel's (wq_gemm_qs.hip), with 16-row tiles for the bigger
// matrix-core operation:
//   - an item is 16 weight rows (a tile) x 512 k: four 128-bit loads per lane,
//     each reading 4 rows x 256 bytes (lane l: row 4j + l / 16, bytes
//     16 (l % 16).. of the 256), the shape HBM serves at 6 TB/s and more, and
//     two 8-byte loads of the tile's group headers over those 512 k (one
//     group per 128-k round); these are the only loads in the main loop, 2
//     items ahead in a ring of registers (8 KB of codes per wave, 64 KB per
//     compute unit), so every wait in the loop is a counted one;
//   - v_mfma_f32_16x16x32_f16 wants 16 rows across the lanes instead, so each
//     item goes through the wave's own LDS tile (padded rows: no bank
//     conflicts either way) and comes back as lane (n, g): row n, 16 bytes of
//     each 128-k round, 4 words = 4 steps of 32 k (step s of round r takes
//     k = 128 r + 32 g + 8 s + 0..7 from lane group g);
//   - a wave keeps the same one or two 512-k positions of K for the whole
//     kernel and walks all its stream's tiles at the first, then at the
//     second, so only the first position's X (16 batch rows, the A operand,
//     in registers) is waited for before the stream starts; the P waves of a
//     row stream split K between them;
//   - codes unpack exactly to fp16 1024 + q (even k) and 64 + q (odd k); each
//     round's accumulation starts at -C1 (the offsets' weighted X sum, kept
//     in LDS with the plain sum C2) and the round's group header is applied
//     once in fp32 ("the kernel reconstructs an approximate float from the
//     integer and the endpoints as it reads", "Quantization"):
//         sum_k (q - z) s x = s * (sum_k u_k x_k - C1 - z * C2);
//   - a wave's 16 x 16 sums of a tile go to LDS (added to on its second
//     position); after the last tile the block adds the P waves' sums of
//     every output in wave order (deterministic) and writes Y.  The loop has
//     no barrier.
// Loads past the last row or the stream's end fall outside the buffer and
// return zero without touching memory.  No scratch memory.  Requires 4-bit
// codes, group 128, K % 512 == 0, 8-byte aligned header arrays and K <= 8192
// (at most two positions per wave).
#include <type_traits>

#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

namespace {

constexpr int TS_W = 8;                   // waves per block (one block per compute unit)
constexpr int TS_D = 2;                   // items in flight per wave
constexpr int TS_ROW = 256 + 16;          // LDS row of a wave's tile (bytes, padded)
constexpr int TS_TILE_LDS = TS_W * 16 * TS_ROW;
constexpr int TS_MAX_LDS = 160 * 1024;
constexpr int kTsBufWord3 = 0x00020000;   // raw, unswizzled gfx9 buffer
constexpr uint32_t kTsFar = 0x80000000u;  // a per-lane offset past every buffer this kernel reads

typedef unsigned int ts_v4u __attribute__((ext_vector_type(4)));
typedef unsigned int ts_v2u __attribute__((ext_vector_type(2)));

struct TsArgs {
    const uint16_t* X;
    const uint8_t* codes;
    const uint16_t* scales;
    const uint16_t* zeros;
    uint16_t* Y;
    int32_t B, N, K;
    int32_t ngrp;          // groups (128-k rounds) per row
    int32_t npos;          // 512-k positions (the last may be partial)
    int32_t P, R;          // waves per row stream, row streams per block
    int32_t ntiles;        // tiles of 16 rows
    int32_t S;             // row streams in the grid
    int32_t QB;            // tiles per stream at most
    uint32_t row_bytes;    // K / 2
    uint32_t code_bytes;   // N * K / 2
    uint32_t hdr_bytes;    // N * ngrp * 2
};

// LDS: the waves' tiles; their round sums, [wave][NPW][-C1, C2][4 rounds][16
// batch rows] floats; the waves' per-tile sums, [R][QB][P][64 lanes][4] floats.
constexpr size_t ts_csum_lds(int npw) { return (size_t)TS_W * npw * 2 * 4 * 16 * sizeof(float); }
size_t ts_red_lds(int R, int QB, int P) { return (size_t)R * QB * P * 1024; }

__device__ __forceinline__ uint4 ts_order8(uint4 in) {
    uint4 o;
    o.x = __builtin_amdgcn_perm(in.z, in.x, 0x05040100u);   // x0 | x4 << 16
    o.y = __builtin_amdgcn_perm(in.z, in.x, 0x07060302u);   // x1 | x5 << 16
    o.z = __builtin_amdgcn_perm(in.w, in.y, 0x05040100u);   // x2 | x6 << 16
    o.w = __builtin_amdgcn_perm(in.w, in.y, 0x07060302u);   // x3 | x7 << 16
    return o;
}

// Tiles of a row stream: tile st + q * S for q < the stream's count.
__device__ __forceinline__ uint32_t ts_tile(const TsArgs& a, int st, int q) { return (uint32_t)(st + q * a.S); }
__device__ __forceinline__ int ts_nt(const TsArgs& a, int st) {
    return st < a.ntiles ? (a.ntiles - st + a.S - 1) / a.S : 0;
}

// The block meets with its LDS writes done (loads stay in flight).
__device__ __forceinline__ void ts_meet() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0) only
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// NPW: positions per wave (1 or 2).
template <int NPW>
__global__ __launch_bounds__(TS_W * 64, 1) void gemm_ts_kernel(const TsArgs a) {
    extern __shared__ __align__(16) unsigned char ts_lds[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nwaves = a.R * a.P;
    const int r16 = lane & 15;           // matrix-core row / column of this lane
    const int g4 = lane >> 4;            // its k group (and its D rows 4 g4 .. 4 g4 + 3)
    const int rs = wave / a.P;           // row stream of the block
    const int pw = wave - rs * a.P;      // wave within the stream
    const int stream = blockIdx.x * a.R + rs;
    const int nt = ts_nt(a, stream);     // <= QB
    // Each pass (one position) walks the stream's tiles; a pass is padded to
    // whole rings, so ring slot = item % TS_D in both passes.
    const int ntp = (nt + TS_D - 1) / TS_D * TS_D;
    unsigned char* const tb = ts_lds + (size_t)wave * 16 * TS_ROW;
    float* const csum = reinterpret_cast<float*>(ts_lds + TS_TILE_LDS) + (size_t)wave * NPW * 128;
    float* const red_all = reinterpret_cast<float*>(ts_lds + TS_TILE_LDS + ts_csum_lds(NPW));

    // Per position slot: its position, this lane's code offset within a tile
    // and its header offset (row r16's 4 groups of the position, 8 bytes).
    int pos[NPW];
    uint32_t coff[NPW], hoff[NPW];
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
        pos[i] = pw + i * a.P;
        const bool real = pos[i] < a.npos;
        coff[i] = real ? (uint32_t)g4 * a.row_bytes + (uint32_t)pos[i] * 256u + 16u * (uint32_t)r16 : kTsFar;
        hoff[i] = real ? (uint32_t)(r16 * a.ngrp + 4 * pos[i]) * 2u : kTsFar;
    }

    // ---- X of a position slot (registers) ---------------------------------------
    // Lane (i, g) = (r16, g4) holds batch row i at k = 512 p + 128 r + 32 g +
    // 8 v (round r, vector v = 0..3).  Rows past B read zero.
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.X), (short)0, (int)((uint32_t)a.B * (uint32_t)a.K * 2u), kTsBufWord3);
    uint4 xa[NPW][4][4];
    auto load_x = [&](int i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t k0 = (int64_t)pos[i] * 512 + 128 * r + 32 * g4;
            const bool live = pos[i] < a.npos && r16 < a.B && k0 < a.K;
            const uint32_t xo = live ? (uint32_t)(((int64_t)r16 * a.K + k0) * 2) : kTsFar;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const ts_v4u t = __builtin_amdgcn_raw_buffer_load_b128(xrs, (int)(xo + 16u * v), 0, 0);
                xa[i][r][v] = make_uint4(t.x, t.y, t.z, t.w);
            }
        }
    };
    // Round sums C1 (offset-weighted) and C2 (plain) of each batch row into
    // this wave's LDS (the lane's 32 k, then the four k groups: lanes 16
    // apart); X permuted into the order the codes unpack in.
    auto prep_x = [&](int i) {
        const h2_t one = {(_Float16)1.0f, (_Float16)1.0f};
        const h2_t wgt = {(_Float16)1024.0f, (_Float16)64.0f};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float d1 = 0.0f, d2 = 0.0f;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const uint4 x = xa[i][r][v];
                d2 = __builtin_amdgcn_fdot2(as_h2(x.x), one, d2, false);
                d2 = __builtin_amdgcn_fdot2(as_h2(x.y), one, d2, false);
                d2 = __builtin_amdgcn_fdot2(as_h2(x.z), one, d2, false);
                d2 = __builtin_amdgcn_fdot2(as_h2(x.w), one, d2, false);
                d1 = __builtin_amdgcn_fdot2(as_h2(x.x), wgt, d1, false);
                d1 = __builtin_amdgcn_fdot2(as_h2(x.y), wgt, d1, false);
                d1 = __builtin_amdgcn_fdot2(as_h2(x.z), wgt, d1, false);
                d1 = __builtin_amdgcn_fdot2(as_h2(x.w), wgt, d1, false);
                xa[i][r][v] = ts_order8(x);
            }
            d1 += __shfl_xor(d1, 16, 64);
            d2 += __shfl_xor(d2, 16, 64);
            d1 += __shfl_xor(d1, 32, 64);
            d2 += __shfl_xor(d2, 32, 64);
            if (g4 == 0) {
                csum[((i * 2 + 0) * 4 + r) * 16 + r16] = -d1;
                csum[((i * 2 + 1) * 4 + r) * 16 + r16] = d2;
            }
        }
    };

    // ---- the ring ---------------------------------------------------------------------
    // Item it = pass it / ntp (position slot), tile index it % ntp (nothing
    // for indices past the stream's count).  Load j of an item reads rows
    // 4j .. 4j + 3 of the tile, lane l row 4j + l / 16 at 16 (l % 16); the
    // headers: row r16's 4 groups, scales then zeros.
    struct Item {
        uint4 c[4];
        ts_v2u s, z;
    };
    const uint32_t tile_cb = 16u * a.row_bytes, tile_hb = 32u * (uint32_t)a.ngrp;
    // Item it's buffers: each starts at its tile and ends at the matrix's end.
    auto item_bufs = [&](int it, __amdgpu_buffer_rsrc_t& crs, __amdgpu_buffer_rsrc_t& srs,
                         __amdgpu_buffer_rsrc_t& zrs, uint32_t& co, uint32_t& ho) {
        const int i = it >= ntp ? 1 : 0;                 // (NPW == 1: items past ntp read nothing)
        const int q = it - i * ntp;
        const bool live = q < nt && i < NPW;
        const uint32_t tile = ts_tile(a, stream, q);
        const uint32_t cb = live ? tile * tile_cb : 0u, hb = live ? tile * tile_hb : 0u;
        crs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.codes + cb), (short)0,
                                                live ? (int)(a.code_bytes - cb) : 0, kTsBufWord3);
        const int hleft = live ? (int)(a.hdr_bytes - hb) : 0;
        srs = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(a.scales)) + hb,
                                                (short)0, hleft, kTsBufWord3);
        zrs = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(a.zeros)) + hb,
                                                (short)0, hleft, kTsBufWord3);
        co = NPW == 1 || i == 0 ? coff[0] : coff[NPW - 1];
        ho = NPW == 1 || i == 0 ? hoff[0] : hoff[NPW - 1];
    };
    auto load_codes = [&](int it, Item& dst) {
        __amdgpu_buffer_rsrc_t crs, srs, zrs;
        uint32_t co, ho;
        item_bufs(it, crs, srs, zrs, co, ho);
#pragma unroll
        for (int jl = 0; jl < 4; ++jl) {
            const ts_v4u t = __builtin_amdgcn_raw_buffer_load_b128(crs, (int)(co + 4u * (uint32_t)jl * a.row_bytes), 0, 2);
            dst.c[jl] = make_uint4(t.x, t.y, t.z, t.w);
        }
    };
    auto load_hdr = [&](int it, Item& dst) {
        __amdgpu_buffer_rsrc_t crs, srs, zrs;
        uint32_t co, ho;
        item_bufs(it, crs, srs, zrs, co, ho);
        dst.s = __builtin_amdgcn_raw_buffer_load_b64(srs, (int)ho, 0, 0);
        dst.z = __builtin_amdgcn_raw_buffer_load_b64(zrs, (int)ho, 0, 0);
    };

    // Start: the first position's X, the ring, then the second position's X
    // (its wait comes only at the second pass).
    load_x(0);
    Item ring[TS_D];
#pragma unroll
    for (int d = 0; d < TS_D; ++d) {
        load_codes(d, ring[d]);
        load_hdr(d, ring[d]);
    }
    if constexpr (NPW == 2) load_x(1);
    prep_x(0);

    // ---- the stream -------------------------------------------------------------------
    const uint32_t m_lo = vgpr_const(0x000F000Fu), m_hi = vgpr_const(0x00F000F0u);
    const uint32_t g_lo = vgpr_const(0x64006400u), g_hi = vgpr_const(0x54005400u);
    float* const red = red_all + (size_t)rs * a.QB * a.P * 256;

    // The item's 4 loads -> the wave's tile (row 4j + l / 16, 16 bytes at
    // 16 (l % 16)).
    auto stage = [&](const Item& it) {
#pragma unroll
        for (int jl = 0; jl < 4; ++jl)
            *reinterpret_cast<uint4*>(tb + (4 * jl + g4) * TS_ROW + 16 * r16) = it.c[jl];
    };
    // One item from the wave's tile (position slot I, tile index q, headers
    // s4/z4): 4 rounds x 4 steps, then the headers; the tile's sums go to (or
    // are added to) this wave's LDS entry.
    auto compute = [&](auto I, int q, ts_v2u s4, ts_v2u z4) {
        constexpr int i = decltype(I)::value;
        f4_t tot = {0.0f, 0.0f, 0.0f, 0.0f};
        if (pos[i] < a.npos) {
            uint4 ch[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ch[r] = *reinterpret_cast<const uint4*>(tb + r16 * TS_ROW + 64 * r + 16 * g4);
            f4_t acc[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[r] = *reinterpret_cast<const f4_t*>(&csum[((i * 2 + 0) * 4 + r) * 16 + 4 * g4]);
            // Step s of the four rounds goes out before step s + 1: four
            // independent accumulation chains.
#pragma unroll
            for (int st = 0; st < 4; ++st)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t w = st == 0 ? ch[r].x : st == 1 ? ch[r].y : st == 2 ? ch[r].z : ch[r].w;
                    const uint32_t w8 = w >> 8;
                    const uint4 b = make_uint4((w & m_lo) | g_lo, (w & m_hi) | g_hi, (w8 & m_lo) | g_lo,
                                               (w8 & m_hi) | g_hi);
                    acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, xa[i][r][st]),
                                                                    __builtin_bit_cast(h8_t, b), acc[r], 0, 0, 0);
                }
            const uint32_t sw[2] = {s4.x, s4.y}, zw[2] = {z4.x, z4.y};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float sc = (r & 1) ? (float)as_h2(sw[r >> 1]).y : (float)as_h2(sw[r >> 1]).x;
                const float ze = (r & 1) ? (float)as_h2(zw[r >> 1]).y : (float)as_h2(zw[r >> 1]).x;
                const f4_t c2 = *reinterpret_cast<const f4_t*>(&csum[((i * 2 + 1) * 4 + r) * 16 + 4 * g4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) tot[e] = __builtin_fmaf(sc, __builtin_fmaf(-ze, c2[e], acc[r][e]), tot[e]);
            }
        }
        f4_t* const dst = reinterpret_cast<f4_t*>(&red[((size_t)q * a.P + pw) * 256 + 4 * lane]);
        if constexpr (i == 0) *dst = tot;
        else *dst = *dst + tot;
    };
    auto pass = [&](auto I) {
        constexpr int i = decltype(I)::value;
        for (int q0 = 0; q0 < ntp; q0 += TS_D) {
#pragma unroll
            for (int d = 0; d < TS_D; ++d) {
                const int q = q0 + d;
                if (q < nt) stage(ring[d]);
                // The code registers are free once the item is in the tile:
                // refill them now; the header registers after their use (so
                // no value moves between registers across the loop).
                load_codes(i * ntp + q + TS_D, ring[d]);
                asm volatile("" ::: "memory");
                if (q < nt) compute(I, q, ring[d].s, ring[d].z);
                load_hdr(i * ntp + q + TS_D, ring[d]);
            }
        }
    };
    pass(std::integral_constant<int, 0>{});
    if constexpr (NPW == 2) {
        prep_x(1);
        pass(std::integral_constant<int, 1>{});
    }
    ts_meet();

    // ---- Y: the P waves' sums of every output, in wave order -------------
    // Output (tile q, weight row n, batch row b) sits with lane n + 16 (b / 4),
    // element b % 4.
    const int per_stream = a.QB * 16 * a.B;
    for (int o = threadIdx.x; o < a.R * per_stream; o += nwaves * 64) {
        const int r = o / per_stream;
        const int rem = o - r * per_stream;
        const int b = rem % a.B;
        const int qn = rem / a.B;
        const int q = qn >> 4, n = qn & 15;
        const int st_r = blockIdx.x * a.R + r;
        const int64_t row = (int64_t)ts_tile(a, st_r, q) * 16 + n;
        if (q >= ts_nt(a, st_r) || row >= a.N) continue;
        const float* src = red_all + (((size_t)r * a.QB + q) * a.P) * 256 + 4 * (n + 16 * (b >> 2)) + (b & 3);
        float t = 0.0f;
        for (int w = 0; w < a.P; ++w) t += src[(size_t)w * 256];
        a.Y[(int64_t)b * a.N + row] = float_to_half_bits_rne(t);
    }
    // Loads issued past the end: let them land before the block ends.
    __builtin_amdgcn_s_waitcnt(0);
}

struct TsPlan {
    int npw, P, R, blocks, QB;
    size_t lds;
};

// Positions per wave, waves per stream, streams per block, then the grid,
// grown until the per-tile sums fit in LDS.
bool ts_plan(int64_t K, int64_t N, int num_cus, TsPlan& pl) {
    const int64_t npos = (K + 511) / 512;
    const int npw = npos <= TS_W ? 1 : 2;
    if (npos > (int64_t)TS_W * npw) return false;
    const int P = (int)((npos + npw - 1) / npw);
    const int R = TS_W / P;
    const int64_t ntiles = (N + 15) / 16;
    int64_t blocks = (ntiles + R - 1) / R;
    if (blocks > num_cus) blocks = num_cus;
    for (;;) {
        const int64_t S = blocks * R;
        const int QB = (int)((ntiles + S - 1) / S);
        const size_t lds = TS_TILE_LDS + ts_csum_lds(npw) + ts_red_lds(R, QB, P);
        if (lds <= (size_t)TS_MAX_LDS) {
            pl = TsPlan{npw, P, R, (int)blocks, QB, lds};
            return true;
        }
        if (blocks >= ntiles) return false;
        blocks = blocks * 2 < ntiles ? blocks * 2 : ntiles;
    }
}

}  // namespace

bool ts_supports(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits) {
    if (bits != 4 || B < 1 || B > 16 || K < 512 || K % 512 != 0 || group != 128 || N < 1) return false;
    // 32-bit buffer offsets with room for the far offset.
    if ((uint64_t)N * (uint64_t)(K / 2) + 32ull * (uint64_t)K >= (uint64_t)kTsFar) return false;
    if ((uint64_t)N * (uint64_t)(K / group) * 2ull + 32ull * (uint64_t)K >= (uint64_t)kTsFar) return false;
    if ((uint64_t)B * (uint64_t)K * 2ull >= (uint64_t)kTsFar) return false;
    TsPlan pl;
    return ts_plan(K, N, 256, pl);
}

hipError_t launch_gemm_ts(const void* X, const void* codes, const void* scales, const void* zeros, void* Y,
                          int64_t B, int64_t K, int64_t N, int32_t group, int num_cus, hipStream_t stream) {
    if (!ts_supports(B, K, N, group, 4) || reinterpret_cast<uintptr_t>(scales) % 8 != 0 ||
        reinterpret_cast<uintptr_t>(zeros) % 8 != 0)
        return hipErrorInvalidValue;
    TsPlan pl;
    if (!ts_plan(K, N, num_cus, pl)) return hipErrorInvalidValue;
    const int32_t ngrp = (int32_t)(K / group);
    TsArgs a{static_cast<const uint16_t*>(X), static_cast<const uint8_t*>(codes),
             static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(zeros),
             static_cast<uint16_t*>(Y), (int32_t)B, (int32_t)N, (int32_t)K, ngrp,
             (int32_t)((K + 511) / 512), pl.P, pl.R, (int32_t)((N + 15) / 16), pl.blocks * pl.R, pl.QB,
             (uint32_t)(K / 2), (uint32_t)((uint64_t)N * (uint64_t)(K / 2)),
             (uint32_t)((uint64_t)N * (uint64_t)ngrp * 2ull)};
    const dim3 grid((unsigned)pl.blocks), block((unsigned)(pl.R * pl.P * 64));
    if (pl.npw == 1)
        gemm_ts_kernel<1><<<grid, block, pl.lds, stream>>>(a);
    else
        gemm_ts_kernel<2><<<grid, block, pl.lds, stream>>>(a);
    return hipGetLastError();
}

}  // namespace wq
