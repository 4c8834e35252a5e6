// Matrix-core product for small batches (B <= 32) with the activations held in
// LDS: Y[B,N] = X[B,K] * dequant(W)[N,K]^T.
//
// A decode step reads every weight once for the whole batch ("Quantization &
// inference optimisation", "Bandwidth, not compute"), so the kernel is built
// around one continuous stream of packed codes, like the GEMV path:
//   - a block (one per compute unit: 16 waves, or 8 when B > 16 puts two
//     16-column blocks in each wave) copies a K-slice of X (all B rows, up to
//     128 KB) into LDS once, permuted into the order the codes unpack in,
//     together with two weighted column sums per 128-k round, and never
//     synchronizes again;
//   - every wave then owns whole 16-row tiles of that slice and streams their
//     128-bit code chunks through a ring of registers that runs six to seven
//     rounds ahead, across tile boundaries; group headers arrive eight rounds at a
//     time as 128-bit loads when the layout allows;
//   - v_mfma_f32_16x16x32_f16 multiplies X (A operand, batch rows) by the codes
//     as exact fp16 integers (B operand, weight rows), and the group header is
//     applied per round to the fp32 result ("the kernel reconstructs an
//     approximate float from the integer and the endpoints as it reads",
//     "Quantization"):
//         sum_k (q - z) s x = s * (sum_k u_k x_k - C1 - z * C2)
//     where u_k is the unpacked code (q plus a fixed offset, below) and C1, C2
//     are the round's offset-weighted and plain sums of X;
//   - with several K-slices (when X does not fit in one slice, or to give small
//     matrices enough parallelism) each wave writes its tile's fp32 partial and
//     a second kernel adds the slices in slice order (deterministic).
//
// Unpack arithmetic.  A 32-bit code word holds 8 nibbles n0..n7 (k0..k7).  With
// the exponent bits of 1024 (ulp 1) and 64 (ulp 1/16) OR-ed in,
//   (w      & 0x000F000F) | 0x64006400 = (1024 + n0, 1024 + n4)
//   (w      & 0x00F000F0) | 0x54005400 = (  64 + n1,   64 + n5)
//   (w >> 8 & 0x000F000F) | 0x64006400 = (1024 + n2, 1024 + n6)
//   (w >> 8 & 0x00F000F0) | 0x54005400 = (  64 + n3,   64 + n7)
// exactly: even k carry +1024, odd k +64, so C1 = 1024 * sum_even x +
// 64 * sum_odd x.  The k order of an operand is (0,4,1,5,2,6,3,7) within each
// 8 k.  8-bit codes unpack as (1024 + b0, 1024 + b2), (1024 + b1, 1024 + b3),
// order (0,2,1,3) within each 4 k, C1 = 1024 * sum x.  X is stored in LDS in
// the same order.
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

namespace {

constexpr int XR_SLOTS = 8;      // register ring of code chunks, refilled two rounds at a time

// How a wave gets the group headers of its rows.
enum XrHeader {
    XR_HDR_ROUND = 0,   // one 16-bit load of s and of z per round (any group size)
    XR_HDR_TURN = 1,    // one group per round: 8 groups per 128-bit load
    XR_HDR_ROW = 2      // one group per row: loaded once per tile
};

// Waves per block (one block per compute unit): 16 while the registers of one
// 16-column block fit 128 per lane, 8 with two column blocks.
constexpr int xr_waves(int btx) { return btx > 16 ? 8 : 16; }

template <int BITS, int BTX>
struct XrGeom {
    static constexpr int VALS = 128 / BITS;        // codes per 16-byte chunk
    static constexpr int KR = 4 * VALS;            // k per round (4 lane groups)
    static constexpr int KSTEPS = KR / 32;         // 16x16x32 MFMAs per round
    static constexpr int SEGR = KR / 8;            // 16-byte X vectors per column and round
    static constexpr int KSL = 65536 / BTX;        // X slice length (halves): 128 KB of LDS
    static constexpr int ROW = KSL + 8;            // padded LDS row: rows land on distinct banks
    static constexpr int RMAX = KSL / KR;          // rounds per slice at most
    static constexpr int WAVES = xr_waves(BTX);
};

// One product of a launch, and the launch: up to XR_MAX_ITEMS products of
// one batch size, bit width and header mode, passed by value (the kernel
// reads the table from its argument segment with scalar loads).
constexpr int XR_MAX_ITEMS = 8;

struct XrItem {
    const uint16_t* X;
    const uint4* codes;
    const uint16_t* scales;
    const uint16_t* zeros;
    uint16_t* Y;
    float* part;          // fp32 partials [slices][B][N], or null with one slice
    int64_t N, K, ngrp;
    uint64_t rpg_magic;
    int32_t RS;           // rounds per slice
    int32_t per_slice;    // blocks per slice
    int32_t slices;
    int32_t block0;       // first block of this product
};

struct XrLaunch {
    XrItem it[XR_MAX_ITEMS];
    int64_t B;
    int32_t count;
};

// The reduction of a launch: every product with several slices, its outputs
// numbered from t0 in one flat index space.
struct XrReduceItem {
    const float* part;
    uint16_t* Y;
    int64_t count;        // B * N
    int64_t t0;
    int32_t slices;
    int32_t vec;          // count % 4 == 0 and Y 8-byte aligned: 16-byte partial loads
};

struct XrReduce {
    XrReduceItem it[XR_MAX_ITEMS];
    int32_t count;
};

// X vector reordered to the unpack order (see above).
template <int BITS>
__device__ __forceinline__ uint4 order8(uint4 in) {
    uint4 o;
    if constexpr (BITS == 4) {
        o.x = __builtin_amdgcn_perm(in.z, in.x, 0x05040100u);
        o.y = __builtin_amdgcn_perm(in.z, in.x, 0x07060302u);
        o.z = __builtin_amdgcn_perm(in.w, in.y, 0x05040100u);
        o.w = __builtin_amdgcn_perm(in.w, in.y, 0x07060302u);
    } else {
        o.x = __builtin_amdgcn_perm(in.y, in.x, 0x05040100u);
        o.y = __builtin_amdgcn_perm(in.y, in.x, 0x07060302u);
        o.z = __builtin_amdgcn_perm(in.w, in.z, 0x05040100u);
        o.w = __builtin_amdgcn_perm(in.w, in.z, 0x07060302u);
    }
    return o;
}

// Offset-weighted and plain sums of one natural-order X vector (products with
// 1, 64 and 1024 are exact in fp32).
template <int BITS>
__device__ __forceinline__ void offset_sums(uint4 v, float& c1, float& c2) {
    const h2_t one = {(_Float16)1.0f, (_Float16)1.0f};
    float s = __builtin_amdgcn_fdot2(as_h2(v.x), one, 0.0f, false);
    s = __builtin_amdgcn_fdot2(as_h2(v.y), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(v.z), one, s, false);
    s = __builtin_amdgcn_fdot2(as_h2(v.w), one, s, false);
    if constexpr (BITS == 4) {
        // Even k sit in the low halves of the words, odd k in the high halves.
        const h2_t wgt = {(_Float16)1024.0f, (_Float16)64.0f};
        float w = __builtin_amdgcn_fdot2(as_h2(v.x), wgt, 0.0f, false);
        w = __builtin_amdgcn_fdot2(as_h2(v.y), wgt, w, false);
        w = __builtin_amdgcn_fdot2(as_h2(v.z), wgt, w, false);
        c1 = __builtin_amdgcn_fdot2(as_h2(v.w), wgt, w, false);
    } else {
        c1 = 1024.0f * s;
    }
    c2 = s;
}

struct Consts {
    uint32_t m_lo, m_hi, g_lo, g_hi;  // nibble/byte masks and exponent patterns
};

// B operand of k-step j of one lane's chunk: the unpacked codes (see above).
template <int BITS>
__device__ __forceinline__ h8_t unpack(const uint4& cw, int j, const Consts& c) {
    uint4 b;
    if constexpr (BITS == 4) {
        const uint32_t w = j == 0 ? cw.x : j == 1 ? cw.y : j == 2 ? cw.z : cw.w;
        const uint32_t w8 = w >> 8;
        b.x = (w & c.m_lo) | c.g_lo;
        b.y = (w & c.m_hi) | c.g_hi;
        b.z = (w8 & c.m_lo) | c.g_lo;
        b.w = (w8 & c.m_hi) | c.g_hi;
    } else {
        const uint32_t w0 = j == 0 ? cw.x : cw.z;
        const uint32_t w1 = j == 0 ? cw.y : cw.w;
        b.x = (w0 & c.m_lo) | c.g_lo;
        b.y = ((w0 >> 8) & c.m_lo) | c.g_lo;
        b.z = (w1 & c.m_lo) | c.g_lo;
        b.w = ((w1 >> 8) & c.m_lo) | c.g_lo;
    }
    return __builtin_bit_cast(h8_t, b);
}

// Half i (0..7) of a 128-bit vector of fp16 values, as float.
__device__ __forceinline__ float half_of(const uint4& v, int i) {
    const uint32_t w = i < 4 ? (i < 2 ? v.x : v.y) : (i < 6 ? v.z : v.w);
    return (i & 1) ? (float)as_h2(w).y : (float)as_h2(w).x;
}

// Grid: one dimension over the products of the launch.  Product i owns blocks
// [block0, block0 + per_slice * slices); its block b works on K-slice
// b / per_slice, which covers rounds [slice*RS, (slice+1)*RS) (RS a multiple
// of XR_SLOTS; rounds past K meet zero X in LDS and add nothing), as block
// x = b % per_slice of that slice.  Tiles are 16 weight rows; wave w of
// block x owns tiles w*per_slice + x + i*stride, so every block has work.
// With several slices, part receives fp32 partials [slice][b][n].  For
// XR_HDR_ROUND the group of round r is (r * rpg_magic) >> 32 =
// floor(r / (G / KR)), exact for r < 2^16 with rpg_magic = ceil(2^32 / (G / KR)).
template <int BITS, int BTX, int HM>
__global__ __launch_bounds__(xr_waves(BTX) * 64) void gemm_xr_kernel(const XrLaunch L) {
    typedef XrGeom<BITS, BTX> XG;
    // This block's product (a uniform scan of the launch table).
    int item = 0;
#pragma unroll
    for (int j = 1; j < XR_MAX_ITEMS; ++j)
        if (j < L.count && (int)blockIdx.x >= L.it[j].block0) item = j;
    const XrItem& P = L.it[item];
    const uint16_t* __restrict__ X = P.X;
    const uint4* __restrict__ codes = P.codes;
    const uint16_t* __restrict__ scales = P.scales;
    const uint16_t* __restrict__ zeros = P.zeros;
    uint16_t* __restrict__ Y = P.Y;
    float* __restrict__ part = P.part;
    const int64_t B = L.B, N = P.N, K = P.K, ngrp = P.ngrp;
    const uint64_t rpg_magic = P.rpg_magic;
    const int32_t RS = P.RS;
    const int lb = (int)blockIdx.x - P.block0;
    const int slice = lb / P.per_slice;
    const int bx = lb - slice * P.per_slice;
    constexpr int NCB = (BTX + 15) / 16;                   // 16-column blocks
    __shared__ __align__(16) uint16_t xs[BTX * XG::ROW];
    __shared__ __align__(16) float cneg1[XG::RMAX][BTX];   // -C1 per (round, column)
    __shared__ __align__(16) float csum2[XG::RMAX][BTX];   //  C2 per (round, column)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15;
    const int g4 = lane >> 4;
    const int64_t rounds = K / XG::KR;
    const int64_t round0 = (int64_t)slice * RS;               // first round of the slice
    const int64_t ntiles = (N + 15) / 16;
    const int64_t stride = (int64_t)P.per_slice * XG::WAVES;
    const int64_t t0 = (int64_t)wave * P.per_slice + bx;
    const int64_t chunks_per_row = K / XG::VALS;

    // Weight row r16 of tile t, clamped to N - 1 (tiles past the end reread
    // the last row; their results are never stored).
    auto tile_row = [&](int64_t t) -> int64_t {
        const int64_t tt = t < ntiles ? t : ntiles - 1;
        const int64_t row = tt * 16 + r16;
        return row < N ? row : N - 1;
    };

    // ---- X slice: issue its loads first --------------------------------------
    // Row c of xs holds X[c, slice] in the unpack order, 8 k per 16-byte vector;
    // columns past B, k past K and vectors past the slice are zero.  These
    // loads go out before the ring's, so waiting for them leaves the code
    // stream in flight.
    constexpr int VROW = XG::KSL / 8;                              // vectors per LDS row
    constexpr int FILL = BTX * VROW / (XG::WAVES * 64);             // vectors per thread
    const int vec_used = RS * XG::SEGR;                            // vectors of this slice
    const int64_t k0 = round0 * XG::KR;
    uint4 xv[FILL];
#pragma unroll
    for (int u = 0; u < FILL; ++u) {
        const int v = tid + u * XG::WAVES * 64;
        const int col = v / VROW, seg = v % VROW;
        const int64_t k = k0 + (int64_t)seg * 8;
        const bool ok = col < B && seg < vec_used && k < K;
        xv[u] = *reinterpret_cast<const uint4*>(ok ? X + col * K + k : X);
    }

    // ---- the load ring ------------------------------------------------------
    // Rounds past K read the last round again; they meet zero X and zero sums.
    uint4 cw[XR_SLOTS];
    auto load_codes = [&](int slot, const uint4* pc, int64_t lr) {
        int64_t ra = round0 + lr;
        ra = ra < rounds ? ra : rounds - 1;
        cw[slot] = pc[ra * 4];
    };
    // Headers.  ROUND: per slot; TURN: 8 rounds per 128-bit load, one turn
    // ahead; ROW: per tile, one tile ahead.
    uint32_t hs[XR_SLOTS], hz[XR_SLOTS];
    uint4 hsc, hzc, hsn, hzn;             // TURN: current and next turn
    uint32_t ts_c, tz_c, ts_n, tz_n;      // ROW: current and next tile
    auto load_hdr_round = [&](int slot, int64_t hrow, int64_t lr) {
        int64_t ra = round0 + lr;
        ra = ra < rounds ? ra : rounds - 1;
        const int64_t gi = hrow + (int64_t)(((uint64_t)ra * rpg_magic) >> 32);
        hs[slot] = scales[gi];
        hz[slot] = zeros[gi];
    };
    auto load_hdr_turn = [&](int64_t hrow, int64_t lr) {
        int64_t ga = round0 + lr;                 // one group per round: ngrp == rounds
        ga = ga + 8 <= rounds ? ga : rounds - 8;
        hsn = *reinterpret_cast<const uint4*>(scales + hrow + ga);
        hzn = *reinterpret_cast<const uint4*>(zeros + hrow + ga);
    };

    int64_t t = t0;
    const uint4* pc = codes + tile_row(t) * chunks_per_row + g4;
    int64_t ph = tile_row(t) * ngrp;
    const uint4* nc = codes + tile_row(t + stride) * chunks_per_row + g4;
    int64_t nh = tile_row(t + stride) * ngrp;
    if constexpr (HM == XR_HDR_TURN) load_hdr_turn(ph, 0);
    if constexpr (HM == XR_HDR_ROW) {
        ts_c = scales[ph];
        tz_c = zeros[ph];
        ts_n = scales[nh];
        tz_n = zeros[nh];
    }
#pragma unroll
    for (int s = 0; s < XR_SLOTS - 2; ++s) {
        load_codes(s, pc, s);
        if constexpr (HM == XR_HDR_ROUND) load_hdr_round(s, ph, s);
    }

    // ---- X slice -> LDS, with its per-round column sums ---------------------
#pragma unroll
    for (int u = 0; u < FILL; ++u) {
        const int v = tid + u * XG::WAVES * 64;
        const int col = v / VROW, seg = v % VROW;
        const int64_t k = k0 + (int64_t)seg * 8;
        const uint4 x = col < B && seg < vec_used && k < K ? xv[u] : uint4{0u, 0u, 0u, 0u};
        float c1, c2;
        offset_sums<BITS>(x, c1, c2);
        // The SEGR vectors of one (column, round) sit in adjacent lanes.
        c1 = group_sum<XG::SEGR>(c1);
        c2 = group_sum<XG::SEGR>(c2);
        if (seg < vec_used) {
            *reinterpret_cast<uint4*>(&xs[col * XG::ROW + seg * 8]) = order8<BITS>(x);
            if (seg % XG::SEGR == 0) {
                cneg1[seg / XG::SEGR][col] = -c1;
                csum2[seg / XG::SEGR][col] = c2;
            }
        }
    }
    // Only the LDS writes need to be complete here; the code loads issued
    // above keep streaming through the barrier.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    const Consts cst = BITS == 4 ? Consts{vgpr_const(0x000F000Fu), vgpr_const(0x00F000F0u), vgpr_const(0x64006400u), vgpr_const(0x54005400u)}
                                 : Consts{vgpr_const(0x00FF00FFu), 0u, vgpr_const(0x64006400u), 0u};
    // A operand of column block cb: batch row cb*16 + r16 (mod BTX), 8 k at the
    // lane group's offset.  Accumulator lane layout: batch rows
    // cb*16 + 4*g4 + i (mod BTX), weight row r16.  The unpacked codes of a
    // k-step feed every column block.
    const uint16_t* xa[NCB];
    int cbase[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        xa[cb] = &xs[((cb * 16 + r16) % BTX) * XG::ROW + g4 * XG::VALS];
        cbase[cb] = (cb * 16 + 4 * g4) % BTX;
    }

    f4_t tot[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) tot[cb] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
    auto compute = [&](int slot, int lr, float s, float z) {
        f4_t acc[NCB], c2[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            acc[cb] = *reinterpret_cast<const f4_t*>(&cneg1[lr][cbase[cb]]);
            c2[cb] = *reinterpret_cast<const f4_t*>(&csum2[lr][cbase[cb]]);
        }
#pragma unroll
        for (int j = 0; j < XG::KSTEPS; ++j) {
            const h8_t b = unpack<BITS>(cw[slot], j, cst);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const h8_t a = __builtin_bit_cast(
                    h8_t, *reinterpret_cast<const uint4*>(xa[cb] + lr * XG::KR + 8 * j));
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[cb], 0, 0, 0);
            }
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                tot[cb][i] = __builtin_fmaf(s, __builtin_fmaf(-z, c2[cb][i], acc[cb][i]), tot[cb][i]);
    };
    // Header of step k of a turn (values for round it*8 + k).
    auto hdr_s = [&](int k) -> float {
        if constexpr (HM == XR_HDR_ROUND) return half_bits_to_float((uint16_t)hs[k]);
        else if constexpr (HM == XR_HDR_TURN) return half_of(hsc, k);
        else return half_bits_to_float((uint16_t)ts_c);
    };
    auto hdr_z = [&](int k) -> float {
        if constexpr (HM == XR_HDR_ROUND) return half_bits_to_float((uint16_t)hz[k]);
        else if constexpr (HM == XR_HDR_TURN) return half_of(hzc, k);
        else return half_bits_to_float((uint16_t)tz_c);
    };

    const int nit = RS / XR_SLOTS;
    for (; t < ntiles; t += stride) {
        // Steps of one ring turn: compute round it*8 + k of tile t.  Every
        // second step refills the two slots computed in the two steps before
        // with the rounds six and seven ahead (of this tile or, late in the
        // last turn, of the next tile): the pair covers whole 128-byte lines
        // of each row, so the two loads leave the L1 as one request per line.
        for (int it = 0; it < nit - 1; ++it) {
            if constexpr (HM == XR_HDR_TURN) {
                hsc = hsn;
                hzc = hzn;
                load_hdr_turn(ph, (int64_t)(it + 1) * XR_SLOTS);
            }
#pragma unroll
            for (int k = 0; k < XR_SLOTS; ++k) {
                if (k % 2 == 0) {
#pragma unroll
                    for (int d = 6; d < 8; ++d) {
                        const int ls = (k + d) % XR_SLOTS;
                        load_codes(ls, pc, it * XR_SLOTS + k + d);
                        if constexpr (HM == XR_HDR_ROUND) load_hdr_round(ls, ph, it * XR_SLOTS + k + d);
                    }
                }
                compute(k, it * XR_SLOTS + k, hdr_s(k), hdr_z(k));
            }
        }
        {
            const int it = nit - 1;
            if constexpr (HM == XR_HDR_TURN) {
                hsc = hsn;
                hzc = hzn;
                load_hdr_turn(nh, 0);
            }
#pragma unroll
            for (int k = 0; k < XR_SLOTS; ++k) {
                if (k % 2 == 0) {
#pragma unroll
                    for (int d = 6; d < 8; ++d) {
                        const int ls = (k + d) % XR_SLOTS;
                        if (k + d < XR_SLOTS) {
                            load_codes(ls, pc, it * XR_SLOTS + k + d);
                            if constexpr (HM == XR_HDR_ROUND) load_hdr_round(ls, ph, it * XR_SLOTS + k + d);
                        } else {
                            load_codes(ls, nc, k + d - XR_SLOTS);
                            if constexpr (HM == XR_HDR_ROUND) load_hdr_round(ls, nh, k + d - XR_SLOTS);
                        }
                    }
                }
                compute(k, it * XR_SLOTS + k, hdr_s(k), hdr_z(k));
            }
        }
        const int64_t row = t * 16 + r16;
        const int bmax = (int)(B < BTX ? B : BTX);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const bool mine = row < N && cb * 16 + 4 * g4 < BTX;
            if (!part) {
                if (mine) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int col = cb * 16 + 4 * g4 + i;
                        if (col < bmax) Y[col * N + row] = float_to_half_bits_rne(tot[cb][i]);
                    }
                }
            } else if (mine) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int col = cb * 16 + 4 * g4 + i;
                    if (col < bmax) part[((int64_t)slice * B + col) * N + row] = tot[cb][i];
                }
            }
            tot[cb] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
        pc = nc;
        ph = nh;
        nc = codes + tile_row(t + 2 * stride) * chunks_per_row + g4;
        nh = tile_row(t + 2 * stride) * ngrp;
        if constexpr (HM == XR_HDR_ROW) {
            ts_c = ts_n;
            tz_c = tz_n;
            ts_n = scales[nh];
            tz_n = zeros[nh];
        }
    }
}

// Y = fp16(sum over slices of part[z]), slices added in order 0, 1, 2, ...,
// for every product of the table (one flat index space over their outputs).
__global__ __launch_bounds__(256) void xr_reduce_kernel(const XrReduce R) {
    // Each thread sums four consecutive outputs; products start on
    // 1024-output boundaries, so the product is uniform per block.
    const int64_t g0 = (int64_t)blockIdx.x * 1024;
    int item = 0;
#pragma unroll
    for (int j = 1; j < XR_MAX_ITEMS; ++j)
        if (j < R.count && g0 >= R.it[j].t0) item = j;
    const XrReduceItem& P = R.it[item];
    const int64_t i0 = g0 - P.t0 + 4 * (int64_t)threadIdx.x;
    if (i0 >= P.count) return;
    if (P.vec) {
        const float4* p4 = reinterpret_cast<const float4*>(P.part);
        const int64_t c4 = P.count / 4, j = i0 / 4;
        float4 s = p4[j];
        for (int z = 1; z < P.slices; ++z) {
            const float4 v = p4[(int64_t)z * c4 + j];
            s.x += v.x;
            s.y += v.y;
            s.z += v.z;
            s.w += v.w;
        }
        reinterpret_cast<uint2*>(P.Y)[j] =
            make_uint2((uint32_t)float_to_half_bits_rne(s.x) | ((uint32_t)float_to_half_bits_rne(s.y) << 16),
                       (uint32_t)float_to_half_bits_rne(s.z) | ((uint32_t)float_to_half_bits_rne(s.w) << 16));
        return;
    }
    for (int e = 0; e < 4 && i0 + e < P.count; ++e) {
        float s = P.part[i0 + e];
        for (int z = 1; z < P.slices; ++z) s += P.part[(int64_t)z * P.count + i0 + e];
        P.Y[i0 + e] = float_to_half_bits_rne(s);
    }
}

// Slices, rounds per slice and blocks per slice of one product.  Slices: as
// few as LDS allows, more when the tiles alone cannot give every compute
// unit's waves work (each slice keeps at least one ring turn), unless
// `fewest` (no scratch for partials) holds them to the LDS minimum.
template <int BITS, int BTX>
bool xr_plan(int64_t K, int64_t N, int num_cus, bool fewest, int64_t& slices, int64_t& rs,
             int64_t& per_slice) {
    typedef XrGeom<BITS, BTX> XG;
    const int64_t rounds = K / XG::KR;
    const int64_t ntiles = (N + 15) / 16;
    slices = (rounds + XG::RMAX - 1) / XG::RMAX;
    const int64_t want_items = (int64_t)num_cus * XG::WAVES / 2;
    if (!fewest && ntiles * slices < want_items) {
        const int64_t s = (want_items + ntiles - 1) / ntiles;
        const int64_t smax = (rounds + XR_SLOTS - 1) / XR_SLOTS;
        slices = s < smax ? s : smax;
        if (slices < 1) slices = 1;
    }
    rs = (rounds + slices - 1) / slices;
    rs = (rs + XR_SLOTS - 1) / XR_SLOTS * XR_SLOTS;
    if (rs > XG::RMAX) return false;
    slices = (rounds + rs - 1) / rs;
    per_slice = ((int64_t)num_cus + slices - 1) / slices;
    if (per_slice > ntiles) per_slice = ntiles;
    if (per_slice < 1) per_slice = 1;
    return true;
}

// Plan of a product launched together with others.  Their blocks run side by
// side, so the other products supply the parallelism that extra K-slices give
// a single product: every product keeps the fewest slices LDS allows, and its
// blocks per slice are sized so that each wave of the whole launch gets about
// `per_wave` tiles (this amortizes a block's X staging over more rounds).
template <int BITS, int BTX>
bool xr_plan_grouped(int64_t K, int64_t N, int64_t per_wave, int64_t& slices, int64_t& rs,
                     int64_t& per_slice) {
    typedef XrGeom<BITS, BTX> XG;
    const int64_t rounds = K / XG::KR;
    const int64_t ntiles = (N + 15) / 16;
    slices = (rounds + XG::RMAX - 1) / XG::RMAX;
    rs = (rounds + slices - 1) / slices;
    rs = (rs + XR_SLOTS - 1) / XR_SLOTS * XR_SLOTS;
    if (rs > XG::RMAX) return false;
    slices = (rounds + rs - 1) / rs;
    per_slice = (ntiles + XG::WAVES * per_wave - 1) / (XG::WAVES * per_wave);
    if (per_slice < 1) per_slice = 1;
    return true;
}

// How a product's kernel reads its group headers.
template <int BITS, int BTX>
int xr_mode(const XrProduct& p) {
    typedef XrGeom<BITS, BTX> XG;
    const int64_t ngrp = p.K / p.group;
    const bool aligned16 = (reinterpret_cast<uintptr_t>(p.scales) % 16 == 0) &&
                           (reinterpret_cast<uintptr_t>(p.zeros) % 16 == 0);
    if (ngrp == 1) return XR_HDR_ROW;
    if (p.group == XG::KR && ngrp % 8 == 0 && aligned16) return XR_HDR_TURN;
    return XR_HDR_ROUND;
}

// One launch for up to XR_MAX_ITEMS products of one header mode, plus one
// reduction launch for those of them that have several K-slices.  The fp32
// partials of all of them share the caller's scratch (sized, not launched, in
// sizing mode).
template <int BITS, int BTX, int HM>
hipError_t launch_xr_items(const XrProduct* const* prods, int n, int64_t B, int num_cus,
                           const Scratch& ws, hipStream_t stream) {
    typedef XrGeom<BITS, BTX> XG;
    XrLaunch L{};
    XrReduce R{};
    size_t part_off[XR_MAX_ITEMS] = {};
    size_t part_total = 0;
    int64_t blocks = 0;
    // Several products: tiles per wave from the launch's total (see
    // xr_plan_grouped); one product keeps the single-product plan.
    int64_t per_wave = 1;
    if (n > 1) {
        int64_t items = 0;
        for (int i = 0; i < n; ++i) {
            int64_t slices = 0, rs = 0, per_slice = 0;
            if (!xr_plan_grouped<BITS, BTX>(prods[i]->K, prods[i]->N, 1, slices, rs, per_slice))
                return hipErrorInvalidValue;
            items += (prods[i]->N + 15) / 16 * slices;
        }
        const int64_t slots = (int64_t)num_cus * XG::WAVES;
        per_wave = (items + slots - 1) / slots;
        if (per_wave < 1) per_wave = 1;
    }
    for (int i = 0; i < n; ++i) {
        const XrProduct& p = *prods[i];
        int64_t slices = 0, rs = 0, per_slice = 0;
        const bool fewest = !ws.sizing() && !ws.ptr;
        const bool ok = n > 1 ? xr_plan_grouped<BITS, BTX>(p.K, p.N, per_wave, slices, rs, per_slice)
                              : xr_plan<BITS, BTX>(p.K, p.N, num_cus, fewest, slices, rs, per_slice);
        if (!ok) return hipErrorInvalidValue;
        XrItem& it = L.it[i];
        it.X = static_cast<const uint16_t*>(p.X);
        it.codes = static_cast<const uint4*>(p.codes);
        it.scales = static_cast<const uint16_t*>(p.scales);
        it.zeros = static_cast<const uint16_t*>(p.zeros);
        it.Y = static_cast<uint16_t*>(p.Y);
        it.part = nullptr;
        it.N = p.N;
        it.K = p.K;
        it.ngrp = p.K / p.group;
        const uint64_t rpg = (uint64_t)(p.group / XG::KR);
        it.rpg_magic = ((1ull << 32) + rpg - 1) / rpg;
        it.RS = (int32_t)rs;
        it.per_slice = (int32_t)per_slice;
        it.slices = (int32_t)slices;
        it.block0 = (int32_t)blocks;
        blocks += per_slice * slices;
        if (slices > 1) {
            part_off[i] = part_total;
            part_total += ((size_t)slices * B * p.N * sizeof(float) + 255) / 256 * 256;
        }
    }
    L.B = B;
    L.count = n;
    if (blocks <= 0 || blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (ws.sizing()) {
        ws.want(part_total);
        return hipSuccess;
    }
    if (part_total > 0 && !ws.ptr) return hipErrorInvalidValue;   // callers route these elsewhere
    float* base = static_cast<float*>(ws.ptr);
    int64_t t = 0;
    for (int i = 0; i < n; ++i) {
        XrItem& it = L.it[i];
        if (it.slices > 1) {
            it.part = reinterpret_cast<float*>(reinterpret_cast<char*>(base) + part_off[i]);
            XrReduceItem& r = R.it[R.count++];
            r.part = it.part;
            r.Y = it.Y;
            r.count = B * it.N;
            r.t0 = t;
            r.slices = it.slices;
            r.vec = r.count % 4 == 0 && reinterpret_cast<uintptr_t>(r.Y) % 8 == 0;
            t += (r.count + 1023) / 1024 * 1024;
        }
    }
    gemm_xr_kernel<BITS, BTX, HM><<<dim3((unsigned)blocks), dim3(XG::WAVES * 64), 0, stream>>>(L);
    hipError_t e = hipGetLastError();
    if (R.count > 0 && e == hipSuccess) {
        xr_reduce_kernel<<<dim3((unsigned)(t / 1024)), dim3(256), 0, stream>>>(R);
        e = hipGetLastError();
    }
    return e;
}

// Products of one batch size and bit width, grouped by header mode into
// launches of at most XR_MAX_ITEMS products (in the given order within a mode).
template <int BITS, int BTX>
hipError_t launch_xr_bt(const XrProduct* prods, int count, int64_t B, int num_cus,
                        const Scratch& ws, hipStream_t stream) {
    // Without scratch, products whose X needs several K-slices run alone on
    // the tiled kernel (one split); the others share launches as usual.
    const bool no_scratch = !ws.sizing() && !ws.ptr;
    if (no_scratch) {
        for (int i = 0; i < count; ++i) {
            const XrProduct& p = prods[i];
            if (xr_single_slice(B, p.K, BITS)) continue;
            const hipError_t e = launch_gemm_mfma(p.X, p.codes, p.scales, p.zeros, p.Y, B, p.K, p.N,
                                                  p.group, BITS, num_cus, ws, stream);
            if (e != hipSuccess) return e;
        }
    }
    for (int hm = 0; hm < 3; ++hm) {
        const XrProduct* sel[XR_MAX_ITEMS];
        int n = 0;
        for (int i = 0; i <= count; ++i) {
            const bool take = i < count && xr_mode<BITS, BTX>(prods[i]) == hm &&
                              (!no_scratch || xr_single_slice(B, prods[i].K, BITS));
            if (take) sel[n++] = &prods[i];
            if (n == XR_MAX_ITEMS || (i == count && n > 0)) {
                hipError_t e = hipSuccess;
                const XrProduct& p0 = *sel[0];
                if (n == 1 && !xr_supports(B, p0.K, p0.group, BITS))
                    // Alone in its launch: the single-call choice of kernel.
                    e = launch_gemm_mfma(p0.X, p0.codes, p0.scales, p0.zeros, p0.Y, B, p0.K, p0.N,
                                         p0.group, BITS, num_cus, ws, stream);
                else if (hm == XR_HDR_ROUND) e = launch_xr_items<BITS, BTX, XR_HDR_ROUND>(sel, n, B, num_cus, ws, stream);
                else if (hm == XR_HDR_TURN) e = launch_xr_items<BITS, BTX, XR_HDR_TURN>(sel, n, B, num_cus, ws, stream);
                else e = launch_xr_items<BITS, BTX, XR_HDR_ROW>(sel, n, B, num_cus, ws, stream);
                if (e != hipSuccess) return e;
                n = 0;
            }
        }
    }
    return hipSuccess;
}

}  // namespace

bool xr_groupable(int64_t B, int64_t K, int32_t group, int32_t bits) {
    if (B < 1 || B > 32 || (bits != 4 && bits != 8)) return false;
    const int kr = bits == 4 ? XrGeom<4, 16>::KR : XrGeom<8, 16>::KR;
    return group % kr == 0 && K % kr == 0 && K / kr < 65536;
}

bool xr_supports(int64_t B, int64_t K, int32_t group, int32_t bits) {
    if (B < 1 || B > 32 || (bits != 4 && bits != 8)) return false;
    const int kr = bits == 4 ? XrGeom<4, 16>::KR : XrGeom<8, 16>::KR;
    if (group % kr != 0 || K % kr != 0 || K / kr >= 65536) return false;
    // Past 16 columns a slice holds 2048 k; beyond four slices the partial
    // sums cost more than the tiled kernel's staging (measured at K = 11008).
    return B <= 16 || K <= 4 * XrGeom<4, 32>::KSL;
}

bool xr_single_slice(int64_t B, int64_t K, int32_t bits) {
    // The slice length of the batch tile wq_gemm_xr_many picks for B.
    const int64_t ksl = B <= 8 ? XrGeom<4, 8>::KSL : B <= 16 ? XrGeom<4, 16>::KSL : XrGeom<4, 32>::KSL;
    (void)bits;   // the slice holds k values, whatever their code width
    return K <= ksl;
}

hipError_t launch_gemm_xr_many(const XrProduct* prods, int count, int64_t B, int32_t bits,
                               int num_cus, const Scratch& ws, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    if (bits == 4) {
        if (B <= 8) return launch_xr_bt<4, 8>(prods, count, B, num_cus, ws, stream);
        if (B <= 16) return launch_xr_bt<4, 16>(prods, count, B, num_cus, ws, stream);
        return launch_xr_bt<4, 32>(prods, count, B, num_cus, ws, stream);
    }
    if (B <= 8) return launch_xr_bt<8, 8>(prods, count, B, num_cus, ws, stream);
    if (B <= 16) return launch_xr_bt<8, 16>(prods, count, B, num_cus, ws, stream);
    return launch_xr_bt<8, 32>(prods, count, B, num_cus, ws, stream);
}

}  // namespace wq
