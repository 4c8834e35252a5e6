// Matrix-core product for batches of up to 64 rows on tall matrices, with the
// waves of a block splitting K between them.
//
// Every weight is read once per call and serves the whole batch ("Serving many
// users at once", "Batching: one read, many users"); below the ridge the code
// stream sets the time ("Quantization & inference optimisation", "Bandwidth,
// not compute"), so the design keeps that stream whole and moves as little
// else as it can:
//   - a block (4 waves, one per SIMD) owns TPB (2 to 8) 16-row tiles of W
//     across all of K; wave w takes the w-th quarter of K, so each X value
//     reaches the compute unit once, and the waves' fp32 sums are added in
//     LDS, in wave order, at the end: no partial sums leave the compute unit;
//   - K is walked in rounds of 128 k (one group): lane (r16, g4) of tile t
//     holds the 16-byte code chunk of row 16 t + r16 at k [32 g4, 32 g4 + 32)
//     of the round, the weight operand of v_mfma_f32_16x16x32_f16 for the
//     round's 4 k-steps: at B <= 16 the exact integers 1024 + q (even k) and
//     64 + q (odd k), with the round's group header applied to the products
//     in fp32 (s * (sum u x - C1 - z C2), C1 and C2 from two more products
//     per k-step), past 16 dequantized in registers to fp16 (q - z) * s / 2,
//     once for all the batch blocks;
//   - code chunks come two rounds at a time (the two halves of each 128-byte
//     line of a row together) into a two-deep register ring;
//   - the group headers of the block's tiles (all of K) are copied into LDS
//     once, at the start, by LDS-DMA loads of whole 16-byte chunks, while the
//     first code loads are already in flight; header chunk p of row r sits at
//     position p ^ (r & (chunks per row - 1));
//   - a wave copies its rounds of X [16 NCB rows x 128 k] into an LDS ring of
//     DX rounds (four at B <= 32, two past) with LDS-DMA loads that read whole
//     lines (4 rows x 256 bytes per instruction); chunk p of row r goes to
//     position p ^ (r & 15), so the X-operand reads (16 rows, one chunk each,
//     per 16 lanes) hit distinct banks;
//   - a wave's loads complete in issue order, so X and codes are issued with
//     a fixed lead: X of round r + DX after round r, the codes of step d + 2
//     (rounds 2d + 4, 2d + 5) after round 2d + 1, behind that round's X; the
//     wait before each round counts exactly the loads issued after the ones
//     it needs;
//   - blocks start their walks through their quarters at different steps, so
//     that the chip's loads are spread over the columns of the matrix.
// Needs group 128, K = 2048, 4096 or 8192, X 16-byte aligned; it uses no
// scratch.
#include "wq_device.h"
#include "wq_launch.h"
#include "wq_mfma_dq.h"
#include "wq_nf4_levels.h"

namespace wq {

namespace {

constexpr int kKwBufWord3 = 0x00020000;     // raw, unswizzled gfx9 buffer
constexpr uint32_t kKwFar = 0x80000000u;    // a per-lane offset past every buffer the kernel reads
constexpr int kKwLgkm0 = 0xC07F;             // s_waitcnt lgkmcnt(0), vmcnt and expcnt unconstrained

typedef __attribute__((address_space(3))) void kw_lds_void;
typedef unsigned int kw_v4u __attribute__((ext_vector_type(4)));
typedef unsigned int kw_v3u __attribute__((ext_vector_type(3)));
typedef unsigned int kw_v2u __attribute__((ext_vector_type(2)));

// How the weight operand is formed: dequantized in registers to fp16
// (q - z) * s / 2 (4-bit codes), or exact integers with the header applied
// per round in fp32, with an integer zero point or a float offset, or (NF4,
// 4-bit codes, blocks of 64) looked up as fp16 level pairs and scaled in fp16.
constexpr int KW_DEQUANT = 0, KW_ZERO = 1, KW_OFFSET = 2, KW_NF4 = 3;
constexpr int kKwLutCopies = 32;   // NF4 table copies (one per LDS bank of a 32-lane cycle)

struct KwArgs {
    const uint16_t* X;
    const uint8_t* codes;
    const uint16_t* scales;
    const uint16_t* zeros;
    uint16_t* Y;
    int32_t B, N, K;
    int32_t ngrp;      // groups per row (K / 128)
    int32_t cpr;       // 16-byte header chunks per row (ngrp / 8, a power of two)
    int32_t nd;        // two-round steps per wave (K / (256 W))
};

// s_waitcnt with vmcnt(n) (bits 3:0 and 15:14) and no wait on the other counters.
constexpr int kw_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// The loads that may still be in flight when round r starts (steady state),
// for the issue order of the kernel: at the end of round e, X of round e + DX,
// then, if e is odd, the codes of step (e - 1) / 2 + 2 (NXL and NSL
// loads).  Round r needs X of round r (issued at the end of round r - DX) and
// its step r / 2 (issued at the end of round 2 (r / 2) - 3, after that round's
// X); everything issued after the later of the two may be outstanding.
constexpr int kw_inflight(int DX, int NXL, int NSL, int r) {
    const int ex = r - DX, es = 2 * (r / 2) - 3;
    const bool step_later = es >= ex;
    const int e = step_later ? es : ex;
    int n = (!step_later && (e & 1)) ? NSL : 0;
    for (int q = e + 1; q < r; ++q) n += NXL + ((q & 1) ? NSL : 0);
    return n < 63 ? n : 63;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t kw_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kKwBufWord3);
}

// NCB: 16-row batch blocks (B <= 16 NCB).  TPB: 16-row weight tiles per block.
// DX: rounds in the X ring (2 or 4): X is issued DX - 1 rounds before use,
// the codes of a step two rounds before its first round.  W: waves per block
// (one per SIMD), each taking a W-th of K.
template <int NCB, int TPB, int DX, int W, int BITS, int MODE, int NXL = NCB * 4>
__global__ __launch_bounds__(64 * W, 1) void gemm_kw_kernel(const KwArgs a) {
    static_assert(DX == 2 || DX == 4, "an X ring of 2 or 4 rounds");
    static_assert(BITS == 2 || BITS == 3 || BITS == 4, "2-, 3- or 4-bit codes");
    static_assert((MODE != KW_DEQUANT && MODE != KW_NF4) || BITS == 4, "fp16 operands take 4-bit codes");
    constexpr bool EXACT = MODE == KW_ZERO || MODE == KW_OFFSET;
    constexpr bool NF4 = MODE == KW_NF4;
    constexpr int XR = NCB * 16 * 16;   // 16-byte X chunks per round
    // The rounds of the ring are separate objects, so that the compiler can
    // tell the LDS-DMA writes of one from those of another and waits only for
    // the round that is read.
    __shared__ __align__(16) uint4 xs0[W * XR];
    __shared__ __align__(16) uint4 xs1[W * XR];
    __shared__ __align__(16) uint4 xs2[DX > 2 ? W * XR : 1];
    __shared__ __align__(16) uint4 xs3[DX > 2 ? W * XR : 1];
    // The block's group headers (scales, zero points), up to 64 groups per
    // row: row r's 16-byte chunk p (8 groups) at position r * cpr +
    // (p ^ (r & (cpr - 1))), so that 16 rows read at one group hit distinct
    // banks.
    // NF4 has no zero points and blocks of 64: up to 128 scales (16 chunks)
    // per row in hs, in the space the zero points take otherwise.
    constexpr int HCH = TPB * 16 * (NF4 ? 16 : 8);
    __shared__ __align__(16) uint4 hs[HCH];
    __shared__ __align__(16) uint4 hz[NF4 ? 1 : HCH];
    // NF4: code byte b -> fp16 pair (level[b & 15], level[b >> 4]), entry b of
    // copy c at word b * 32 + c; lane l reads copy l % 32.
    __shared__ uint32_t lut[NF4 ? 256 * kKwLutCopies : 1];
    // NXL: LDS-DMA loads per round (4 batch rows each).  At B <= 8 only the
    // first two are issued: rows 8 .. 15 of the slot keep whatever it held,
    // which only reaches output rows past B (each output row of a product
    // depends on its own A row), and those are not stored.
    static_assert(NXL >= 1 && NXL <= NCB * 4, "X loads per round");
    constexpr int NSL = 2 * TPB;        // code loads per two-round step
    constexpr int WAIT_EVEN = kw_vmcnt(kw_inflight(DX, NXL, NSL, 100));
    constexpr int WAIT_ODD = kw_vmcnt(kw_inflight(DX, NXL, NSL, 101));

    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if constexpr (NF4) {
        for (int e = (int)threadIdx.x; e < 256 * kKwLutCopies; e += 64 * W) {
            const int b = e / kKwLutCopies;
            lut[e] = (uint32_t)kNf4LevelBits[b & 15] | ((uint32_t)kNf4LevelBits[b >> 4] << 16);
        }
        __syncthreads();
    }
    const uint32_t* const lutl = lut + (NF4 ? (lane & (kKwLutCopies - 1)) : 0);
    uint4* const xw[4] = {xs0 + w * XR, xs1 + w * XR, xs2 + (DX > 2 ? w * XR : 0),
                          xs3 + (DX > 2 ? w * XR : 0)};   // this wave's rounds (slot = round % DX)

    const int tile0 = blockIdx.x * TPB;
    const int rows_blk = a.N - tile0 * 16 < TPB * 16 ? a.N - tile0 * 16 : TPB * 16;
    const uint32_t row_bytes = (uint32_t)a.K * BITS / 8;
    constexpr uint32_t RB = 16 * BITS;   // bytes of a row per 128-k round
    const uint8_t* const cbase = a.codes + (size_t)tile0 * 16 * row_bytes;
    const uint32_t cbytes = (uint32_t)rows_blk * row_bytes;
    const size_t hbase = (size_t)tile0 * 16 * a.ngrp;
    const uint32_t hbytes = (uint32_t)rows_blk * a.ngrp * 2;
    const uint32_t xbytes = (uint32_t)a.B * a.K * 2;

    // This lane's row in each tile (rows past N reread the block's last row;
    // their sums are not stored).
    uint32_t coff[TPB];
    int hrow[TPB], hswz[TPB];
#pragma unroll
    for (int t = 0; t < TPB; ++t) {
        int rl = t * 16 + r16;
        rl = rl < rows_blk ? rl : rows_blk - 1;
        coff[t] = (uint32_t)rl * row_bytes + (RB / 4) * g4;
        hrow[t] = rl * a.cpr;
        hswz[t] = rl & (a.cpr - 1);
    }
    const int d0 = w * a.nd;   // the wave's first two-round step
    const int nr = 2 * a.nd;   // the wave's rounds
    // Blocks start their walks at different steps (and wrap), so that the
    // chip's loads do not all fall on the same columns at once; blocks are
    // dealt to the 8 XCDs in turn, so neighbours on one XCD differ too.
    const int soff = (int)((blockIdx.x + (blockIdx.x >> 3)) & (uint32_t)(a.nd - 1));

    // X of local round rl: instruction q covers rows 4q .. 4q + 3; lane l takes
    // chunk (l & 15) ^ (row & 15) of row 4q + l / 16 and writes position l.
    uint32_t xoff[NXL];
#pragma unroll
    for (int q = 0; q < NXL; ++q) {
        const int row = 4 * q + (lane >> 4);
        const int chunk = (lane & 15) ^ (row & 15);
        xoff[q] = (uint32_t)row * a.K * 2 + (uint32_t)chunk * 16;
    }
    // Each round's loads go through a buffer whose base is the round's first
    // byte (the per-lane offsets stay fixed, and the address arithmetic is
    // scalar).  Batch rows past B lie past its end and read as zeros.  Rounds
    // past the wave's range are issued too, with an empty buffer: they read
    // nothing and write zeros into a free slot, and every round of the loop
    // issues the same loads (one wait count holds).
    auto load_x = [&](int rl, int slot) {   // slot = rl % DX, a compile-time constant at every call
        const uint32_t rg = (uint32_t)(2 * d0 + ((rl + 2 * soff) & (nr - 1)));
        const __amdgpu_buffer_rsrc_t xrs =
            kw_rsrc(reinterpret_cast<const uint8_t*>(a.X) + 256u * rg, rl < nr ? xbytes - 256u * rg : 0u);
#pragma unroll
        for (int q = 0; q < NXL; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (kw_lds_void*)(xw[slot] + q * 64), 16, (int)xoff[q], 0, 0,
                                                     0);
    };

    struct Step {
        uint32_t c[TPB][2][BITS];   // this lane's code words of the step's two rounds
    };
    // The same for the code words of a step (2 RB bytes of every row from
    // byte 2 RB dg on; the last row's last words end within the buffer): one
    // load of BITS words per lane, tile and round (32 codes: k in
    // [32 g4, 32 g4 + 32) of the round).
    auto load_words = [&](const __amdgpu_buffer_rsrc_t& crs, uint32_t off, uint32_t* dst) {
        if constexpr (BITS == 4) {
            const kw_v4u v = __builtin_amdgcn_raw_buffer_load_b128(crs, (int)off, 0, 0);
            dst[0] = v.x, dst[1] = v.y, dst[2] = v.z, dst[3] = v.w;
        } else if constexpr (BITS == 3) {
            const kw_v3u v = __builtin_amdgcn_raw_buffer_load_b96(crs, (int)off, 0, 0);
            dst[0] = v.x, dst[1] = v.y, dst[2] = v.z;
        } else {
            const kw_v2u v = __builtin_amdgcn_raw_buffer_load_b64(crs, (int)off, 0, 0);
            dst[0] = v.x, dst[1] = v.y;
        }
    };
    // (At 2 bits, one 16-byte load per lane covering both rounds of a step,
    // regrouped across lanes with half swaps, measured slower than two 8-byte
    // loads: 27.8/29.8 against 26.2/27.8 us at B = 16 on 28672 x 8192.)
    auto load_step = [&](int dl, Step& st) {
        const uint32_t dg = (uint32_t)(d0 + ((dl + soff) & (a.nd - 1)));
        const __amdgpu_buffer_rsrc_t crs = kw_rsrc(cbase + 2 * RB * dg, dl < a.nd ? cbytes - 2 * RB * dg : 0u);
#pragma unroll
        for (int t = 0; t < TPB; ++t) {
            load_words(crs, coff[t], st.c[t][0]);
            load_words(crs, coff[t] + RB, st.c[t][1]);
        }
    };

    const dq::DqConsts cst{vgpr_const(0x000F000Fu), vgpr_const(0x00F000F0u), vgpr_const(0x60006000u),
                           vgpr_const(0x50005000u)};
    // Exact-integer operands.  A code masked in place at bit position p of a
    // half, under an exponent whose ulp is 2^-p, is the fp16 value E + q
    // exactly; the B operand whose products give C1 holds each slot's E, and
    // the one for C2 holds ones (same k order).
    //   4 bits: word j = k-step j, pairs (k0,k4) (k1,k5) (k2,k6) (k3,k7) at
    //     bit 0, 4, 0, 4 (w, w, w >> 8, w >> 8): E = 1024, 64, 1024, 64.
    //   3 bits: 24-bit unit j = k-step j; t = low half of u | high half of
    //     u << 4 holds the pair (k_r, k_r+4) at bit 3r, r = 0..3; r = 3 (bits
    //     9-11) does not fit the 10-bit mantissa and is taken from t >> 9 at
    //     bit 0: E = 1024, 128, 16, 1024.
    //   2 bits: word d = k-steps 2d, 2d + 1; (w, w >> 8) masked at bit 2m hold
    //     (k_m, k_m+8) and (k_m+4, k_m+12); k-step 2d + hs takes m = 2 hs and
    //     2 hs + 1: E = 1024, 1024, 256, 256 (hs 0) and 64, 64, 16, 16 (hs 1).
    constexpr uint32_t E1024 = 0x64006400u, E256 = 0x5C005C00u, E128 = 0x58005800u, E64 = 0x54005400u,
                       E16 = 0x4C004C00u;
    const uint32_t ex_a = vgpr_const(BITS == 2 ? E256 : BITS == 3 ? E128 : E64);
    const uint32_t ex_b = vgpr_const(BITS == 2 ? E64 : E16);
    const uint32_t ex_c = vgpr_const(E16);
    const uint32_t ex_0 = vgpr_const(E1024);
    const uint32_t mk_0 = vgpr_const(BITS == 2 ? 0x00030003u : BITS == 3 ? 0x00070007u : 0x000F000Fu);
    const uint32_t mk_1 = vgpr_const(BITS == 2 ? 0x000C000Cu : BITS == 3 ? 0x00380038u : 0x00F000F0u);
    const uint32_t mk_2 = vgpr_const(BITS == 2 ? 0x00300030u : 0x01C001C0u);
    const uint32_t mk_3 = vgpr_const(0x00C000C0u);
    const h8_t kone = __builtin_bit_cast(h8_t, uint4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u});
    const h2_t zmul = {(_Float16)0.5f, (_Float16)0.5f};
    const h2_t zadd = {(_Float16)512.0f, (_Float16)32.0f};

    f4_t acc[TPB][NCB];
#pragma unroll
    for (int t = 0; t < TPB; ++t)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[t][cb] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // One round: half h of a step's codes and headers, X from LDS slot xr.
    auto compute = [&](const Step& st, const uint32_t* hsv, const uint32_t* hzv, int h, const uint4* xr) {
        if constexpr (NF4) {
            // Lane g4's 32 codes of the round lie in block 2 (round) + g4 / 2 of
            // 64; hsv[t] holds the two blocks of round h (low: g4 < 2).  Each
            // code byte is the pair (k even, k odd), so X is read in its
            // natural order; the operand is level * s, rounded once to fp16.
            const uint32_t selg = g4 >= 2 ? 0x07060706u : 0x05040504u;
            h2_t ss[TPB];
#pragma unroll
            for (int t = 0; t < TPB; ++t) ss[t] = as_h2(__builtin_amdgcn_perm(hsv[t], hsv[t], selg));
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                h8_t xo[NCB];
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    xo[cb] = __builtin_bit_cast(h8_t, xr[(cb * 16 + r16) * 16 + ((4 * g4 + j) ^ r16)]);
#pragma unroll
                for (int t = 0; t < TPB; ++t) {
                    const uint32_t wv = st.c[t][h][j];
                    uint32_t pr[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) pr[i] = lutl[((wv >> (8 * i)) & 0xFFu) * kKwLutCopies];
                    const uint4 u = {as_u32(as_h2(pr[0]) * ss[t]), as_u32(as_h2(pr[1]) * ss[t]),
                                     as_u32(as_h2(pr[2]) * ss[t]), as_u32(as_h2(pr[3]) * ss[t])};
                    const h8_t bop = __builtin_bit_cast(h8_t, u);
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
                        acc[t][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xo[cb], bop, acc[t][cb], 0, 0, 0);
                }
            }
            return;
        }
        if constexpr (EXACT) {
            // The codes enter as exact integers E + q (E per operand slot); two
            // more products per k-step give C1 = sum E_k x_k and C2 = sum x_k
            // in every column, and the group header is applied once per round
            // in fp32:  s * (sum u x - C1) - s z C2  (integer zero point), or
            // s * (sum u x - C1) + m C2  (float offset m).  At 2 and 3 bits E
            // is subtracted from each operand in fp16 (exact), so the operand
            // is q itself and C1 = 0: with so few levels most codes sit near
            // the zero point, sum q x is small next to sum E x, and carrying E
            // through the fp32 sums loses too much of it.
            float sf[TPB], zf[TPB];
#pragma unroll
            for (int t = 0; t < TPB; ++t) {
                const h2_t s2 = as_h2(hsv[t]), z2 = as_h2(hzv[t]);
                sf[t] = (float)(h ? s2.y : s2.x);
                zf[t] = (float)(h ? z2.y : z2.x);
            }
            f4_t c1[NCB], c2[NCB], ra[TPB][NCB];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                c1[cb] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
                c2[cb] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int t = 0; t < TPB; ++t) ra[t][cb] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
            }
            uint4 xc[NCB][2];   // 2 bits: the two X chunks of a code word
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                h8_t xo[NCB];
                uint4 ko;
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    const uint4* xrow = xr + (cb * 16 + r16) * 16;
                    if constexpr (BITS == 2) {
                        const int hs = j & 1;
                        if (hs == 0) {
                            xc[cb][0] = xrow[(4 * g4 + j) ^ r16];
                            xc[cb][1] = xrow[(4 * g4 + j + 1) ^ r16];
                        }
                        const uint32_t a0 = hs ? xc[cb][0].y : xc[cb][0].x, a1 = hs ? xc[cb][1].y : xc[cb][1].x;
                        const uint32_t b0 = hs ? xc[cb][0].w : xc[cb][0].z, b1 = hs ? xc[cb][1].w : xc[cb][1].z;
                        const uint4 v = {__builtin_amdgcn_perm(a1, a0, 0x05040100u), __builtin_amdgcn_perm(b1, b0, 0x05040100u),
                                         __builtin_amdgcn_perm(a1, a0, 0x07060302u), __builtin_amdgcn_perm(b1, b0, 0x07060302u)};
                        xo[cb] = __builtin_bit_cast(h8_t, v);
                    } else {
                        xo[cb] = __builtin_bit_cast(h8_t, dq::permute8<4>(xrow[(4 * g4 + j) ^ r16]));
                    }
                }
                if constexpr (BITS == 4) ko = uint4{ex_0, ex_a, ex_0, ex_a};
                else if constexpr (BITS == 3) ko = uint4{ex_0, ex_a, ex_b, ex_0};
                else ko = (j & 1) ? uint4{ex_b, ex_b, ex_c, ex_c} : uint4{ex_0, ex_0, ex_a, ex_a};
                const h8_t koff = __builtin_bit_cast(h8_t, ko);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    if constexpr (BITS == 4)
                        c1[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xo[cb], koff, c1[cb], 0, 0, 0);
                    c2[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xo[cb], kone, c2[cb], 0, 0, 0);
                }
#pragma unroll
                for (int t = 0; t < TPB; ++t) {
                    const uint32_t* cw = st.c[t][h];
                    uint4 u;
                    if constexpr (BITS == 4) {
                        const uint32_t wv = cw[j], w8 = wv >> 8;
                        u = uint4{(wv & mk_0) | ex_0, (wv & mk_1) | ex_a, (w8 & mk_0) | ex_0, (w8 & mk_1) | ex_a};
                    } else if constexpr (BITS == 3) {
                        const uint32_t uu = j == 0   ? cw[0]
                                            : j == 1 ? __builtin_amdgcn_alignbit(cw[1], cw[0], 24)
                                            : j == 2 ? __builtin_amdgcn_alignbit(cw[2], cw[1], 16)
                                                     : cw[2] >> 8;
                        const uint32_t tt = ((uu << 4) & 0xFFFF0000u) | (uu & 0x0000FFFFu);
                        u = uint4{(tt & mk_0) | ex_0, (tt & mk_1) | ex_a, (tt & mk_2) | ex_b, ((tt >> 9) & mk_0) | ex_0};
                    } else {
                        const uint32_t wv = cw[j >> 1], w8 = wv >> 8;
                        if (j & 1)
                            u = uint4{(wv & mk_2) | ex_b, (w8 & mk_2) | ex_b, (wv & mk_3) | ex_c, (w8 & mk_3) | ex_c};
                        else
                            u = uint4{(wv & mk_0) | ex_0, (w8 & mk_0) | ex_0, (wv & mk_1) | ex_a, (w8 & mk_1) | ex_a};
                    }
                    if constexpr (BITS != 4) {   // q, exactly
                        u = uint4{as_u32(as_h2(u.x) - as_h2(ko.x)), as_u32(as_h2(u.y) - as_h2(ko.y)),
                                  as_u32(as_h2(u.z) - as_h2(ko.z)), as_u32(as_h2(u.w) - as_h2(ko.w))};
                    }
                    const h8_t bop = __builtin_bit_cast(h8_t, u);
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
                        ra[t][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xo[cb], bop, ra[t][cb], 0, 0, 0);
                }
            }
#pragma unroll
            for (int t = 0; t < TPB; ++t)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float v = ra[t][cb][i] - c1[cb][i];
                        if constexpr (MODE == KW_OFFSET)
                            acc[t][cb][i] = __builtin_fmaf(zf[t], c2[cb][i], __builtin_fmaf(sf[t], v, acc[t][cb][i]));
                        else
                            acc[t][cb][i] = __builtin_fmaf(sf[t], __builtin_fmaf(-zf[t], c2[cb][i], v), acc[t][cb][i]);
                    }
            return;
        }
        h2_t nz[TPB], ss[TPB];
        const uint32_t sel = h ? 0x07060706u : 0x05040504u;   // that group's half, twice
#pragma unroll
        for (int t = 0; t < TPB; ++t) {
            nz[t] = as_h2(__builtin_amdgcn_perm(hzv[t], hzv[t], sel)) * zmul + zadd;   // (512 + z/2, 32 + z/2)
            ss[t] = as_h2(__builtin_amdgcn_perm(hsv[t], hsv[t], sel));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            h8_t xo[NCB];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                xo[cb] = __builtin_bit_cast(h8_t, dq::permute8<4>(xr[(cb * 16 + r16) * 16 + ((4 * g4 + j) ^ r16)]));
#pragma unroll
            for (int t = 0; t < TPB; ++t) {
                const uint32_t* cwp = st.c[t][h];
                const uint4 cw = {cwp[0], cwp[1], cwp[2], cwp[3]};
                const h8_t bop = dq::dequant<4>(cw, j, cst, nz[t], ss[t]);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    acc[t][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xo[cb], bop, acc[t][cb], 0, 0, 0);
            }
        }
    };

    // Two rounds of one step from ring slot st, each followed by the loads of
    // its issue slot (X DX rounds later; after the odd round, the codes two
    // steps later).  dl is even for ring0 and odd for ring1, and the loop
    // below starts every pair of steps at a round that is a multiple of 4, so
    // the X slots are compile-time constants.
    auto step = [&](Step& st, int dl, int pos) {   // pos: dl % 2
        const int r = 2 * dl;
        __builtin_amdgcn_s_waitcnt(WAIT_EVEN);
        asm volatile("" ::: "memory");
        // The step's two groups (2 dg, 2 dg + 1) share one 8-group chunk.
        const int dg = d0 + ((dl + soff) & (a.nd - 1));
        uint32_t hsv[TPB], hzv[TPB], hs1[TPB];
#pragma unroll
        for (int t = 0; t < TPB; ++t) {
            if constexpr (NF4) {
                // Four blocks of 64 per step: dwords 2 (dg & 1) and + 1 of chunk dg / 2.
                const int at = (hrow[t] + ((dg >> 1) ^ hswz[t])) * 4 + 2 * (dg & 1);
                hsv[t] = reinterpret_cast<const uint32_t*>(hs)[at];
                hs1[t] = reinterpret_cast<const uint32_t*>(hs)[at + 1];
                hzv[t] = 0;
            } else {
                const int at = (hrow[t] + ((dg >> 2) ^ hswz[t])) * 4 + (dg & 3);
                hsv[t] = reinterpret_cast<const uint32_t*>(hs)[at];
                hzv[t] = reinterpret_cast<const uint32_t*>(hz)[at];
                hs1[t] = hsv[t];
            }
        }
        compute(st, hsv, hzv, 0, xw[(2 * pos) % DX]);
        // The next load into this slot writes LDS behind the wave's back: every
        // LDS read of the round must have returned first (the compiler leaves
        // the last X reads in flight past the issue of the load otherwise, and
        // a load that lands early, e.g. rows past B, which read as zeros at
        // once, overwrites X the round has not read yet).
        __builtin_amdgcn_s_waitcnt(kKwLgkm0);
        asm volatile("" ::: "memory");
        load_x(r + DX, (2 * pos) % DX);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(WAIT_ODD);
        asm volatile("" ::: "memory");
        compute(st, NF4 ? hs1 : hsv, hzv, 1, xw[(2 * pos + 1) % DX]);
        __builtin_amdgcn_s_waitcnt(kKwLgkm0);
        asm volatile("" ::: "memory");
        load_x(r + 1 + DX, (2 * pos + 1) % DX);
        // The wait counts need X of a round issued wholly before the next
        // step's codes: keep the two groups of loads in program order.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        load_step(dl + 2, st);
        __builtin_amdgcn_sched_barrier(0);
    };

    // The headers first (the oldest loads: complete at the first wait), shared
    // between the waves: instruction i fills positions 64 i .. 64 i + 63.
    {
        const __amdgpu_buffer_rsrc_t srs = kw_rsrc(a.scales + hbase, hbytes);
        const __amdgpu_buffer_rsrc_t zrs = kw_rsrc(a.zeros + hbase, hbytes);
        const int total = rows_blk * a.cpr;
        for (int i = w; i * 64 < total; i += W) {
            const int flat = i * 64 + lane;
            const int row = flat / a.cpr, p = flat & (a.cpr - 1);
            const uint32_t src = flat < total ? (uint32_t)(row * a.cpr + (p ^ (row & (a.cpr - 1)))) * 16u : kKwFar;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (kw_lds_void*)(hs + i * 64), 16, (int)src, 0, 0, 0);
            if constexpr (!NF4)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(zrs, (kw_lds_void*)(hz + i * 64), 16, (int)src, 0, 0, 0);
        }
    }
    Step ring0, ring1;
    // The prologue issues what the steady state would have issued at the
    // ends of rounds -4 .. -1.
    if constexpr (DX == 4) {
        load_x(0, 0);
        load_x(1, 1);
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    load_step(0, ring0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    load_x(DX - 2, DX - 2);
    load_x(DX - 1, DX - 1);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    load_step(1, ring1);
    __builtin_amdgcn_sched_barrier(0);
    // Every wave's header loads are done once its first wait has passed.
    __builtin_amdgcn_s_waitcnt(WAIT_EVEN);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    for (int dl = 0; dl < a.nd; dl += 2) {
        step(ring0, dl, 0);
        step(ring1, dl + 1, 1);
    }

    // The waves' sums, added in wave order (the ring is free once every wave
    // is past its last round).  Accumulator lane layout: batch row
    // 16 cb + 4 g4 + i, weight row r16 of tile t; the operand carried a 1/2.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // Wave w's sums go to ring object w & 1 at float offset (w >> 1) * PER * 64
    // (W / 2 waves of TPB * NCB KB in each object of W * NCB * 4 KB: TPB <= 8).
    constexpr int PER = TPB * NCB * 4;   // floats per lane per wave
    static_assert((W / 2) * PER * 64 * 4 <= W * XR * 16, "partial sums must fit the ring");
    auto red_of = [&](int ww) {
        return reinterpret_cast<float*>((ww & 1) ? xs1 : xs0) + (ww >> 1) * PER * 64;
    };
    {
        float* red = red_of(w);
#pragma unroll
        for (int t = 0; t < TPB; ++t)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i) red[((t * NCB + cb) * 4 + i) * 64 + lane] = acc[t][cb][i];
    }
    __syncthreads();
#pragma unroll
    for (int e = (int)threadIdx.x; e < PER * 64; e += 64 * W) {   // e = ((t * NCB + cb) * 4 + i) * 64 + lane
        float v = red_of(0)[e];
#pragma unroll
        for (int ww = 1; ww < W; ++ww) v += red_of(ww)[e];
        const int q = e >> 6, l = e & 63;
        const int t = q / (NCB * 4), cb = (q / 4) % NCB, i = q % 4;
        const int row = tile0 * 16 + t * 16 + (l & 15);
        const int b = cb * 16 + 4 * (l >> 4) + i;
        if (row < a.N && b < a.B) a.Y[(size_t)b * a.N + row] = float_to_half_bits_rne(MODE == KW_DEQUANT ? 2.0f * v : v);
    }
}

template <int NCB, int TPB, int BITS, int MODE, int NXL = NCB * 4>
hipError_t launch_tpb(KwArgs a, hipStream_t stream) {
    const int ntiles = (a.N + 15) / 16;
    const dim3 grid((unsigned)((ntiles + TPB - 1) / TPB));
    // Four waves (eight would double the row streams each compute unit keeps
    // open, and the code stream slows down); four rounds of X in flight
    // where they fit in LDS (4 * NCB * 16 KB).
    // (NF4 keeps a 32 KB level table: two rounds of X past one batch block.)
    constexpr int DX = NCB == 1 || (NCB == 2 && MODE != KW_NF4) ? 4 : 2;
    a.nd = a.K / (256 * 4);
    gemm_kw_kernel<NCB, TPB, DX, 4, BITS, MODE, NXL><<<grid, dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

template <int NCB, int BITS, int MODE, int NXL = NCB * 4>
hipError_t launch_ncb(const KwArgs& a, int tpb, hipStream_t stream) {
    switch (tpb) {
        case 2: return launch_tpb<NCB, 2, BITS, MODE, NXL>(a, stream);
        case 3: return launch_tpb<NCB, 3, BITS, MODE, NXL>(a, stream);
        case 4: return launch_tpb<NCB, 4, BITS, MODE, NXL>(a, stream);
        case 5: return launch_tpb<NCB, 5, BITS, MODE, NXL>(a, stream);
        case 6: return launch_tpb<NCB, 6, BITS, MODE, NXL>(a, stream);
        case 7: return launch_tpb<NCB, 7, BITS, MODE, NXL>(a, stream);
        default: return launch_tpb<NCB, 8, BITS, MODE, NXL>(a, stream);
    }
}

// Up to 32 batch rows: one or two 16-row batch blocks on exact-integer
// operands (2-, 3-bit codes, float offsets).
template <int BITS, int MODE>
hipError_t launch_exact(const KwArgs& a, int tpb, hipStream_t stream) {
    if (a.B <= 16) return launch_ncb<1, BITS, MODE>(a, tpb, stream);
    return launch_ncb<2, BITS, MODE>(a, tpb, stream);
}

}  // namespace

// Tiles per block: the fewest that keep one block per compute unit, 2 to 8.
// Every block streams its quarter-K slices of X whole, so a block of two tiles
// reads as many X bytes as code bytes at B = 16; that still beats a grid with
// K split across blocks, whose partial sums go through HBM.
int kw_tiles_per_block(int64_t N, int num_cus) {
    const int64_t ntiles = (N + 15) / 16;
    int64_t tpb = (ntiles + num_cus - 1) / num_cus;
    return tpb < 2 ? 2 : tpb > 8 ? 8 : (int)tpb;
}

// At least 1.8 tiles per compute unit: blocks of two tiles then still occupy
// 90 % of the compute units; below that, half-empty grids leave the kernels
// that split K the faster choice.
static bool kw_enough_tiles(int64_t N, int num_cus) {
    return (N + 15) / 16 * 10 >= 18 * (int64_t)num_cus;
}

bool kw_supports(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits, bool offset) {
    // K = 2048, 4096 or 8192: 16, 32 or 64 groups per row (a power-of-two
    // number of 16-byte header chunks, all of them in LDS).
    const bool int4 = bits == 4 && !offset;
    return (bits == 2 || bits == 3 || bits == 4) && group == 128 && B >= 1 && B <= (int4 ? 64 : 32) &&
           (K == 2048 || K == 4096 || K == 8192) && N >= 16 && N <= (1 << 24);
}

static bool kw_aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// Taken on matrices of at least 1.8 tiles per compute unit, with X and the
// header arrays 16-byte aligned (the headers are staged by 16-byte loads; a
// null pointer, as in a size query, counts as aligned); for 4-bit
// codes with integer zero points past 4 batch rows (at 4 and below the
// quad-stream kernel reads the codes in a faster load shape and needs no
// padding rows), for the other formats from 2 batch rows (at 1 the bit-stream
// GEMV streams them as fast).
bool kw_takes(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits, bool offset, const void* X,
              const void* scales, const void* zeros, int num_cus) {
    const bool int4 = bits == 4 && !offset;
    return B > (int4 ? 4 : 1) && kw_supports(B, K, N, group, bits, offset) && kw_aligned16(X) &&
           kw_aligned16(scales) && kw_aligned16(zeros) && kw_enough_tiles(N, num_cus);
}

// NF4 (blocks of 64, 4-bit codes indexing the level table): 2 <= B <= 32.
bool kw_nf4_takes(int64_t B, int64_t K, int64_t N, int32_t group, const void* X, const void* scales,
                  int num_cus) {
    return B >= 2 && B <= 32 && group == 64 && (K == 2048 || K == 4096 || K == 8192) && N >= 16 &&
           N <= (1 << 24) && kw_aligned16(X) && kw_aligned16(scales) && kw_enough_tiles(N, num_cus);
}

hipError_t launch_gemm_kw_nf4(const void* X, const void* codes, const void* scales, void* Y, int64_t B, int64_t K,
                              int64_t N, int32_t group, int num_cus, hipStream_t stream) {
    if (!kw_nf4_takes(B, K, N, group, X, scales, num_cus)) return hipErrorInvalidValue;
    KwArgs a;
    a.X = static_cast<const uint16_t*>(X);
    a.codes = static_cast<const uint8_t*>(codes);
    a.scales = static_cast<const uint16_t*>(scales);
    a.zeros = static_cast<const uint16_t*>(scales);   // unused
    a.Y = static_cast<uint16_t*>(Y);
    a.B = (int32_t)B;
    a.N = (int32_t)N;
    a.K = (int32_t)K;
    a.ngrp = (int32_t)(K / 64);
    a.cpr = a.ngrp / 8;
    return launch_exact<4, KW_NF4>(a, kw_tiles_per_block(N, num_cus), stream);
}

hipError_t launch_gemm_kw(const void* X, const void* codes, const void* scales, const void* zeros, void* Y,
                          int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits, bool offset, int num_cus,
                          hipStream_t stream) {
    if (!kw_supports(B, K, N, group, bits, offset) || !kw_aligned16(X) || !kw_aligned16(scales) ||
        !kw_aligned16(zeros))
        return hipErrorInvalidValue;
    KwArgs a;
    a.X = static_cast<const uint16_t*>(X);
    a.codes = static_cast<const uint8_t*>(codes);
    a.scales = static_cast<const uint16_t*>(scales);
    a.zeros = static_cast<const uint16_t*>(zeros);
    a.Y = static_cast<uint16_t*>(Y);
    a.B = (int32_t)B;
    a.N = (int32_t)N;
    a.K = (int32_t)K;
    a.ngrp = (int32_t)(K / 128);
    a.cpr = a.ngrp / 8;
    const int tpb = kw_tiles_per_block(N, num_cus);
    if (offset) {
        if (bits == 2) return launch_exact<2, KW_OFFSET>(a, tpb, stream);
        if (bits == 3) return launch_exact<3, KW_OFFSET>(a, tpb, stream);
        return launch_exact<4, KW_OFFSET>(a, tpb, stream);
    }
    if (bits == 2) return launch_exact<2, KW_ZERO>(a, tpb, stream);
    if (bits == 3) return launch_exact<3, KW_ZERO>(a, tpb, stream);
    // 4-bit codes with integer zero points: exact-integer operands at one
    // batch block, where the fp16 dequantization of every weight feeds a
    // single product; from two batch blocks on, the per-round correction of
    // every block costs more than the dequantization it saves.
    if (B <= 8) return launch_ncb<1, 4, KW_ZERO, 2>(a, tpb, stream);
    if (B <= 16) return launch_ncb<1, 4, KW_ZERO>(a, tpb, stream);
    if (B <= 32) return launch_ncb<2, 4, KW_DEQUANT>(a, tpb, stream);
    return launch_ncb<4, 4, KW_DEQUANT>(a, tpb, stream);
}

}  // namespace wq
