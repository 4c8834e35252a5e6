// Decode attention over an int4 KV cache (gfx950), and the quantize-on-append
// step that fills it.
//
// "What actually happens when you quantize a KV cache": one decode step
// scores the new query against every cached key and averages the values with
// the softmax weights (§2); the cache holds the group-wise asymmetric int4
// codec of §3-§4, K grouped per channel over 128 tokens and V per token (§7
// "axis choice"), with the newest tokens that do not fill a K group in fp16;
// the step streams the whole cache, so it is bandwidth-bound (§6).
//
// Cache of one head (head dimension D = 128, blocks of G = 128 tokens):
//   kcodes [blocks][G tokens][64 B]   token-major: byte i of token t holds
//                                     channels 2i (low nibble) and 2i+1
//   kscales, kzeros [blocks][D]       fp16, one per channel per block
//   vcodes [blocks][D channels][64 B] channel-major: byte i of channel d
//                                     holds tokens 2i (low nibble) and 2i+1
//   vscales, vzeros [blocks * G]      fp16, one per token
//   kres, vres [G][D]                 fp16, the residual tokens (token-major)
// Codes are stored against the grouping axis on purpose: a score is
//   sum_d q_d s_d (c_td - z_d) = sum_d a_d c_td - sum_d a_d z_d,  a_d = q_d s_d,
// a dot product along a 64-byte token row with a per-block vector a, and an
// output channel is
//   sum_t p_t s_t (c_dt - z_t) = sum_t w_t c_dt - sum_t w_t z_t,  w_t = p_t s_t,
// a dot product along a 64-byte channel row with a per-block vector w.  Both
// run like the weight GEMV: codes unpack to fp16 (1024 + c) or (1024 + 16c)
// pairs with one AND-OR, and v_dot2_f32_f16 multiplies them by a or w, held as
// an fp16 hi/lo pair (a = hi + lo to 2^-22) so the products keep fp32
// accuracy; the offsets and zero points enter once per block.
//
// Attention is split over the context (flash decoding): each (head, split)
// workgroup streams its blocks with a running max, sum and output, and a
// second kernel combines the splits.  Scores are kept in log2 units (log2(e)
// and 1/sqrt(D) folded into a), so the softmax uses v_exp_f32 directly.
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

namespace {

constexpr int kD = 128;         // head dimension
constexpr int kG = 128;         // tokens per block
constexpr int kRow = 64;        // bytes per code row
constexpr uint32_t kMagic = 0x64006400u;

// LDS slot (in fp16 units) of position u (0..127) of a row in unpack order:
// quarter k = u / 32 is one 16-byte chunk; within it word j = (u % 32) / 8
// holds 8 codes, unpacked as the pairs (0,4) (1,5) (2,6) (3,7) -> uint4
// components x, y, z, w; the first code of a pair is the low half.
__device__ __forceinline__ int pair_slot(int u) {
    const int k = u >> 5, j = (u >> 3) & 3, r = u & 7;
    return (((k * 4 + j) * 4 + (r & 3)) << 1) | (r >> 2);
}

// Offset that position u carries in the unpacked pair: 1024 (even u) or,
// after the 1/16 rescale, 64 (odd u).
__device__ __forceinline__ float unpack_offset(int u) { return (u & 1) ? 64.0f : 1024.0f; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// dot of one 16-byte chunk (32 codes) with the hi/lo vector of its quarter
// (xh, xl: 4 uint4 each), codes as (1024 + c) / (1024 + 16c) pairs.
__device__ __forceinline__ float chunk_dot_hl(const uint4& w4, const uint4* xh, const uint4* xl,
                                              uint32_t m_lo, uint32_t m_hi) {
    const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
    float pa = 0.0f, pb = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t sh = w[j] >> 8;
        const h2_t q04 = as_h2((w[j] & m_lo) | kMagic);
        const h2_t q15 = as_h2((w[j] & m_hi) | kMagic);
        const h2_t q26 = as_h2((sh & m_lo) | kMagic);
        const h2_t q37 = as_h2((sh & m_hi) | kMagic);
        pa = __builtin_amdgcn_fdot2(q04, as_h2(xh[j].x), pa, false);
        pa = __builtin_amdgcn_fdot2(q04, as_h2(xl[j].x), pa, false);
        pb = __builtin_amdgcn_fdot2(q15, as_h2(xh[j].y), pb, false);
        pb = __builtin_amdgcn_fdot2(q15, as_h2(xl[j].y), pb, false);
        pa = __builtin_amdgcn_fdot2(q26, as_h2(xh[j].z), pa, false);
        pa = __builtin_amdgcn_fdot2(q26, as_h2(xl[j].z), pa, false);
        pb = __builtin_amdgcn_fdot2(q37, as_h2(xh[j].w), pb, false);
        pb = __builtin_amdgcn_fdot2(q37, as_h2(xl[j].w), pb, false);
    }
    return __builtin_fmaf(pb, 0.0625f, pa);
}

// Block-wide sum / max over the four waves through `red` (one barrier).  The
// caller keeps `red` untouched until every thread has read it: the kernels
// below use a separate `red` per reduction of a block and reach another
// barrier before a reduction reuses its array.
__device__ __forceinline__ float block_sum(float v, float* red) {
    v = group_sum<64>(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
}

struct KvPtrs {
    const uint8_t* kc;
    const uint16_t* ks;
    const uint16_t* kz;
    const uint8_t* vc;
    const uint16_t* vs;
    const uint16_t* vz;
    const uint16_t* kr;
    const uint16_t* vr;
    int64_t max_blocks;
};

// One workgroup per (head, split).  Thread i: quad i/4 owns rows r0 = i/4 and
// r0 + 64 of a block (tokens in the score phase, channels in the output
// phase), lane i%4 the quarter (32 codes) of those rows.
__global__ __launch_bounds__(256) void kv_attn_kernel(const uint16_t* __restrict__ Q, const KvPtrs P,
                                                      const int32_t* __restrict__ lens, int splits,
                                                      float q_scale, float* __restrict__ part,
                                                      uint16_t* __restrict__ out) {
    // Per-block vectors in unpack order, hi and lo halves: a (K side) and w
    // (V side) in separate arrays, and one reduction array per block-wide
    // reduction.  Barrier order then keeps every array's readers ahead of its
    // next writers: a thread rewrites kh/kl only after all threads passed the
    // previous block's softmax barrier (their last kh/kl reads came before
    // it), and vh/vl only after all passed this block's C_K barrier.
    __shared__ __align__(16) uint16_t kh[kD], kl[kD], vh[kG], vl[kG];
    __shared__ float qf[kD];
    __shared__ float pr[kG];                        // residual-token weights
    __shared__ float red_k[4], red_m[4], red_v[4], red_r[4];

    const int h = blockIdx.x;
    const int sp = blockIdx.y;
    const int tid = threadIdx.x;
    const int quad = tid >> 2, qk = tid & 3;
    const int r0 = quad, r1 = quad + 64;

    // Tokens of this head, clamped to what the cache holds.
    int64_t len = lens[h];
    const int64_t cap = P.max_blocks * kG + (kG - 1);
    len = len < 0 ? 0 : (len > cap ? cap : len);
    const int nblk = (int)(len / kG) < P.max_blocks ? (int)(len / kG) : (int)P.max_blocks;
    const int nres = (int)(len - (int64_t)nblk * kG);
    const int bps = (nblk + splits - 1) / splits;
    const int j0 = sp * bps;
    const int j1 = (j0 + bps) < nblk ? (j0 + bps) : nblk;
    const bool last = sp == splits - 1;

    if (tid < kD) qf[tid] = half_bits_to_float(Q[(int64_t)h * kD + tid]) * q_scale;
    __syncthreads();

    const uint32_t m_lo = vgpr_const(0x000F000Fu);
    const uint32_t m_hi = vgpr_const(0x00F000F0u);
    float M = -__builtin_huge_valf();    // running max (log2 units)
    float lsum = 0.0f;                   // this thread's share of sum p (lane qk == 0 rows)
    float o0 = 0.0f, o1 = 0.0f;          // output channels r0, r1 (all four lanes of the quad)

    // One block's loads for this thread: its four 16-byte code chunks, the K
    // header of channel tid % 128 and the V headers of its two tokens.  Every
    // lane issues the same ten loads in the order they are consumed (lanes
    // that do not use a header still load it), so the K side's waits leave
    // the next block's loads in flight.  The prefetch is conditional (no
    // block past the split is read), so the V side's header waits drain them;
    // an unconditional, clamped prefetch kept them in flight but measured no
    // faster and re-read one block per split.
    struct Blk {
        uint4 k0, k1, v0, v1;
        uint32_t ks, kz, vs0, vs1, vz0, vz1;
    };
    const int64_t hb = (int64_t)h * P.max_blocks;
    auto load_blk = [&](int j, Blk& b) {
        const int64_t blk = hb + j;
        const uint4* kc = reinterpret_cast<const uint4*>(P.kc + blk * (kG * kRow));
        const uint4* vc = reinterpret_cast<const uint4*>(P.vc + blk * (kD * kRow));
        const int64_t tb = blk * kG;
        b.k0 = load_stream(kc + r0 * 4 + qk);
        b.k1 = load_stream(kc + r1 * 4 + qk);
        b.ks = P.ks[blk * kD + (tid & (kD - 1))];
        b.kz = P.kz[blk * kD + (tid & (kD - 1))];
        b.v0 = load_stream(vc + r0 * 4 + qk);
        b.v1 = load_stream(vc + r1 * 4 + qk);
        b.vs0 = P.vs[tb + r0];
        b.vs1 = P.vs[tb + r1];
        b.vz0 = P.vz[tb + r0];
        b.vz1 = P.vz[tb + r1];
    };
    auto process = [&](const Blk& b) {
        // ---- K side: a_d = q_d s_d as hi/lo, and C_K = sum_d a_d (off_d + z_d).
        float ck = 0.0f;
        if (tid < kD) {
            const float a = qf[tid] * half_bits_to_float((uint16_t)b.ks);
            const _Float16 ah = (_Float16)a;
            const _Float16 al = (_Float16)(a - (float)ah);
            kh[pair_slot(tid)] = __builtin_bit_cast(uint16_t, ah);
            kl[pair_slot(tid)] = __builtin_bit_cast(uint16_t, al);
            ck = ((float)ah + (float)al) * (unpack_offset(tid) + half_bits_to_float((uint16_t)b.kz));
        }
        const float CK = block_sum(ck, red_k);      // (its barrier also publishes kh/kl)
        const uint4* khq = reinterpret_cast<const uint4*>(kh) + qk * 4;
        const uint4* klq = reinterpret_cast<const uint4*>(kl) + qk * 4;
        const float s0 = group_sum<4>(chunk_dot_hl(b.k0, khq, klq, m_lo, m_hi)) - CK;
        const float s1 = group_sum<4>(chunk_dot_hl(b.k1, khq, klq, m_lo, m_hi)) - CK;

        // ---- softmax update over the block's 128 scores.
        const float bm = block_max(__builtin_fmaxf(s0, s1), red_m);
        const float Mn = __builtin_fmaxf(M, bm);
        const float alpha = exp2_fast(M - Mn);
        M = Mn;
        const float p0 = exp2_fast(s0 - Mn), p1 = exp2_fast(s1 - Mn);
        lsum = lsum * alpha + (qk == 0 ? p0 + p1 : 0.0f);
        o0 *= alpha;
        o1 *= alpha;

        // ---- V side: w_t = p_t s_t as hi/lo, C_V = sum_t w_t (off_t + z_t),
        // written by lane 0 of each quad for its two tokens.
        float cv = 0.0f;
        if (qk == 0) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int t = e ? r1 : r0;
                const float w = (e ? p1 : p0) * half_bits_to_float((uint16_t)(e ? b.vs1 : b.vs0));
                const _Float16 wh = (_Float16)w;
                const _Float16 wl = (_Float16)(w - (float)wh);
                vh[pair_slot(t)] = __builtin_bit_cast(uint16_t, wh);
                vl[pair_slot(t)] = __builtin_bit_cast(uint16_t, wl);
                cv += ((float)wh + (float)wl) *
                      (unpack_offset(t) + half_bits_to_float((uint16_t)(e ? b.vz1 : b.vz0)));
            }
        }
        const float CV = block_sum(cv, red_v);      // (its barrier also publishes vh/vl)
        const uint4* vhq = reinterpret_cast<const uint4*>(vh) + qk * 4;
        const uint4* vlq = reinterpret_cast<const uint4*>(vl) + qk * 4;
        o0 += group_sum<4>(chunk_dot_hl(b.v0, vhq, vlq, m_lo, m_hi)) - CV;
        o1 += group_sum<4>(chunk_dot_hl(b.v1, vhq, vlq, m_lo, m_hi)) - CV;
    };

    Blk A = {}, B = {};
    if (j0 < j1) load_blk(j0, A);
    for (int j = j0; j < j1; j += 2) {
        if (j + 1 < j1) load_blk(j + 1, B);
        process(A);
        if (j + 1 >= j1) break;
        if (j + 2 < j1) load_blk(j + 2, A);
        process(B);
    }

    // ---- residual tokens (fp16), last split only.
    if (last && nres > 0) {
        const uint16_t* kr = P.kr + (int64_t)h * kG * kD;
        const uint16_t* vr = P.vr + (int64_t)h * kG * kD;
        float s = -__builtin_huge_valf();
        if (tid < nres) {
            s = 0.0f;
            const uint4* row = reinterpret_cast<const uint4*>(kr + (int64_t)tid * kD);
#pragma unroll 4
            for (int c = 0; c < kD / 8; ++c) {
                const uint4 u = row[c];
                const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    s = __builtin_fmaf(half_bits_to_float((uint16_t)(w[i] & 0xFFFFu)), qf[8 * c + 2 * i], s);
                    s = __builtin_fmaf(half_bits_to_float((uint16_t)(w[i] >> 16)), qf[8 * c + 2 * i + 1], s);
                }
            }
        }
        const float bm = block_max(s, red_r);
        const float Mn = __builtin_fmaxf(M, bm);
        const float alpha = exp2_fast(M - Mn);
        M = Mn;
        const float p = tid < nres ? exp2_fast(s - Mn) : 0.0f;
        if (tid < kG) pr[tid] = p;
        lsum = lsum * alpha + p;          // residual weights counted by their own thread
        o0 *= alpha;
        o1 *= alpha;
        __syncthreads();
        if (qk == 0) {
            float a0 = 0.0f, a1 = 0.0f;
            for (int t = 0; t < nres; ++t) {
                a0 = __builtin_fmaf(pr[t], half_bits_to_float(vr[(int64_t)t * kD + r0]), a0);
                a1 = __builtin_fmaf(pr[t], half_bits_to_float(vr[(int64_t)t * kD + r1]), a1);
            }
            o0 += a0;
            o1 += a1;
        }
        // (the other lanes of the quad keep stale o0/o1; only qk == 0 stores)
    }

    // Total of the per-thread sums of p (red_k's last readers passed at least
    // two barriers since, or it was never used).
    const float lt = block_sum(lsum, red_k);

    if (splits == 1) {
        if (qk == 0) {
            const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
            out[(int64_t)h * kD + r0] = float_to_half_bits_rne(o0 * inv);
            out[(int64_t)h * kD + r1] = float_to_half_bits_rne(o1 * inv);
        }
        return;
    }
    float* pp = part + ((int64_t)h * splits + sp) * (kD + 4);
    if (tid == 0) {
        pp[0] = M;
        pp[1] = lt;
    }
    if (qk == 0) {
        pp[4 + r0] = o0;
        pp[4 + r1] = o1;
    }
}

// out[h, d] = sum_s 2^(M_s - M) o_s[d] / sum_s 2^(M_s - M) l_s.
__global__ __launch_bounds__(128) void kv_combine_kernel(const float* __restrict__ part, int splits,
                                                         uint16_t* __restrict__ out) {
    const int h = blockIdx.x;
    const int d = threadIdx.x;
    const float* pp = part + (int64_t)h * splits * (kD + 4);
    float M = -__builtin_huge_valf();
    for (int s = 0; s < splits; ++s) M = __builtin_fmaxf(M, pp[s * (kD + 4)]);
    float num = 0.0f, den = 0.0f;
    if (M > -__builtin_huge_valf()) {
        for (int s = 0; s < splits; ++s) {
            const float f = exp2_fast(pp[s * (kD + 4)] - M);
            num = __builtin_fmaf(f, pp[s * (kD + 4) + 4 + d], num);
            den = __builtin_fmaf(f, pp[s * (kD + 4) + 1], den);
        }
    }
    out[(int64_t)h * kD + d] = float_to_half_bits_rne(den > 0.0f ? num / den : 0.0f);
}

// ---- quantize-on-append ------------------------------------------------------
// Eight workgroups per head (K by channel quarters, V by token quarters): the
// head's block of G tokens of K and V (fp16, token-major [G][D]) becomes
// block `block` of its cache.  K: min/max per channel over the G tokens; V:
// per token over the D channels; both with the exact decisions of the weight
// quantizer.
//
// A workgroup owns Q = 32 groups of 128 elements (K: channels 32q .. 32q + 31
// over the tokens; V: tokens 32q .. 32q + 31 over the channels).  Thread
// (p, e) = (tid % 16, tid / 16) holds groups 2p and 2p + 1 at elements
// 8e .. 8e + 7 in registers, so its two group headers are two values in
// registers rather than one LDS read per code: min/max over the element
// blocks (lanes 16 and 32 apart, then the 4 waves through LDS), the headers
// from 32 lanes, then the fp32 estimate of every code with the exact
// fallback of the weight quantizer when a lane of the wave needs it.  Code
// byte (2p, 2p + 1) of element row r goes into an LDS tile of the
// workgroup's 128 rows x 16 bytes, from which each thread writes 8 bytes of
// one row.
__device__ __forceinline__ float kv_encode_exact(float x, float s, float rcp, float Z) {
    const float t = __builtin_amdgcn_fmed3f(x * rcp, -Z - 2.0f, 15.0f - Z + 2.0f);
    const float kl = __builtin_floorf(t);
    const float r = __builtin_fmaf(-(kl + 0.5f), s, x);
    const float half = kl * 0.5f;
    const bool odd = __builtin_rintf(half) != half;
    const bool inc = (r > 0.0f) | ((r == 0.0f) & odd);   // no short-circuit branches
    return inc ? kl + 1.0f : kl;
}

__global__ __launch_bounds__(256) void kv_quantize_kernel(const uint16_t* __restrict__ K,
                                                          const uint16_t* __restrict__ V,
                                                          uint8_t* __restrict__ kc, uint16_t* __restrict__ ks,
                                                          uint16_t* __restrict__ kz, uint8_t* __restrict__ vc,
                                                          uint16_t* __restrict__ vs, uint16_t* __restrict__ vz,
                                                          int64_t max_blocks, int64_t block) {
    constexpr int Q = 32;                       // groups per workgroup
    __shared__ float mnx[4][2][Q];              // per-wave partial min / max
    __shared__ float4 hdr[Q];                   // s, rcp, Z, thr
    __shared__ __align__(8) uint8_t ctile[kG * (Q / 2)];   // [128 rows][16 bytes]

    const int h = blockIdx.x;
    const int side = blockIdx.y >> 2, q = blockIdx.y & 3;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int p = tid & 15, e = tid >> 4;
    const int64_t blk = (int64_t)h * max_blocks + block;

    // x[g][i]: group 2p + g at element 8e + i.
    float x[2][8];
    if (side == 0) {
        // K [G][D]: channels 32q + 2p, + 1 of tokens 8e .. 8e + 7 (one dword each).
        const uint16_t* src = K + ((int64_t)h * kG + 8 * e) * kD + Q * q + 2 * p;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t u = *reinterpret_cast<const uint32_t*>(src + (int64_t)i * kD);
            x[0][i] = half_bits_to_float((uint16_t)u);
            x[1][i] = half_bits_to_float((uint16_t)(u >> 16));
        }
    } else {
        // V [G][D]: channels 8e .. 8e + 7 of tokens 32q + 2p, + 1 (16 bytes each).
        const uint16_t* src = V + ((int64_t)h * kG + Q * q + 2 * p) * kD + 8 * e;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const uint4 u = *reinterpret_cast<const uint4*>(src + (int64_t)g * kD);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[g][2 * j] = half_bits_to_float((uint16_t)w[j]);
                x[g][2 * j + 1] = half_bits_to_float((uint16_t)(w[j] >> 16));
            }
        }
    }
    float mn[2], mx[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        mn[g] = x[g][0];
        mx[g] = x[g][0];
#pragma unroll
        for (int i = 1; i < 8; ++i) {
            mn[g] = __builtin_fminf(mn[g], x[g][i]);
            mx[g] = __builtin_fmaxf(mx[g], x[g][i]);
        }
#pragma unroll
        for (int o = 16; o < 64; o <<= 1) {   // the wave's 4 element blocks
            mn[g] = __builtin_fminf(mn[g], __shfl_xor(mn[g], o, 64));
            mx[g] = __builtin_fmaxf(mx[g], __shfl_xor(mx[g], o, 64));
        }
    }
    if (lane < 16) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            mnx[wv][0][2 * p + g] = mn[g];
            mnx[wv][1][2 * p + g] = mx[g];
        }
    }
    __syncthreads();
    if (tid < Q) {
        float a = mnx[0][0][tid], b = mnx[0][1][tid];
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) {
            a = __builtin_fminf(a, mnx[ww][0][tid]);
            b = __builtin_fmaxf(b, mnx[ww][1][tid]);
        }
        const GroupHeader g = make_header(a, b, 15);
        hdr[tid] = make_float4(g.s, g.rcp, g.Z, g.thr);
        if (side == 0) {
            ks[blk * kD + Q * q + tid] = g.sbits;
            kz[blk * kD + Q * q + tid] = g.zbits;
        } else {
            vs[blk * kG + Q * q + tid] = g.sbits;
            vz[blk * kG + Q * q + tid] = g.zbits;
        }
    }
    __syncthreads();
    const float4 h0 = hdr[2 * p], h1 = hdr[2 * p + 1];
    const float hs_[2] = {h0.x, h1.x}, hr_[2] = {h0.y, h1.y}, hz_[2] = {h0.z, h1.z}, ht_[2] = {h0.w, h1.w};
    float k[2][8];
    bool near = false;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float t = x[g][i] * hr_[g];
            k[g][i] = __builtin_rintf(t);
            near |= __builtin_fabsf(t - k[g][i]) > ht_[g];
        }
    if (__builtin_amdgcn_ballot_w64(near) != 0) {
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int i = 0; i < 8; ++i) k[g][i] = kv_encode_exact(x[g][i], hs_[g], hr_[g], hz_[g]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t q0 = (uint32_t)__builtin_amdgcn_fmed3f(k[0][i] + hz_[0], 0.0f, 15.0f);
        const uint32_t q1 = (uint32_t)__builtin_amdgcn_fmed3f(k[1][i] + hz_[1], 0.0f, 15.0f);
        ctile[(8 * e + i) * (Q / 2) + p] = (uint8_t)(q0 | (q1 << 4));
    }
    __syncthreads();
    // Row r = tid / 2 (K: token, V: channel), bytes [8 (tid & 1), + 8) of the
    // quarter's 16.
    const int r = tid >> 1, hb = tid & 1;
    const uint2 w = *reinterpret_cast<const uint2*>(ctile + r * (Q / 2) + 8 * hb);
    uint8_t* dst = side == 0 ? kc + (blk * kG + r) * kRow : vc + (blk * kD + r) * kRow;
    *reinterpret_cast<uint2*>(dst + (Q / 2) * q + 8 * hb) = w;
}

}  // namespace

int kv_splits(int64_t heads, int64_t max_blocks, int num_cus) {
    // About six (head, split) workgroups per compute unit, but at least eight
    // blocks per split (each split pays for its query set-up, its prefetch
    // ramp and a partial in the combine), and at most 64 splits.  Measured on
    // 1024 heads x 4096 tokens (2 splits), 256 x 4096 (4) and 32 x 32768 (32).
    const int64_t h = heads > 0 ? heads : 1;
    int64_t s = ((int64_t)6 * num_cus + h - 1) / h;
    const int64_t by_len = max_blocks / 8 > 1 ? max_blocks / 8 : 1;
    if (s > by_len) s = by_len;
    if (s > 64) s = 64;
    return (int)(s < 1 ? 1 : s);
}

hipError_t launch_kv_attention(const void* q, const KvCacheArgs& c, const int32_t* lens, void* out,
                               int num_cus, const Scratch& ws, hipStream_t stream) {
    // Context splits write (max, sum, output row) partials into the scratch;
    // without scratch every head is one split.
    const int planned = kv_splits(c.heads, c.max_blocks, num_cus);
    const size_t part_bytes = planned > 1 ? (size_t)c.heads * planned * (kD + 4) * sizeof(float) : 0;
    if (ws.sizing()) {
        ws.want(part_bytes);
        return hipSuccess;
    }
    const int splits = ws.ptr ? planned : 1;
    float* part = splits > 1 ? static_cast<float*>(ws.ptr) : nullptr;
    const KvPtrs P{static_cast<const uint8_t*>(c.kcodes), static_cast<const uint16_t*>(c.kscales),
                   static_cast<const uint16_t*>(c.kzeros), static_cast<const uint8_t*>(c.vcodes),
                   static_cast<const uint16_t*>(c.vscales), static_cast<const uint16_t*>(c.vzeros),
                   static_cast<const uint16_t*>(c.kres), static_cast<const uint16_t*>(c.vres), c.max_blocks};
    // log2(e) / sqrt(D): scores in log2 units for v_exp_f32.
    const float q_scale = 1.4426950408889634f / 11.313708498984761f;
    kv_attn_kernel<<<dim3((unsigned)c.heads, (unsigned)splits), dim3(256), 0, stream>>>(
        static_cast<const uint16_t*>(q), P, lens, splits, q_scale, part, static_cast<uint16_t*>(out));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    kv_combine_kernel<<<dim3((unsigned)c.heads), dim3(kD), 0, stream>>>(part, splits, static_cast<uint16_t*>(out));
    return hipGetLastError();
}

hipError_t launch_kv_quantize(const void* K, const void* V, const KvCacheArgs& c, int64_t block,
                              hipStream_t stream) {
    kv_quantize_kernel<<<dim3((unsigned)c.heads, 8), dim3(256), 0, stream>>>(
        static_cast<const uint16_t*>(K), static_cast<const uint16_t*>(V), static_cast<uint8_t*>(c.kcodes),
        static_cast<uint16_t*>(c.kscales), static_cast<uint16_t*>(c.kzeros), static_cast<uint8_t*>(c.vcodes),
        static_cast<uint16_t*>(c.vscales), static_cast<uint16_t*>(c.vzeros), c.max_blocks, block);
    return hipGetLastError();
}

}  // namespace wq
