// Quantize/pack kernels (gfx950): fp16 W[N, K] -> codes, fp16 scales, fp16 zeros.
//
// Codec of "What actually happens when you quantize a KV cache", §3 steps 3-5
// and §4, per group of G consecutive k of a row:
//   min/max -> s = (max-min)/(2^b-1) stored fp16 -> z = round(-min/s) stored
//   fp16 -> q = clamp(round(x/s) + z, 0, 2^b-1) -> packed little-endian per row
//   (b = 4: even k in the low nibble).
// Rounding is half-to-even and every decision is the exact-rational one (see
// wq_device.h).  Degenerate scale -> 1.0; zero point saturates at +-65504.
//
// Layout: W, codes, scales and zeros are all flat row-major, and K % G == 0,
// so group gi covers W[gi*G .. gi*G + G) and writes scales[gi], zeros[gi]
// and codes bytes [gi*G*b/8, (gi+1)*G*b/8).  Each lane handles 8 consecutive
// values (one 16-byte load, one 4- or 8-byte store), so loads and stores of a
// wave are contiguous.
#include "wq_device.h"
#include "wq_launch.h"

namespace wq {

namespace {

template <int BITS>
struct Pack8;

template <>
struct Pack8<4> {
    typedef uint32_t type;  // 8 nibbles
    __device__ static type pack(const float* q) {
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) w |= (uint32_t)q[i] << (4 * i);
        return w;
    }
};

template <>
struct Pack8<8> {
    typedef uint2 type;  // 8 bytes
    __device__ static type pack(const float* q) {
        uint2 w;
        w.x = (uint32_t)q[0] | ((uint32_t)q[1] << 8) | ((uint32_t)q[2] << 16) | ((uint32_t)q[3] << 24);
        w.y = (uint32_t)q[4] | ((uint32_t)q[5] << 8) | ((uint32_t)q[6] << 16) | ((uint32_t)q[7] << 24);
        return w;
    }
};

__device__ __forceinline__ void load8(const uint16_t* p, float* x) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = half_bits_to_float((uint16_t)(w[i] & 0xFFFFu));
        x[2 * i + 1] = half_bits_to_float((uint16_t)(w[i] >> 16));
    }
}

// Per-group header from the exact min and max.
struct GroupHeader {
    float s, rcp, Z;
    uint16_t sbits, zbits;
};

__device__ __forceinline__ GroupHeader make_header(float mn, float mx, int M) {
    GroupHeader h;
    h.sbits = scale_bits_exact(mn, mx, M);
    h.s = half_bits_to_float(h.sbits);
    h.rcp = __builtin_amdgcn_rcpf(h.s);
    // z = round(-min / s): estimates beyond +-2^17 all saturate the fp16 zero.
    float k = rne_div_exact(-mn, h.s, h.rcp, -131072.0f, 131072.0f);
    h.zbits = zero_bits_from_int(k);
    h.Z = half_bits_to_float(h.zbits);
    return h;
}

template <int BITS>
__device__ __forceinline__ typename Pack8<BITS>::type encode8(const float* x, const GroupHeader& h) {
    constexpr float M = (float)((1 << BITS) - 1);
    // Outside [-Z-2, M-Z+2] every estimate clamps to code 0 or M anyway.
    const float lo = -h.Z - 2.0f, hi = M - h.Z + 2.0f;
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float k = rne_div_exact(x[i], h.s, h.rcp, lo, hi) + h.Z;
        q[i] = __builtin_fminf(__builtin_fmaxf(k, 0.0f), M);
    }
    return Pack8<BITS>::pack(q);
}

// Groups of G = 8*T values, T lanes per group (T a power of two <= 64).
// Thread t owns chunk t (values [8t, 8t+8) of the flat array).
template <int BITS, int T>
__global__ __launch_bounds__(256) void quantize_team_kernel(
    const uint16_t* __restrict__ W, typename Pack8<BITS>::type* __restrict__ codes,
    uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros, int64_t nchunks) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool live = t < nchunks;           // teams are all live or all dead
    const int64_t c = live ? t : nchunks - 1;
    float x[8];
    load8(W + c * 8, x);
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
        mn = __builtin_fminf(mn, x[i]);
        mx = __builtin_fmaxf(mx, x[i]);
    }
    group_minmax<T>(mn, mx);
    const GroupHeader h = make_header(mn, mx, (1 << BITS) - 1);
    if (!live) return;
    codes[c] = encode8<BITS>(x, h);
    if ((threadIdx.x & (T - 1)) == 0) {
        scales[c / T] = h.sbits;
        zeros[c / T] = h.zbits;
    }
}

// One wave per group for wide groups (G > 512 or G/8 not a power of two):
// pass 1 reduces min/max over the group, pass 2 re-reads and encodes.
template <int BITS>
__global__ __launch_bounds__(256) void quantize_wave_kernel(
    const uint16_t* __restrict__ W, typename Pack8<BITS>::type* __restrict__ codes,
    uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros, int64_t ngroups,
    int64_t G) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t g = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
    if (g >= ngroups) return;                // whole wave leaves together
    const int64_t cpg = G / 8;               // chunks per group
    const int64_t c0 = g * cpg;
    float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
    for (int64_t j = lane; j < cpg; j += kWave) {
        float x[8];
        load8(W + (c0 + j) * 8, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            mn = __builtin_fminf(mn, x[i]);
            mx = __builtin_fmaxf(mx, x[i]);
        }
    }
    group_minmax<kWave>(mn, mx);
    const GroupHeader h = make_header(mn, mx, (1 << BITS) - 1);
    for (int64_t j = lane; j < cpg; j += kWave) {
        float x[8];
        load8(W + (c0 + j) * 8, x);
        codes[c0 + j] = encode8<BITS>(x, h);
    }
    if (lane == 0) {
        scales[g] = h.sbits;
        zeros[g] = h.zbits;
    }
}

template <int BITS>
hipError_t launch_bits(const void* W, int64_t N, int64_t K, int32_t G, void* codes,
                       void* scales, void* zeros, hipStream_t stream) {
    typedef typename Pack8<BITS>::type P;
    const uint16_t* w = static_cast<const uint16_t*>(W);
    P* c = static_cast<P*>(codes);
    uint16_t* s = static_cast<uint16_t*>(scales);
    uint16_t* z = static_cast<uint16_t*>(zeros);
    const int64_t nchunks = N * K / 8;
    const int64_t ngroups = N * K / G;
    const int T = G / 8;
    const dim3 block(256);
    const dim3 team_grid((unsigned)((nchunks + 255) / 256));
    switch ((G <= 512 && (T & (T - 1)) == 0) ? T : 0) {
        case 1: quantize_team_kernel<BITS, 1><<<team_grid, block, 0, stream>>>(w, c, s, z, nchunks); break;
        case 2: quantize_team_kernel<BITS, 2><<<team_grid, block, 0, stream>>>(w, c, s, z, nchunks); break;
        case 4: quantize_team_kernel<BITS, 4><<<team_grid, block, 0, stream>>>(w, c, s, z, nchunks); break;
        case 8: quantize_team_kernel<BITS, 8><<<team_grid, block, 0, stream>>>(w, c, s, z, nchunks); break;
        case 16: quantize_team_kernel<BITS, 16><<<team_grid, block, 0, stream>>>(w, c, s, z, nchunks); break;
        case 32: quantize_team_kernel<BITS, 32><<<team_grid, block, 0, stream>>>(w, c, s, z, nchunks); break;
        case 64: quantize_team_kernel<BITS, 64><<<team_grid, block, 0, stream>>>(w, c, s, z, nchunks); break;
        default: {
            const dim3 grid((unsigned)((ngroups + 3) / 4));
            quantize_wave_kernel<BITS><<<grid, block, 0, stream>>>(w, c, s, z, ngroups, G);
        }
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_pack(const void* W, int64_t N, int64_t K, int32_t group,
                                int32_t bits, void* codes, void* scales, void* zeros,
                                hipStream_t stream) {
    if (bits == 4) return launch_bits<4>(W, N, K, group, codes, scales, zeros, stream);
    return launch_bits<8>(W, N, K, group, codes, scales, zeros, stream);
}

}  // namespace wq
