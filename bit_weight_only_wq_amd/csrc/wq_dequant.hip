// Dequantization of packed codes to fp32 [N, K]: the reconstruction a
// product performs as it reads ("Quantization & inference optimisation",
// "Quantization": the integer and the group's endpoints give back an
// approximate float), written out as a tensor so that it can be compared with
// a reference value for value.  Not on the hot path.
//
//   schemes 0-2 (integer zero point):  W = (q - z) * s
//   scheme 3 (NF4, 4-bit):             W = level[q] * s
//   scheme 4 (float offset):           W = q * s + m     (zeros holds m)
//
// Each form is rounded once to fp32: q - z is an integer of at most 17 bits
// (exact), level and s are fp16 (their product has at most 22 significant
// bits, exact), and q * s + m is one fused multiply-add.
//
// Codes of a row form a little-endian bit stream (code k at bits
// [k*bits, k*bits + bits) of the row's bytes), so 8 consecutive codes occupy
// exactly `bits` bytes.  One thread reconstructs one such octet; groups are
// multiples of 8, so an octet never spans two groups.
#include "wq_device.h"
#include "wq_launch.h"
#include "wq_nf4_levels.h"

namespace wq {

namespace {

__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint16_t* __restrict__ zeros,
                                                      float* __restrict__ W, int64_t N, int64_t K,
                                                      int32_t G, int32_t bits, int32_t scheme) {
    const int64_t per_row = K / 8;
    const int64_t oct = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (oct >= N * per_row) return;
    const int64_t n = oct / per_row, j = oct - n * per_row;
    const uint8_t* p = codes + n * (K / 8 * bits) + j * bits;
    uint64_t u = 0;
    for (int i = 0; i < bits; ++i) u |= (uint64_t)p[i] << (8 * i);
    const int64_t gi = n * (K / G) + (j * 8) / G;
    const float s = half_bits_to_float(scales[gi]);
    const float z = half_bits_to_float(zeros[gi]);
    const uint32_t mask = (1u << bits) - 1u;
    float out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t q = (uint32_t)(u >> (i * bits)) & mask;
        if (scheme == 3) out[i] = half_bits_to_float(kNf4LevelBits[q & 15u]) * s;
        else if (scheme == 4) out[i] = __builtin_fmaf((float)q, s, z);
        else out[i] = ((float)q - z) * s;
    }
    float4* w = reinterpret_cast<float4*>(W + n * K + j * 8);
    w[0] = make_float4(out[0], out[1], out[2], out[3]);
    w[1] = make_float4(out[4], out[5], out[6], out[7]);
}

}  // namespace

hipError_t launch_dequantize(const void* codes, const void* scales, const void* zeros, void* W,
                             int64_t N, int64_t K, int32_t group, int32_t bits, int32_t scheme,
                             hipStream_t stream) {
    const int64_t octets = N * (K / 8);
    if (octets == 0) return hipSuccess;
    const int64_t blocks = (octets + 255) / 256;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    dequant_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
        static_cast<const uint8_t*>(codes), static_cast<const uint16_t*>(scales),
        static_cast<const uint16_t*>(zeros), static_cast<float*>(W), N, K, group, bits, scheme);
    return hipGetLastError();
}

}  // namespace wq
