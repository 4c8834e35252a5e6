// Internal launchers (C++), called by the C ABI after validation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

// Caller-owned scratch of one call.  Every launcher that can use scratch runs
// in one of two modes:
//   - sizing (need != nullptr): nothing is launched; *need is raised to the
//     bytes the call's preferred plan uses (the largest of its launches, which
//     run one after another on the stream and so share the buffer);
//   - launching (need == nullptr): with ptr set (at least the sized bytes,
//     16-byte aligned) the preferred plan runs; with ptr null a plan that
//     needs no scratch runs instead.
// Both modes take the same decisions, so the size always matches the launch.
struct Scratch {
    void* ptr = nullptr;
    size_t* need = nullptr;
    bool sizing() const { return need != nullptr; }
    void want(size_t bytes) const {
        if (need && *need < bytes) *need = bytes;
    }
};

// scheme: 0 asymmetric, 1 symmetric per group, 2 symmetric per tensor (the
// last needs scratch for its maximum: quantize_scratch_bytes), 3 NF4,
// 4 float offset.
size_t quantize_scratch_bytes(int32_t scheme);
hipError_t launch_quantize_pack(const void* W, int64_t N, int64_t K, int32_t group,
                                int32_t bits, int32_t scheme, void* codes, void* scales,
                                void* zeros, void* scratch, hipStream_t stream);

// Codes + headers -> fp32 W [N, K] for any scheme (see wq_dequant.hip).
hipError_t launch_dequantize(const void* codes, const void* scales, const void* zeros, void* W,
                             int64_t N, int64_t K, int32_t group, int32_t bits, int32_t scheme,
                             hipStream_t stream);

// GEMV family: returns hipErrorInvalidValue when the shape is outside what the
// instantiated tilings cover (the caller maps that to WQ_ERR_UNSUPPORTED).
bool gemv_supports(int64_t K, int32_t bits);
hipError_t launch_gemv(const void* X, const void* codes, const void* scales,
                       const void* zeros, void* Y, int64_t B, int64_t K, int64_t N,
                       int32_t group, int32_t bits, int num_cus, hipStream_t stream);

// Bit-stream GEMV (any batch; codes re-streamed once per 4 batch rows): 2/3-bit
// codes with integer zero points (offset = 0), or 2/3/4/8-bit codes of the
// float-offset variant (offset = 1, `zeros` holds the group minima).
bool gemv_lowbit_supports(int64_t K, int32_t group, int32_t bits);
hipError_t launch_gemv_lowbit(const void* X, const void* codes, const void* scales,
                              const void* zeros, void* Y, int64_t B, int64_t K, int64_t N,
                              int32_t group, int32_t bits, int offset, int num_cus, hipStream_t stream);

// NF4 GEMV (level table lookup; any batch, codes re-streamed per four rows).
bool gemv_nf4_supports(int64_t K, int32_t group);
hipError_t launch_gemv_nf4(const void* X, const void* codes, const void* scales, void* Y, int64_t B,
                           int64_t K, int64_t N, int32_t group, int num_cus, hipStream_t stream);

// Matrix-core family: the X-resident kernel for B <= 32 (xr_*), the tiled
// kernel beyond.
bool xr_supports(int64_t B, int64_t K, int32_t group, int32_t bits);
// Shapes the X-resident kernel can take at all (a superset of xr_supports:
// beyond it, it is chosen only when other products share the launch).
bool xr_groupable(int64_t B, int64_t K, int32_t group, int32_t bits);
// Whether the X-resident kernel takes the product without scratch (one
// K-slice holds all of X).
bool xr_single_slice(int64_t B, int64_t K, int32_t bits);
// Several X-resident products of one batch size and bit width (each must
// satisfy xr_groupable): products sharing a header mode go into one launch of
// up to eight, with one reduction launch for their K-slices; a product alone
// in its launch that xr_supports rejects runs on the tiled kernel instead, and
// so does, without scratch, a product whose X needs several K-slices.
struct XrProduct {
    const void* X;
    const void* codes;
    const void* scales;
    const void* zeros;
    void* Y;
    int64_t K, N;
    int32_t group;
};
hipError_t launch_gemm_xr_many(const XrProduct* prods, int count, int64_t B, int32_t bits,
                               int num_cus, const Scratch& ws, hipStream_t stream);
bool mfma_supports(int64_t K, int32_t group, int32_t bits);
// Whether launch_gemm_mfma takes the product: the quad-stream or quad-row
// kernels' shapes (B <= 4, groups of 64 or 32 and up, header arrays 16- or
// 8-byte aligned; null header pointers count as aligned), or the tiled
// kernels' group % 128 (bits 4) / 64 (8).
bool qs_takes(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits, const void* scales,
              const void* zeros);
bool q4_takes(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits, const void* scales,
              const void* zeros);
bool mfma_path_takes(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits, const void* scales,
                     const void* zeros);
bool ts_takes(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits, const void* scales,
              const void* zeros);
// K-split-wave matrix-core kernel (wq_gemm_kw.hip): needs no scratch; group
// 128, K = 2048, 4096 or 8192, X 16-byte aligned.  4-bit codes with integer
// zero points up to B = 64; 2- and 3-bit codes, and float offsets (offset:
// `zeros` holds the group minima m, x_hat = q s + m) at bits 2, 3 and 4, up
// to B = 32.  kw_takes adds the shape choice: at least 1.8 16-row tiles
// per compute unit, 16-byte aligned header arrays (null counts as aligned),
// and B > 4 for 4-bit integer-zero codes (where the quad-stream kernel takes
// B <= 4), B >= 2 otherwise.
bool kw_supports(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits, bool offset);
bool kw_takes(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits, bool offset, const void* X,
              const void* scales, const void* zeros, int num_cus);
int kw_tiles_per_block(int64_t N, int num_cus);
// NF4 codes (wq_gemm_nf4) on the same kernel: blocks of 64 only, 2 <= B <= 32,
// K = 2048, 4096 or 8192, at least 1.8 16-row tiles per compute unit, X and
// scales 16-byte aligned.
bool kw_nf4_takes(int64_t B, int64_t K, int64_t N, int32_t group, const void* X, const void* scales,
                  int num_cus);
hipError_t launch_gemm_kw_nf4(const void* X, const void* codes, const void* scales, void* Y, int64_t B, int64_t K,
                              int64_t N, int32_t group, int num_cus, hipStream_t stream);
hipError_t launch_gemm_kw(const void* X, const void* codes, const void* scales, const void* zeros, void* Y,
                          int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits, bool offset, int num_cus,
                          hipStream_t stream);
// Tile-stream 16x16x32 matrix-core kernel for B <= 16 (wq_gemm_ts.hip): needs
// no scratch; group 128, K % 512 == 0, header arrays 8-byte aligned.
bool ts_supports(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits);
hipError_t launch_gemm_ts(const void* X, const void* codes, const void* scales, const void* zeros, void* Y,
                          int64_t B, int64_t K, int64_t N, int32_t group, int num_cus, hipStream_t stream);
// Quad-stream 4x4x4 matrix-core kernel for B <= 4 (wq_gemm_qs.hip): needs no
// scratch; its header arrays must be 16-byte aligned.
bool qs_supports(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits);
hipError_t launch_gemm_qs(const void* X, const void* codes, const void* scales, const void* zeros, void* Y,
                          int64_t B, int64_t K, int64_t N, int32_t group, int num_cus, hipStream_t stream);
// Quad-row 4x4x4 matrix-core kernel for B <= 4 (wq_gemm_q4.hip): needs no
// scratch; its header arrays must be 8-byte aligned.
bool q4_supports(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits);
hipError_t launch_gemm_q4(const void* X, const void* codes, const void* scales, const void* zeros, void* Y,
                          int64_t B, int64_t K, int64_t N, int32_t group, int num_cus, hipStream_t stream);
// Streaming matrix-core kernel for B <= 16 (wq_gemm_sk.hip): needs no scratch.
bool sk_supports(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits);
hipError_t launch_gemm_sk(const void* X, const void* codes, const void* scales, const void* zeros, void* Y,
                          int64_t B, int64_t K, int64_t N, int32_t group, int num_cus, hipStream_t stream);
// Matrix-core product (X-resident kernel when it takes the shape, else the
// tiled kernel); scratch holds fp32 split-K partials.
hipError_t launch_gemm_mfma(const void* X, const void* codes, const void* scales,
                            const void* zeros, void* Y, int64_t B, int64_t K, int64_t N,
                            int32_t group, int32_t bits, int num_cus, const Scratch& ws,
                            hipStream_t stream);

// int4 KV cache of `heads` heads (head dimension 128, blocks of 128 tokens,
// `max_blocks` blocks per head); layouts in wq_kv.hip.
struct KvCacheArgs {
    void* kcodes;
    void* kscales;
    void* kzeros;
    void* vcodes;
    void* vscales;
    void* vzeros;
    void* kres;
    void* vres;
    int64_t heads, max_blocks;
};
int kv_splits(int64_t heads, int64_t max_blocks, int num_cus);
// Scratch holds the fp32 partials of the context splits; without it every
// head runs as one split.
hipError_t launch_kv_attention(const void* q, const KvCacheArgs& c, const int32_t* lens, void* out,
                               int num_cus, const Scratch& ws, hipStream_t stream);
hipError_t launch_kv_quantize(const void* K, const void* V, const KvCacheArgs& c, int64_t block,
                              hipStream_t stream);

}  // namespace wq
