/*
 * wq.h — C ABI of the MI355X (gfx950) weight-only group-quantized decode GEMM.
 *
 * The library stores a weight matrix W[N, K] (fp16, row-major) as low-bit
 * codes plus one fp16 scale and one fp16 zero point per group of `group`
 * consecutive k of one row, and multiplies a batch of activations X[B, K]
 * against it while dequantizing in registers:
 *
 *     Y[b, n] = sum_k X[b, k] * (q[n, k] - z[n, k/G]) * s[n, k/G]
 *
 * Sources (by page title and section):
 *   "What actually happens when you quantize a KV cache", §3 steps 3-5 and §4:
 *       s = (max - min) / (2^b - 1), z = round(-min / s),
 *       q = clamp(round(x / s) + z, 0, 2^b - 1), x_hat = (q - z) * s,
 *       two 4-bit codes per byte with the even channel in the low nibble, and a
 *       4-byte header (fp16 scale + fp16 zero) per group kept in separate
 *       contiguous arrays.
 *   "Quantization & inference optimisation", sections "Bandwidth, not
 *       compute" (one decode step reads the weights once for the batch: 2B/w
 *       FLOP per byte) and "Quantization" (groups of consecutive weights from
 *       one row; the kernel reconstructs the float as it reads).
 *   "Serving many users at once: batching and quantization", sections
 *       "Batching" (the B users' rows are stacked into X and multiplied once per
 *       weight) and "Quantization" (groups along the in-features of a weight).
 *
 * Conventions shared by every entry point:
 *   - All array pointers are DEVICE pointers to row-major, contiguous buffers
 *     that the caller allocates, owns and frees.  The library allocates no
 *     device memory and keeps no state beyond a lazily cached device property
 *     (the compute-unit count).
 *   - Workspace.  Some calls can use scratch memory (fp32 partial sums when
 *     the product or the attention splits its work, the per-tensor maximum of
 *     the symmetric quantizer).  They take `workspace` (a device pointer,
 *     16-byte aligned) and `workspace_bytes`, and a matching
 *     wq_*_workspace_size query returns the bytes the call needs on the
 *     current device (0 if none).  workspace = NULL with workspace_bytes = 0
 *     means none: the call then takes a plan that needs no scratch (fewer work
 *     splits; same results within the product tolerance), except the
 *     per-tensor quantizer, which then fails with WQ_ERR_INVALID_ARG.  A
 *     workspace smaller than the query's answer is WQ_ERR_INVALID_ARG, a
 *     misaligned one WQ_ERR_MISALIGNED, both before any launch.  Its contents
 *     on entry do not matter; the call overwrites what it uses.  The
 *     workspace belongs to the call until the stream has run it: calls that
 *     may overlap (different streams) need different workspaces.
 *   - `stream` is a hipStream_t (NULL means the default stream).  Work is
 *     enqueued on it and the call returns at once; the library never
 *     synchronizes.  Buffers must stay alive until the stream has run the work.
 *   - Arguments are validated synchronously before any launch; on error
 *     nothing is enqueued.  A failed launch is reported as WQ_ERR_HIP.  No C++
 *     exception crosses the ABI.  wq_last_error() describes the last failure
 *     of the calling thread.
 *   - Inputs must be finite (no NaN/Inf); this is not checked.
 *   - Buffers must not alias one another.
 */
#ifndef WQ_H
#define WQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    WQ_OK = 0,
    WQ_ERR_INVALID_ARG = 1,  /* bad size, null pointer, K % group != 0, ... */
    WQ_ERR_UNSUPPORTED = 2,  /* valid for the codec, but not a layout the GPU kernels take */
    WQ_ERR_MISALIGNED = 3,   /* a pointer or row stride is not aligned as required */
    WQ_ERR_HIP = 4           /* the HIP runtime reported an error at launch */
} wq_status;

/* Kernel family for wq_gemm_ex. */
typedef enum {
    WQ_PATH_AUTO = 0,  /* GEMV for small batches, MFMA skinny GEMM beyond */
    WQ_PATH_GEMV = 1,  /* VALU dot products with wavefront (DPP) reductions */
    WQ_PATH_MFMA = 2   /* fp16 matrix-core tiles with fp32 accumulation */
} wq_path;

/*
 * Quantize and pack W (group-wise asymmetric, groups along K), as defined by
 * "What actually happens when you quantize a KV cache" §3 steps 3-5 and §4:
 *   per row n and group g of `group` consecutive k:
 *     s = fp16(round-half-even((max - min) / (2^bits - 1)))  (1.0 if that is 0)
 *     z = round-half-even(-min / s), stored as fp16 (saturating at +-65504;
 *         0 is stored as +0.0)
 *     q = clamp(round-half-even(x / s) + z, 0, 2^bits - 1)
 *   All rounding decisions are exact (as in exact rational arithmetic).
 *
 * W       fp16 [N, K]                 input, 16-byte aligned
 * codes   u8   [N, K*bits/8]          output; row n, code k sits at bits
 *                                     [k*bits, k*bits+bits) of the row
 *                                     (bits = 4: even k in the low nibble)
 * scales  fp16 [N, K/group]           output (group index fastest)
 * zeros   fp16 [N, K/group]           output
 * N >= 0 (N == 0 is a no-op), K >= 1, group >= 1, K % group == 0.
 * bits in 2..8 (wq_gemm reads 4 and 8); group % 8 == 0, so every 8 codes
 * fill exactly `bits` bytes; codes 16-byte aligned; scales/zeros 2-byte
 * aligned.
 */
wq_status wq_quantize_pack(const void* W, int64_t N, int64_t K, int32_t group,
                           int32_t bits, void* codes, void* scales, void* zeros,
                           void* stream);

/* Scale scheme for wq_quantize_pack_ex. */
typedef enum {
    WQ_SCHEME_ASYM = 0,       /* min/max per group, integer zero point (wq_quantize_pack) */
    WQ_SCHEME_SYM = 1,        /* symmetric, absolute maximum per group */
    WQ_SCHEME_SYM_TENSOR = 2, /* symmetric, one absolute maximum for the whole matrix */
    WQ_SCHEME_NF4 = 3,        /* NF4 levels, absolute maximum per group (bits = 4) */
    WQ_SCHEME_OFFSET = 4      /* min/max per group, float minimum kept as the offset */
} wq_scheme;

/*
 * wq_quantize_pack with a choice of scale scheme.  The symmetric schemes
 * follow "Quantization & inference optimisation", sections "Quantize a matrix
 * by hand" and "Per-channel, and what it buys" (and the 2-bit levels of
 * "Serving many users at once", "Quantization: rounding the weights"):
 *     A = max |x| over the group (WQ_SCHEME_SYM; group = K gives one scale
 *         per output channel) or over all of W (WQ_SCHEME_SYM_TENSOR)
 *     s = fp16(round-half-even(A / (2^(bits-1) - 1)))  (1.0 if that is 0)
 *     q = clamp(round-half-even(x / s), -2^(bits-1), 2^(bits-1) - 1)
 * stored in the layout of wq_quantize_pack as the code q + 2^(bits-1) with
 * zero point 2^(bits-1) in every group header (and, per tensor, the one scale
 * repeated in every group header), so wq_gemm multiplies by q * s unchanged.
 * Arguments, layout and errors as wq_quantize_pack; an unknown scheme is
 * WQ_ERR_INVALID_ARG.  WQ_SCHEME_SYM_TENSOR enqueues two small reduction
 * launches before the quantize launch and needs a workspace
 * (wq_quantize_workspace_size; 4100 bytes), the other schemes none.
 *
 * WQ_SCHEME_NF4 ("Gör inference billig: KV cache, batching och
 * kvantisering", the NF4 paragraph; bits must be 4, else
 * WQ_ERR_UNSUPPORTED): sixteen fixed levels, level i = the standard normal
 * quantile at (i + 1/2)/16 normalised to [-1, 1] and rounded to fp16;
 * s = the group's largest |w| (1.0 for an all-zero group); code = the level
 * nearest to w / s, decided exactly, ties to the lower code.  Codes two per
 * byte as for 4-bit integers; `zeros` is written with +0.0 (NF4 has no zero
 * point).  Multiply with wq_gemm_nf4, not wq_gemm.
 *
 * WQ_SCHEME_OFFSET ("Quantization & inference optimisation", section
 * "Quantization", the affine per-group code): s as for WQ_SCHEME_ASYM, the
 * group's minimum m written to `zeros` (fp16, exact), codes
 * round-half-even((x - m) / s) clamped to [0, 2^bits - 1], decided exactly;
 * x_hat = q * s + m.  Any bits 2..8.  Multiply with wq_gemm_offset.
 */
wq_status wq_quantize_pack_ex(const void* W, int64_t N, int64_t K, int32_t group,
                              int32_t bits, int32_t scheme, void* codes, void* scales,
                              void* zeros, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Workspace bytes wq_quantize_pack_ex needs for these arguments (0 unless
 * scheme is WQ_SCHEME_SYM_TENSOR); errors as wq_quantize_pack_ex's shape
 * checks, *bytes = 0 then. */
wq_status wq_quantize_workspace_size(int64_t N, int64_t K, int32_t group, int32_t bits,
                                     int32_t scheme, size_t* bytes);

/*
 * Decode-step product with in-register dequantization ("Quantization &
 * inference optimisation", "Bandwidth, not compute" and "Quantization"):
 *     Y[b, n] = sum_k X[b, k] * (q[n, k] - zeros[n, k/group]) * scales[n, k/group]
 * accumulated in fp32 and rounded once to fp16.
 *
 * X       fp16 [B, K]                 16-byte aligned
 * codes, scales, zeros                as produced by wq_quantize_pack
 *                                     (codes 16-byte aligned)
 * Y       fp16 [B, N]                 output, 2-byte aligned
 * B >= 0, N >= 0 (either 0 is a no-op), K >= 1, K % group == 0.
 * bits 4: K % 32 == 0 and group % 32 == 0.  bits 8: K % 16 == 0 and
 * group % 16 == 0.  The MFMA path additionally needs group % 128 (bits 4) or
 * group % 64 (bits 8); WQ_PATH_AUTO falls back to the GEMV path otherwise.
 * bits 2 and 3 (the bit-stream layout of wq_quantize_pack; "Quantization &
 * inference optimisation", "Quantization", prints their errors next to 4 and
 * 8 bits): group % 32 == 0, K % 64 == 0 (bits 2) or K % 128 == 0 (bits 3),
 * K <= 32768.  They run on the GEMV path (the codes streamed once per four
 * batch rows), except that from B = 2 to 32, on matrices of at least 1.8
 * 16-row tiles per compute unit with group 128 and K = 2048, 4096 or 8192
 * (and X and both header arrays 16-byte aligned), the MFMA path takes them
 * (exact-integer operands,
 * header applied per group in fp32); WQ_PATH_MFMA outside those shapes is
 * WQ_ERR_UNSUPPORTED.  bits 1, 5, 6 and 7 are WQ_ERR_UNSUPPORTED.
 * Results are deterministic: no atomics, fixed reduction order.
 * wq_gemm takes no workspace: it runs plans that need none (the matrix-core
 * kernels without K splits).  wq_gemm_ex with a workspace is faster where
 * splitting K pays (few rows, or X too large for one block's LDS).
 */
wq_status wq_gemm(const void* X, const void* codes, const void* scales,
                  const void* zeros, void* Y, int64_t B, int64_t K, int64_t N,
                  int32_t group, int32_t bits, void* stream);

/* wq_gemm with an explicit kernel family (for benchmarks and parity tests of
 * each path) and a workspace (see the conventions above; size from
 * wq_gemm_workspace_size with the same shape and path).  Returns
 * WQ_ERR_UNSUPPORTED if the forced path cannot take the shape. */
wq_status wq_gemm_ex(const void* X, const void* codes, const void* scales,
                     const void* zeros, void* Y, int64_t B, int64_t K, int64_t N,
                     int32_t group, int32_t bits, int32_t path, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * wq_gemm_ex without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  It runs the plan
 * wq_gemm_ex runs with a workspace (same kernels, bit-identical results), and
 * takes the scratch that plan needs from a static device array of 16 MiB
 * (16777216 bytes), one per GPU, held from the first call on that GPU until
 * the process ends.  A call whose plan needs more (wq_gemm_workspace_size
 * above 16 MiB, e.g. B = 64 on a 28672 x 8192 matrix) returns
 * WQ_ERR_UNSUPPORTED before any launch.  Every call on one GPU shares that
 * GPU's array: calls that may overlap on one GPU (different streams, or
 * threads enqueuing concurrently) race on it and must be serialized by the
 * caller.  Nothing in the array needs to start at any particular value.
 * Arguments, validation and errors otherwise as wq_gemm_ex.
 */
wq_status wq_gemm_static(const void* X, const void* codes, const void* scales,
                         const void* zeros, void* Y, int64_t B, int64_t K, int64_t N,
                         int32_t group, int32_t bits, int32_t path, void* stream);

/* Workspace bytes wq_gemm_ex needs for this shape and path on the current
 * device (0: none).  Errors as wq_gemm_ex's shape checks (no pointers are
 * involved); *bytes = 0 then. */
wq_status wq_gemm_workspace_size(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits,
                                 int32_t path, size_t* bytes);

/*
 * Product with NF4 weights (codes and scales from wq_quantize_pack_ex with
 * WQ_SCHEME_NF4):
 *     Y[b, n] = sum_k X[b, k] * level[q[n, k]] * scales[n, k/group]
 * fp32 accumulation, Y rounded once to fp16.  X fp16 [B, K] (16-byte
 * aligned), codes u8 [N, K/2] (16-byte aligned), scales fp16 [N, K/group],
 * Y fp16 [B, N].  K % 32 == 0, group % 32 == 0, K <= 16384 (else
 * WQ_ERR_UNSUPPORTED); B or N == 0 is a no-op.  From B = 2 to 32 with group
 * 64, K = 2048, 4096 or 8192, at least 1.8 16-row tiles per compute unit and
 * 16-byte aligned `scales`: a matrix-core kernel (each code byte becomes a
 * pair of fp16 levels through an LDS table, times the scale in fp16);
 * otherwise a VALU kernel with the same table, any B (codes streamed once per
 * four batch rows).
 */
wq_status wq_gemm_nf4(const void* X, const void* codes, const void* scales, void* Y, int64_t B,
                      int64_t K, int64_t N, int32_t group, void* stream);

/*
 * Product with float-offset weights (codes, scales and minima from
 * wq_quantize_pack_ex with WQ_SCHEME_OFFSET; "Quantization & inference
 * optimisation", section "Quantization"):
 *     Y[b, n] = sum_k X[b, k] * (q[n, k] * scales[n, k/group] + mins[n, k/group])
 * fp32 accumulation, Y rounded once to fp16.  bits 2, 3, 4 or 8 (others
 * WQ_ERR_UNSUPPORTED); group % 32 == 0; K % 64 (bits 2), % 128 (bits 3) or
 * % 32 (bits 4, 8); K <= 16384 (32768 at bits 3).  Layout and alignment as
 * wq_gemm, `mins` in place of `zeros`.  From B = 2 to 32 at bits 2, 3 or 4,
 * group 128, K = 2048, 4096 or 8192, at least 1.8 16-row tiles per compute
 * unit and 16-byte aligned `scales` and `mins`: a matrix-core kernel
 * (exact-integer operands; per group
 * s * sum q x + m * sum x in fp32); otherwise the VALU bit-stream kernel, any
 * B (codes streamed once per four batch rows).
 */
wq_status wq_gemm_offset(const void* X, const void* codes, const void* scales, const void* mins,
                         void* Y, int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits,
                         void* stream);

/* The arguments of one wq_gemm call, for wq_gemm_grouped. */
typedef struct wq_gemm_item {
    const void* X;
    const void* codes;
    const void* scales;
    const void* zeros;
    void* Y;
    int64_t B, K, N;
    int32_t group, bits;
} wq_gemm_item;

/*
 * Several products of a decode step (every weight matrix of a layer, say)
 * enqueued together; each item computes what wq_gemm (WQ_PATH_AUTO) computes
 * for it.  The decode step reads each matrix once per token ("Quantization &
 * inference optimisation", "Bandwidth, not compute"); small matrices then
 * spend much of their time in launch ramp, X staging and split-K reduction,
 * which grouping shares out.  Items with 3 <= B <= 32 that the matrix-core
 * path takes and that share B and bits run on the X-resident kernel, up to
 * eight products per launch (one launch per group-header layout), plus one
 * reduction launch; every other item runs as its own wq_gemm, in item order.  A launch of
 * several products splits K into fewer slices than single calls do, so their
 * fp32 sums may differ from wq_gemm's in the last bits (same tolerance);
 * results are deterministic for a given list of items.
 *
 * items   host array of `count` items, read during the call and not kept
 * count   >= 0 (0 is a no-op)
 * Every item is validated as by wq_gemm before anything is enqueued; the
 * first invalid item's status is returned (wq_last_error names the item) and
 * nothing runs.  An item's Y must not overlap any item's inputs or another
 * item's Y.  The launches of a call run one after another and share the
 * workspace (wq_gemm_grouped_workspace_size); without one, products whose X
 * needs several K-slices run alone, as wq_gemm.
 */
wq_status wq_gemm_grouped(const wq_gemm_item* items, int32_t count, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Workspace bytes wq_gemm_grouped needs for this item list on the current
 * device (0: none).  Items are validated as by wq_gemm_grouped. */
wq_status wq_gemm_grouped_workspace_size(const wq_gemm_item* items, int32_t count, size_t* bytes);

/* Largest batch that WQ_PATH_AUTO sends to the GEMV path when the MFMA path
 * can take the shape. */
int32_t wq_gemv_max_batch(void);

/*
 * Reconstruction of the weights from codes and headers, written out as fp32
 * (a test aid, not the hot path: the products reconstruct in registers).
 * "Quantization & inference optimisation", "Quantization": the integer and
 * the group's endpoints give back an approximate float.
 *     schemes 0-2:  W[n, k] = (q - zeros[g]) * scales[g]
 *     NF4 (3):      W[n, k] = level[q] * scales[g]        (bits 4; zeros unused)
 *     offset (4):   W[n, k] = q * scales[g] + zeros[g]    (zeros holds the minimum)
 * with g = n * (K / group) + k / group, each value rounded once to fp32 (the
 * first two forms are exact).
 *
 * codes, scales, zeros   as written by wq_quantize_pack_ex with the same
 *                        group, bits and scheme (caller-owned device memory)
 * W       fp32 [N, K]    output, 16-byte aligned
 * N >= 0 (0 is a no-op), K >= 1, K % group == 0, group % 8 == 0, bits 2..8.
 * Errors: WQ_ERR_INVALID_ARG (shape, unknown scheme, null pointer),
 * WQ_ERR_UNSUPPORTED (bits outside 2..8, NF4 with bits != 4, group not a
 * multiple of 8), WQ_ERR_MISALIGNED, WQ_ERR_HIP.  Enqueued on `stream`.
 */
wq_status wq_dequantize(const void* codes, const void* scales, const void* zeros, int64_t N,
                        int64_t K, int32_t group, int32_t bits, int32_t scheme, void* W,
                        void* stream);

/* Bytes of the codes array: N * K * bits / 8 (0 on invalid input). */
size_t wq_codes_bytes(int64_t N, int64_t K, int32_t bits);

/* Number of groups: N * K / group, the element count of scales and of zeros
 * (-1 on invalid input). */
int64_t wq_num_groups(int64_t N, int64_t K, int32_t group);

/*
 * int4 KV cache for decode attention ("What actually happens when you
 * quantize a KV cache": §2 the decode step, §3-§4 the codec, §5 the byte
 * count, §7 "axis choice").  Head dimension 128; tokens are cached in blocks
 * of 128.  Per head, for each block:
 *   kcodes   u8   [heads][max_blocks][128 tokens][64]   K codes, token-major:
 *                 byte i of a token row holds channels 2i (low nibble), 2i+1
 *   kscales, kzeros fp16 [heads][max_blocks][128]       per channel of a block
 *                 (one K group = one channel over the block's 128 tokens)
 *   vcodes   u8   [heads][max_blocks][128 channels][64] V codes, channel-major:
 *                 byte i of a channel row holds tokens 2i (low nibble), 2i+1
 *   vscales, vzeros fp16 [heads][max_blocks * 128]      per token (one V group
 *                 = one token's 128 values)
 *   kres, vres fp16 [heads][128][128]                    the newest tokens that
 *                 do not fill a block, token-major, in fp16
 * A head holding L tokens has its first L / 128 blocks quantized and the
 * remaining L % 128 tokens in rows 0.. of kres/vres.  The codec is the one of
 * wq_quantize_pack (asymmetric, 4 bits, round half to even, fp16 headers).
 * 136 bytes per token per head (the page's 136 KiB per token over 32 layers of
 * 32 heads).  The caller allocates and owns every buffer; code buffers and
 * kres/vres 16-byte aligned, header arrays 2-byte aligned.
 */
typedef struct wq_kv_cache {
    void* kcodes;
    void* kscales;
    void* kzeros;
    void* vcodes;
    void* vscales;
    void* vzeros;
    void* kres;
    void* vres;
    int64_t heads;
    int64_t max_blocks;
} wq_kv_cache;

/*
 * Quantize-on-append ("cheap enough to run inline as tokens are generated",
 * §4): K and V, fp16 [heads][128 tokens][128] token-major (16-byte aligned),
 * become block `block` (0 <= block < max_blocks) of every head's cache.  K is
 * grouped per channel over the 128 tokens, V per token; codes and headers are
 * bit-identical to the oracle's.  Typically called when a head's residual
 * window fills, with K = kres and V = vres.  heads == 0 is a no-op.
 */
wq_status wq_kv_quantize_block(const void* K, const void* V, const wq_kv_cache* cache,
                               int64_t block, void* stream);

/*
 * Decode attention of one new token per head:
 *     out[h] = softmax(K_h q_h / sqrt(128)) V_h
 * over the cached tokens of head h: its quantized blocks (dequantized as
 * (q - z) * s in registers) followed by its residual fp16 tokens.
 * q, out  fp16 [heads][128] (q 2-byte aligned, out 2-byte aligned)
 * lens    int32 [heads], DEVICE memory: tokens held by each head; values are
 *         clamped to [0, max_blocks * 128 + 127] (a head with 0 tokens gives 0)
 * fp32 scores, softmax and accumulation; with a workspace
 * (wq_kv_workspace_size) the context is split over several workgroups per
 * head when there are few heads, without one each head is one workgroup.
 * Tolerance against the float64 oracle: the product tolerance
 * (max|d| <= 1e-2 max|ref|, rel L2 <= 1e-3).
 */
wq_status wq_kv_attention(const void* q, const wq_kv_cache* cache, const int32_t* lens,
                          void* out, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes wq_kv_attention needs for this cache on the current device
 * (only heads and max_blocks are read; 0: none). */
wq_status wq_kv_workspace_size(const wq_kv_cache* cache, size_t* bytes);

/* Static description of a status code. */
const char* wq_status_string(wq_status s);

/* Description of the calling thread's last failed call ("" if none). */
const char* wq_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int32_t wq_version(void);

#define WQ_VERSION 200

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */
