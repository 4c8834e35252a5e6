// C ABI of the weight-only group-quantized decode GEMM (declared in include/wq.h).
// Validation happens here, synchronously, before anything is enqueued; the
// kernels are then launched on the caller's stream without synchronizing.
// The library allocates no device memory: scratch (split partials, the
// per-tensor maximum) comes from a caller-owned workspace sized by the
// wq_*_workspace_size queries, and calls without one take plans that need
// none.
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <new>

#include "wq.h"
#include "wq_launch.h"

namespace {

thread_local char g_last_error[256] = "";

wq_status fail(wq_status st, const char* fmt, long long a = 0, long long b = 0) {
    snprintf(g_last_error, sizeof(g_last_error), fmt, a, b);
    return st;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Compute units of the current device, cached per device (the one lazily
// cached device property).
int num_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
            v = 256;
        cached[dev] = v;
    }
    return cached[dev];
}

wq_status check_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return WQ_OK;
    snprintf(g_last_error, sizeof(g_last_error), "%s: %s", what, hipGetErrorString(e));
    return WQ_ERR_HIP;
}

// A caller's workspace against the bytes the call needs.  Null with size 0
// means none: the call then takes a plan that needs none.  Otherwise it must
// be 16-byte aligned and hold at least `need` bytes.
wq_status check_workspace(const char* who, const void* ws, size_t ws_bytes, size_t need) {
    if (!ws) {
        if (ws_bytes == 0) return WQ_OK;
        snprintf(g_last_error, sizeof(g_last_error), "%s: null workspace with workspace_bytes=%llu", who,
                 (unsigned long long)ws_bytes);
        return WQ_ERR_INVALID_ARG;
    }
    if (!aligned(ws, 16)) {
        snprintf(g_last_error, sizeof(g_last_error), "%s: workspace needs 16-byte alignment", who);
        return WQ_ERR_MISALIGNED;
    }
    if (ws_bytes < need) {
        snprintf(g_last_error, sizeof(g_last_error), "%s: workspace of %llu bytes, the call needs %llu", who,
                 (unsigned long long)ws_bytes, (unsigned long long)need);
        return WQ_ERR_INVALID_ARG;
    }
    return WQ_OK;
}

// Runs fn(paths) with a host array of count path slots.
template <class F>
wq_status with_paths(int32_t count, F fn) {
    int32_t paths_small[64];
    int32_t* paths = count <= 64 ? paths_small : new (std::nothrow) int32_t[count];
    if (!paths) return fail(WQ_ERR_INVALID_ARG, "wq_gemm_grouped: out of host memory (count=%lld)", count);
    const wq_status st = fn(paths);
    if (paths != paths_small) delete[] paths;
    return st;
}

}  // namespace

// ---- the static scratch of wq_gemm_static -------------------------------------
// For callers that cannot allocate (code under graph capture, tight serving
// loops, harnesses that forbid it): split partials live in this fixed device
// array instead of a caller workspace.  Each GPU the library runs on holds its
// own copy until the process ends.  In host code `scratch` names a host-side
// stand-in, so its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is
// ever passed to kernels.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
wq_status static_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return check_hip(e, "wq_gemm_static: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(WQ_ERR_UNSUPPORTED, "wq_gemm_static: device %lld beyond the %lld the library tracks", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return check_hip(e, "wq_gemm_static: hipGetSymbolAddress(scratch)");
        if (!p) return fail(WQ_ERR_HIP, "wq_gemm_static: null address for the static scratch");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return WQ_OK;
}

}  // namespace

extern "C" {

int32_t wq_version(void) { return WQ_VERSION; }

const char* wq_status_string(wq_status s) {
    switch (s) {
        case WQ_OK: return "ok";
        case WQ_ERR_INVALID_ARG: return "invalid argument";
        case WQ_ERR_UNSUPPORTED: return "unsupported shape or layout";
        case WQ_ERR_MISALIGNED: return "misaligned pointer or stride";
        case WQ_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* wq_last_error(void) { return g_last_error; }

size_t wq_codes_bytes(int64_t N, int64_t K, int32_t bits) {
    if (N < 0 || K < 0 || bits < 1 || bits > 8 || (K * bits) % 8 != 0) return 0;
    return (size_t)(N * K * bits / 8);
}

int64_t wq_num_groups(int64_t N, int64_t K, int32_t group) {
    if (N < 0 || K < 0 || group < 1 || K % group != 0) return -1;
    return N * (K / group);
}

// Measured crossover on MI355X: the GEMV path wins at B <= 2, the matrix-core
// kernels from B = 3 on.
int32_t wq_gemv_max_batch(void) { return 1; }

// ---- quantize/pack -----------------------------------------------------------

// Shape and scheme checks of a quantize call (no pointers).
static wq_status check_quant_shape(int64_t N, int64_t K, int32_t group, int32_t bits, int32_t scheme) {
    if (N < 0 || K < 1 || group < 1)
        return fail(WQ_ERR_INVALID_ARG, "wq_quantize_pack: need N >= 0, K >= 1, group >= 1 (N=%lld K=%lld)", N, K);
    if (K % group != 0)
        return fail(WQ_ERR_INVALID_ARG, "wq_quantize_pack: K=%lld is not a multiple of group=%lld", K, group);
    if (bits < 1 || bits > 8)
        return fail(WQ_ERR_INVALID_ARG, "wq_quantize_pack: bits=%lld out of range", bits);
    if (scheme < WQ_SCHEME_ASYM || scheme > WQ_SCHEME_OFFSET)
        return fail(WQ_ERR_INVALID_ARG, "wq_quantize_pack: unknown scheme %lld", scheme);
    if (scheme == WQ_SCHEME_NF4 && bits != 4)
        return fail(WQ_ERR_UNSUPPORTED, "wq_quantize_pack: NF4 codes are 4 bits (got %lld)", bits);
    if (bits < 2)
        return fail(WQ_ERR_UNSUPPORTED, "wq_quantize_pack: the codec takes bits 2..8 (got %lld)", bits);
    if (group % 8 != 0)
        return fail(WQ_ERR_UNSUPPORTED, "wq_quantize_pack: group=%lld must be a multiple of 8", group);
    return WQ_OK;
}

wq_status wq_quantize_workspace_size(int64_t N, int64_t K, int32_t group, int32_t bits, int32_t scheme,
                                     size_t* bytes) {
    g_last_error[0] = '\0';
    if (!bytes) return fail(WQ_ERR_INVALID_ARG, "wq_quantize_workspace_size: null bytes");
    *bytes = 0;
    const wq_status st = check_quant_shape(N, K, group, bits, scheme);
    if (st != WQ_OK) return st;
    *bytes = N == 0 ? 0 : wq::quantize_scratch_bytes(scheme);
    return WQ_OK;
}

wq_status wq_quantize_pack_ex(const void* W, int64_t N, int64_t K, int32_t group, int32_t bits,
                              int32_t scheme, void* codes, void* scales, void* zeros, void* workspace,
                              size_t workspace_bytes, void* stream) {
    g_last_error[0] = '\0';
    wq_status st = check_quant_shape(N, K, group, bits, scheme);
    if (st != WQ_OK) return st;
    const size_t need = wq::quantize_scratch_bytes(scheme);
    st = check_workspace("wq_quantize_pack", workspace, workspace_bytes, need);
    if (st != WQ_OK) return st;
    if (N == 0) return WQ_OK;
    if (!W || !codes || !scales || !zeros)
        return fail(WQ_ERR_INVALID_ARG, "wq_quantize_pack: null pointer");
    if (!aligned(W, 16) || !aligned(codes, 16) || !aligned(scales, 2) || !aligned(zeros, 2))
        return fail(WQ_ERR_MISALIGNED, "wq_quantize_pack: W and codes need 16-byte alignment");
    if (need > 0 && !workspace)
        return fail(WQ_ERR_INVALID_ARG, "wq_quantize_pack: the per-tensor scheme needs a workspace of %lld bytes",
                    (long long)need);
    return check_hip(wq::launch_quantize_pack(W, N, K, group, bits, scheme, codes, scales, zeros, workspace,
                                              static_cast<hipStream_t>(stream)),
                     "wq_quantize_pack launch");
}

wq_status wq_quantize_pack(const void* W, int64_t N, int64_t K, int32_t group, int32_t bits,
                           void* codes, void* scales, void* zeros, void* stream) {
    return wq_quantize_pack_ex(W, N, K, group, bits, WQ_SCHEME_ASYM, codes, scales, zeros, nullptr, 0,
                               stream);
}

wq_status wq_dequantize(const void* codes, const void* scales, const void* zeros, int64_t N,
                        int64_t K, int32_t group, int32_t bits, int32_t scheme, void* W,
                        void* stream) {
    g_last_error[0] = '\0';
    if (N < 0 || K < 1 || group < 1)
        return fail(WQ_ERR_INVALID_ARG, "wq_dequantize: need N >= 0, K >= 1, group >= 1 (N=%lld K=%lld)", N, K);
    if (K % group != 0)
        return fail(WQ_ERR_INVALID_ARG, "wq_dequantize: K=%lld is not a multiple of group=%lld", K, group);
    if (scheme < WQ_SCHEME_ASYM || scheme > WQ_SCHEME_OFFSET)
        return fail(WQ_ERR_INVALID_ARG, "wq_dequantize: unknown scheme %lld", scheme);
    if (bits < 2 || bits > 8)
        return fail(WQ_ERR_UNSUPPORTED, "wq_dequantize: the codec takes bits 2..8 (got %lld)", bits);
    if (scheme == WQ_SCHEME_NF4 && bits != 4)
        return fail(WQ_ERR_UNSUPPORTED, "wq_dequantize: NF4 codes are 4 bits (got %lld)", bits);
    if (group % 8 != 0)
        return fail(WQ_ERR_UNSUPPORTED, "wq_dequantize: group=%lld must be a multiple of 8", group);
    if (N == 0) return WQ_OK;
    if (!codes || !scales || !zeros || !W) return fail(WQ_ERR_INVALID_ARG, "wq_dequantize: null pointer");
    if (!aligned(W, 16) || !aligned(scales, 2) || !aligned(zeros, 2))
        return fail(WQ_ERR_MISALIGNED, "wq_dequantize: W needs 16-byte alignment");
    return check_hip(wq::launch_dequantize(codes, scales, zeros, W, N, K, group, bits, scheme,
                                           static_cast<hipStream_t>(stream)),
                     "wq_dequantize launch");
}

// ---- products ----------------------------------------------------------------

// Validates the shape of one product and picks its kernel family (path on
// return); checks no pointer.  A no-op product (B == 0 or N == 0) returns
// WQ_OK with path = -1.
// The header pointers (null for a size query: taken as aligned) decide
// between kernels that need aligned header arrays and those that do not.
static wq_status check_gemm_shape(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits,
                                  const void* scales, const void* zeros, int32_t& path) {
    if (B < 0 || N < 0 || K < 1 || group < 1)
        return fail(WQ_ERR_INVALID_ARG, "wq_gemm: need B >= 0, N >= 0, K >= 1, group >= 1 (B=%lld K=%lld)", B, K);
    if (K % group != 0)
        return fail(WQ_ERR_INVALID_ARG, "wq_gemm: K=%lld is not a multiple of group=%lld", K, group);
    if (bits < 1 || bits > 8)
        return fail(WQ_ERR_INVALID_ARG, "wq_gemm: bits=%lld out of range", bits);
    if (bits != 2 && bits != 3 && bits != 4 && bits != 8)
        return fail(WQ_ERR_UNSUPPORTED, "wq_gemm: bits=%lld (GPU kernels take 2, 3, 4 or 8)", bits);
    if (path < WQ_PATH_AUTO || path > WQ_PATH_MFMA)
        return fail(WQ_ERR_INVALID_ARG, "wq_gemm: unknown path %lld", path);
    const bool low = bits == 2 || bits == 3;
    if (low) {
        // 32-code chunks inside one group; rows of whole 16-byte loads.
        const int unit = bits == 2 ? 64 : 128;
        if (K % unit != 0 || group % 32 != 0)
            return fail(WQ_ERR_UNSUPPORTED, "wq_gemm: bits 2/3 need K %% (64 or 128) == 0 and group %% 32 == 0 "
                        "(K=%lld group=%lld)", K, group);
    } else {
        const int vals = 128 / bits;  // codes per 16-byte chunk
        if (K % vals != 0 || group % vals != 0)
            return fail(WQ_ERR_UNSUPPORTED, "wq_gemm: K=%lld and group=%lld must be multiples of the 16-byte chunk",
                        K, group);
    }
    if (low && !wq::gemv_lowbit_supports(K, group, bits))
        return fail(WQ_ERR_UNSUPPORTED, "wq_gemm: the 2/3-bit GEMV does not take K=%lld at bits=%lld", K, bits);
    if (B == 0 || N == 0) {
        path = -1;
        return WQ_OK;
    }
    if (low) {
        // The K-split-wave matrix-core kernel where it takes the shape and
        // the header arrays (X's alignment is checked with the pointers),
        // the bit-stream GEMV otherwise.
        const bool kw = wq::kw_takes(B, K, N, group, bits, false, nullptr, scales, zeros, num_cus());
        if (path == WQ_PATH_MFMA && !kw)
            return fail(WQ_ERR_UNSUPPORTED, "wq_gemm: bits=%lld takes the MFMA path only for 2 <= B <= 32, "
                        "group 128, K = 2048, 4096 or 8192, at least 1.8 16-row tiles per compute unit and "
                        "16-byte aligned header arrays", bits);
        path = (path == WQ_PATH_GEMV || !kw) ? WQ_PATH_GEMV : WQ_PATH_MFMA;
        return WQ_OK;
    }
    const bool gemv_ok = wq::gemv_supports(K, bits);
    const bool mfma_ok = wq::mfma_path_takes(B, K, N, group, bits, scales, zeros);
    int use = path;
    if (use == WQ_PATH_AUTO) {
        if (mfma_ok && (B > wq_gemv_max_batch() || !gemv_ok)) use = WQ_PATH_MFMA;
        else use = WQ_PATH_GEMV;
    }
    if (use == WQ_PATH_GEMV && !gemv_ok)
        return fail(WQ_ERR_UNSUPPORTED, "wq_gemm: GEMV path does not take K=%lld at bits=%lld", K, bits);
    if (use == WQ_PATH_MFMA && !mfma_ok)
        return fail(WQ_ERR_UNSUPPORTED,
                    "wq_gemm: MFMA path needs group %% %lld == 0 (group=%lld), or B <= 4 with aligned header arrays",
                    bits == 4 ? 128 : 64, group);
    path = use;
    return WQ_OK;
}

// Shape, then pointers.
static wq_status check_gemm(const void* X, const void* codes, const void* scales,
                            const void* zeros, const void* Y, int64_t B, int64_t K, int64_t N,
                            int32_t group, int32_t bits, int32_t& path) {
    const wq_status st = check_gemm_shape(B, K, N, group, bits, scales, zeros, path);
    if (st != WQ_OK || path < 0) return st;
    if (!X || !codes || !scales || !zeros || !Y)
        return fail(WQ_ERR_INVALID_ARG, "wq_gemm: null pointer");
    if (!aligned(X, 16) || !aligned(codes, 16) || !aligned(scales, 2) || !aligned(zeros, 2) || !aligned(Y, 2))
        return fail(WQ_ERR_MISALIGNED, "wq_gemm: X and codes need 16-byte alignment");
    return WQ_OK;
}

// Sizes (ws.need set) or launches one validated product on its kernel family.
static wq_status run_gemm(const void* X, const void* codes, const void* scales, const void* zeros,
                          void* Y, int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits,
                          int32_t use, const wq::Scratch& ws, hipStream_t st) {
    if (use == WQ_PATH_MFMA)
        return check_hip(wq::launch_gemm_mfma(X, codes, scales, zeros, Y, B, K, N, group, bits,
                                              num_cus(), ws, st),
                         "wq_gemm (mfma) launch");
    if (ws.sizing()) return WQ_OK;   // the GEMVs use no scratch
    if (bits == 2 || bits == 3)
        return check_hip(wq::launch_gemv_lowbit(X, codes, scales, zeros, Y, B, K, N, group, bits, 0,
                                                num_cus(), st),
                         "wq_gemm (2/3-bit gemv) launch");
    return check_hip(wq::launch_gemv(X, codes, scales, zeros, Y, B, K, N, group, bits, num_cus(), st),
                     "wq_gemm (gemv) launch");
}

wq_status wq_gemm_workspace_size(int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits,
                                 int32_t path, size_t* bytes) {
    g_last_error[0] = '\0';
    if (!bytes) return fail(WQ_ERR_INVALID_ARG, "wq_gemm_workspace_size: null bytes");
    *bytes = 0;
    int32_t use = path;
    const wq_status st = check_gemm_shape(B, K, N, group, bits, nullptr, nullptr, use);
    if (st != WQ_OK || use < 0) return st;
    size_t need = 0;
    wq::Scratch ws;
    ws.need = &need;
    // Sizing launches nothing; the pointers are never read.
    const wq_status s2 = run_gemm(nullptr, nullptr, nullptr, nullptr, nullptr, B, K, N, group, bits, use, ws,
                                  nullptr);
    if (s2 != WQ_OK) return s2;
    *bytes = need;
    return WQ_OK;
}

wq_status wq_gemm_ex(const void* X, const void* codes, const void* scales, const void* zeros,
                     void* Y, int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits,
                     int32_t path, void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error[0] = '\0';
    int32_t use = path;
    wq_status st = check_gemm(X, codes, scales, zeros, Y, B, K, N, group, bits, use);
    if (st != WQ_OK) return st;
    if (use < 0) return check_workspace("wq_gemm", workspace, workspace_bytes, 0);
    size_t need = 0;
    if (workspace) {
        wq::Scratch sz;
        sz.need = &need;
        st = run_gemm(X, codes, scales, zeros, Y, B, K, N, group, bits, use, sz, nullptr);
        if (st != WQ_OK) return st;
    }
    st = check_workspace("wq_gemm", workspace, workspace_bytes, need);
    if (st != WQ_OK) return st;
    wq::Scratch ws;
    ws.ptr = need > 0 ? workspace : nullptr;
    return run_gemm(X, codes, scales, zeros, Y, B, K, N, group, bits, use, ws, static_cast<hipStream_t>(stream));
}

wq_status wq_gemm(const void* X, const void* codes, const void* scales, const void* zeros,
                  void* Y, int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits,
                  void* stream) {
    return wq_gemm_ex(X, codes, scales, zeros, Y, B, K, N, group, bits, WQ_PATH_AUTO, nullptr, 0, stream);
}

wq_status wq_gemm_static(const void* X, const void* codes, const void* scales, const void* zeros,
                         void* Y, int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits,
                         int32_t path, void* stream) {
    g_last_error[0] = '\0';
    int32_t use = path;
    wq_status st = check_gemm(X, codes, scales, zeros, Y, B, K, N, group, bits, use);
    if (st != WQ_OK || use < 0) return st;
    // The plan wq_gemm_ex takes with a workspace, sized first.
    size_t need = 0;
    wq::Scratch sz;
    sz.need = &need;
    st = run_gemm(X, codes, scales, zeros, Y, B, K, N, group, bits, use, sz, nullptr);
    if (st != WQ_OK) return st;
    if (need > kStaticScratchBytes)
        return fail(WQ_ERR_UNSUPPORTED, "wq_gemm_static: the call needs %lld bytes of scratch, the static array "
                    "holds %lld (use wq_gemm_ex with a workspace)", (long long)need, (long long)kStaticScratchBytes);
    wq::Scratch ws;
    if (need > 0) {
        st = static_scratch(&ws.ptr);
        if (st != WQ_OK) return st;
    }
    return run_gemm(X, codes, scales, zeros, Y, B, K, N, group, bits, use, ws, static_cast<hipStream_t>(stream));
}

// Validates every item (paths[i] receives its kernel family, -1 for a no-op).
static wq_status check_items(const wq_gemm_item* items, int32_t count, int32_t* paths) {
    for (int32_t i = 0; i < count; ++i) {
        const wq_gemm_item& it = items[i];
        paths[i] = WQ_PATH_AUTO;
        const wq_status st = check_gemm(it.X, it.codes, it.scales, it.zeros, it.Y, it.B, it.K, it.N,
                                        it.group, it.bits, paths[i]);
        if (st != WQ_OK) {
            char msg[sizeof(g_last_error)];
            snprintf(msg, sizeof(msg), "%s", g_last_error);
            snprintf(g_last_error, sizeof(g_last_error), "item %d: %s", (int)i, msg);
            return st;
        }
    }
    return WQ_OK;
}

// Sizes or launches a validated item list: X-resident products of one
// (B, bits) go out together, in item order; every other product is one
// wq_gemm.  Launches follow one another on the stream, so they share the
// scratch (its size is the largest any of them needs).
static wq_status run_items(const wq_gemm_item* items, int32_t count, int32_t* paths, const wq::Scratch& ws,
                           hipStream_t st) {
    wq::XrProduct group_buf[64];
    for (int32_t i = 0; i < count; ++i) {
        const wq_gemm_item& it = items[i];
        if (paths[i] < 0) continue;
        const bool xr = paths[i] == WQ_PATH_MFMA && wq::xr_groupable(it.B, it.K, it.group, it.bits);
        if (!xr) {
            const wq_status s2 = run_gemm(it.X, it.codes, it.scales, it.zeros, it.Y, it.B, it.K, it.N,
                                          it.group, it.bits, paths[i], ws, st);
            if (s2 != WQ_OK) return s2;
            continue;
        }
        // Collect the not yet issued X-resident items of this (B, bits).
        int n = 0;
        for (int32_t j = i; j < count && n < 64; ++j) {
            const wq_gemm_item& o = items[j];
            if (paths[j] != WQ_PATH_MFMA || o.B != it.B || o.bits != it.bits ||
                !wq::xr_groupable(o.B, o.K, o.group, o.bits))
                continue;
            group_buf[n++] = wq::XrProduct{o.X, o.codes, o.scales, o.zeros, o.Y, o.K, o.N, o.group};
            paths[j] = -1;  // issued
        }
        // (A product left alone in a launch keeps the single-call kernel.)
        const wq_status s2 = check_hip(wq::launch_gemm_xr_many(group_buf, n, it.B, it.bits, num_cus(), ws, st),
                                       "wq_gemm_grouped (x-resident) launch");
        if (s2 != WQ_OK) return s2;
    }
    return WQ_OK;
}

wq_status wq_gemm_grouped_workspace_size(const wq_gemm_item* items, int32_t count, size_t* bytes) {
    g_last_error[0] = '\0';
    if (!bytes) return fail(WQ_ERR_INVALID_ARG, "wq_gemm_grouped_workspace_size: null bytes");
    *bytes = 0;
    if (count < 0 || (count > 0 && !items))
        return fail(WQ_ERR_INVALID_ARG, "wq_gemm_grouped: count=%lld, items=%lld (null)", count,
                    (long long)(items != nullptr));
    return with_paths(count, [&](int32_t* paths) {
        wq_status st = check_items(items, count, paths);
        if (st != WQ_OK) return st;
        size_t need = 0;
        wq::Scratch ws;
        ws.need = &need;
        st = run_items(items, count, paths, ws, nullptr);
        if (st == WQ_OK) *bytes = need;
        return st;
    });
}

wq_status wq_gemm_grouped(const wq_gemm_item* items, int32_t count, void* workspace, size_t workspace_bytes,
                          void* stream) {
    g_last_error[0] = '\0';
    if (count < 0 || (count > 0 && !items))
        return fail(WQ_ERR_INVALID_ARG, "wq_gemm_grouped: count=%lld, items=%lld (null)", count,
                    (long long)(items != nullptr));
    return with_paths(count, [&](int32_t* paths) {
        // Validate everything (and size the scratch) before enqueuing anything.
        wq_status st = check_items(items, count, paths);
        if (st != WQ_OK) return st;
        size_t need = 0;
        if (workspace) {
            // Sizing marks issued items in paths; run it on a copy.
            int32_t copy_small[64];
            int32_t* copy = count <= 64 ? copy_small : new (std::nothrow) int32_t[count];
            if (!copy) return fail(WQ_ERR_INVALID_ARG, "wq_gemm_grouped: out of host memory (count=%lld)", count);
            memcpy(copy, paths, sizeof(int32_t) * (size_t)count);
            wq::Scratch sz;
            sz.need = &need;
            st = run_items(items, count, copy, sz, nullptr);
            if (copy != copy_small) delete[] copy;
            if (st != WQ_OK) return st;
        }
        st = check_workspace("wq_gemm_grouped", workspace, workspace_bytes, need);
        if (st != WQ_OK) return st;
        wq::Scratch ws;
        ws.ptr = need > 0 ? workspace : nullptr;
        return run_items(items, count, paths, ws, static_cast<hipStream_t>(stream));
    });
}

// ---- KV cache ------------------------------------------------------------------

// Validates a cache descriptor (not its contents) and copies it into `a`;
// buffers are checked only when `buffers` is set.
static wq_status check_kv_cache(const wq_kv_cache* c, wq::KvCacheArgs& a, bool buffers = true) {
    if (!c) return fail(WQ_ERR_INVALID_ARG, "kv cache: null descriptor");
    if (c->heads < 0 || c->max_blocks < 1 || c->heads > ((int64_t)1 << 31) - 1 ||
        c->max_blocks > ((int64_t)1 << 24))
        return fail(WQ_ERR_INVALID_ARG, "kv cache: need heads >= 0, 1 <= max_blocks <= 2^24 (heads=%lld max_blocks=%lld)",
                    c->heads, c->max_blocks);
    if (buffers && c->heads > 0) {
        if (!c->kcodes || !c->kscales || !c->kzeros || !c->vcodes || !c->vscales || !c->vzeros || !c->kres ||
            !c->vres)
            return fail(WQ_ERR_INVALID_ARG, "kv cache: null buffer");
        if (!aligned(c->kcodes, 16) || !aligned(c->vcodes, 16) || !aligned(c->kres, 16) || !aligned(c->vres, 16) ||
            !aligned(c->kscales, 2) || !aligned(c->kzeros, 2) || !aligned(c->vscales, 2) || !aligned(c->vzeros, 2))
            return fail(WQ_ERR_MISALIGNED, "kv cache: code and residual buffers need 16-byte alignment");
    }
    a = wq::KvCacheArgs{c->kcodes, c->kscales, c->kzeros, c->vcodes, c->vscales, c->vzeros,
                        c->kres,   c->vres,    c->heads,  c->max_blocks};
    return WQ_OK;
}

wq_status wq_kv_quantize_block(const void* K, const void* V, const wq_kv_cache* cache, int64_t block,
                               void* stream) {
    g_last_error[0] = '\0';
    wq::KvCacheArgs a;
    const wq_status st = check_kv_cache(cache, a);
    if (st != WQ_OK) return st;
    if (block < 0 || block >= a.max_blocks)
        return fail(WQ_ERR_INVALID_ARG, "wq_kv_quantize_block: block=%lld outside [0, %lld)", block, a.max_blocks);
    if (a.heads == 0) return WQ_OK;
    if (!K || !V) return fail(WQ_ERR_INVALID_ARG, "wq_kv_quantize_block: null K or V");
    if (!aligned(K, 16) || !aligned(V, 16))
        return fail(WQ_ERR_MISALIGNED, "wq_kv_quantize_block: K and V need 16-byte alignment");
    return check_hip(wq::launch_kv_quantize(K, V, a, block, static_cast<hipStream_t>(stream)),
                     "wq_kv_quantize_block launch");
}

wq_status wq_kv_workspace_size(const wq_kv_cache* cache, size_t* bytes) {
    g_last_error[0] = '\0';
    if (!bytes) return fail(WQ_ERR_INVALID_ARG, "wq_kv_workspace_size: null bytes");
    *bytes = 0;
    wq::KvCacheArgs a;
    const wq_status st = check_kv_cache(cache, a, false);
    if (st != WQ_OK || a.heads == 0) return st;
    size_t need = 0;
    wq::Scratch ws;
    ws.need = &need;
    const wq_status s2 = check_hip(wq::launch_kv_attention(nullptr, a, nullptr, nullptr, num_cus(), ws, nullptr),
                                   "wq_kv_workspace_size");
    if (s2 == WQ_OK) *bytes = need;
    return s2;
}

wq_status wq_kv_attention(const void* q, const wq_kv_cache* cache, const int32_t* lens, void* out,
                          void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error[0] = '\0';
    wq::KvCacheArgs a;
    wq_status st = check_kv_cache(cache, a);
    if (st != WQ_OK) return st;
    size_t need = 0;
    if (workspace && a.heads > 0) {
        wq::Scratch sz;
        sz.need = &need;
        st = check_hip(wq::launch_kv_attention(nullptr, a, nullptr, nullptr, num_cus(), sz, nullptr),
                       "wq_kv_attention sizing");
        if (st != WQ_OK) return st;
    }
    st = check_workspace("wq_kv_attention", workspace, workspace_bytes, need);
    if (st != WQ_OK) return st;
    if (a.heads == 0) return WQ_OK;
    if (!q || !lens || !out) return fail(WQ_ERR_INVALID_ARG, "wq_kv_attention: null q, lens or out");
    if (!aligned(q, 2) || !aligned(out, 2) || !aligned(lens, 4))
        return fail(WQ_ERR_MISALIGNED, "wq_kv_attention: q/out need 2-byte and lens 4-byte alignment");
    wq::Scratch ws;
    ws.ptr = need > 0 ? workspace : nullptr;
    return check_hip(wq::launch_kv_attention(q, a, lens, out, num_cus(), ws, static_cast<hipStream_t>(stream)),
                     "wq_kv_attention launch");
}

// ---- other weight formats ------------------------------------------------------

wq_status wq_gemm_offset(const void* X, const void* codes, const void* scales, const void* mins,
                         void* Y, int64_t B, int64_t K, int64_t N, int32_t group, int32_t bits,
                         void* stream) {
    g_last_error[0] = '\0';
    if (B < 0 || N < 0 || K < 1 || group < 1)
        return fail(WQ_ERR_INVALID_ARG, "wq_gemm_offset: need B >= 0, N >= 0, K >= 1, group >= 1 (B=%lld K=%lld)", B, K);
    if (K % group != 0)
        return fail(WQ_ERR_INVALID_ARG, "wq_gemm_offset: K=%lld is not a multiple of group=%lld", K, group);
    if (bits < 1 || bits > 8) return fail(WQ_ERR_INVALID_ARG, "wq_gemm_offset: bits=%lld out of range", bits);
    if (!wq::gemv_lowbit_supports(K, group, bits))
        return fail(WQ_ERR_UNSUPPORTED, "wq_gemm_offset: bits 2, 3, 4 or 8, group %% 32 == 0 and K a multiple of "
                    "the load unit (K=%lld bits=%lld)", K, bits);
    if (B == 0 || N == 0) return WQ_OK;
    if (!X || !codes || !scales || !mins || !Y) return fail(WQ_ERR_INVALID_ARG, "wq_gemm_offset: null pointer");
    if (!aligned(X, 16) || !aligned(codes, 16) || !aligned(scales, 2) || !aligned(mins, 2) || !aligned(Y, 2))
        return fail(WQ_ERR_MISALIGNED, "wq_gemm_offset: X and codes need 16-byte alignment");
    if (wq::kw_takes(B, K, N, group, bits, true, X, scales, mins, num_cus()))
        return check_hip(wq::launch_gemm_kw(X, codes, scales, mins, Y, B, K, N, group, bits, true, num_cus(),
                                            static_cast<hipStream_t>(stream)),
                         "wq_gemm_offset (mfma) launch");
    return check_hip(wq::launch_gemv_lowbit(X, codes, scales, mins, Y, B, K, N, group, bits, 1, num_cus(),
                                            static_cast<hipStream_t>(stream)),
                     "wq_gemm_offset launch");
}

wq_status wq_gemm_nf4(const void* X, const void* codes, const void* scales, void* Y, int64_t B,
                      int64_t K, int64_t N, int32_t group, void* stream) {
    g_last_error[0] = '\0';
    if (B < 0 || N < 0 || K < 1 || group < 1)
        return fail(WQ_ERR_INVALID_ARG, "wq_gemm_nf4: need B >= 0, N >= 0, K >= 1, group >= 1 (B=%lld K=%lld)", B, K);
    if (K % group != 0)
        return fail(WQ_ERR_INVALID_ARG, "wq_gemm_nf4: K=%lld is not a multiple of group=%lld", K, group);
    if (!wq::gemv_nf4_supports(K, group))
        return fail(WQ_ERR_UNSUPPORTED, "wq_gemm_nf4: needs K %% 32 == 0, group %% 32 == 0, K <= 16384 (K=%lld group=%lld)",
                    K, group);
    if (B == 0 || N == 0) return WQ_OK;
    if (!X || !codes || !scales || !Y) return fail(WQ_ERR_INVALID_ARG, "wq_gemm_nf4: null pointer");
    if (!aligned(X, 16) || !aligned(codes, 16) || !aligned(scales, 2) || !aligned(Y, 2))
        return fail(WQ_ERR_MISALIGNED, "wq_gemm_nf4: X and codes need 16-byte alignment");
    if (wq::kw_nf4_takes(B, K, N, group, X, scales, num_cus()))
        return check_hip(wq::launch_gemm_kw_nf4(X, codes, scales, Y, B, K, N, group, num_cus(),
                                                static_cast<hipStream_t>(stream)),
                         "wq_gemm_nf4 (mfma) launch");
    return check_hip(wq::launch_gemv_nf4(X, codes, scales, Y, B, K, N, group, num_cus(),
                                         static_cast<hipStream_t>(stream)),
                     "wq_gemm_nf4 launch");
}

}  // extern "C"
