// Split-K workspace, cached per (device, stream).
//
// The matrix-core kernels split K when X does not fit in LDS or when a matrix
// has too few row tiles to keep every compute unit busy.  Their fp32 partials
// and per-tile arrival counters live in one device buffer per (device, stream)
// that is kept for reuse: a call on a stream only ever waits for earlier work
// on that stream, so reuse in stream order is race-free, and calls on
// different streams never share a buffer.  The buffer grows (stream-ordered
// free of the old one, allocation of a larger one) when a call needs more; its
// counter words are zeroed by a small kernel when it is created, and every
// kernel that uses them returns them to zero.
#include <mutex>
#include <unordered_map>

#include "wq_launch.h"

namespace wq {

namespace {

struct Entry {
    void* ptr = nullptr;
    size_t bytes = 0;    // whole buffer
    size_t cbytes = 0;   // counter area at its start (the partials follow)
};

std::mutex g_mu;
std::unordered_map<uint64_t, Entry> g_ws;

uint64_t key_of(int dev, hipStream_t s) {
    return (reinterpret_cast<uint64_t>(s) << 8) ^ (uint64_t)(unsigned)dev;
}

__global__ __launch_bounds__(256) void zero_words(uint32_t* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t workspace_get(hipStream_t stream, size_t counter_words, size_t part_bytes,
                         uint32_t** counters, float** part) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    // Counters first, partials 256-byte aligned after them.  The counter area
    // only ever grows together with a fresh, zeroed buffer, so counter words
    // never overlap old partials.
    const size_t need_c = (counter_words * sizeof(uint32_t) + 255) / 256 * 256;
    std::lock_guard<std::mutex> lock(g_mu);
    Entry& en = g_ws[key_of(dev, stream)];
    if (en.cbytes < need_c || en.bytes - en.cbytes < part_bytes) {
        if (en.ptr) {
            e = hipFreeAsync(en.ptr, stream);
            en = Entry{};
            if (e != hipSuccess) return e;
        }
        const size_t cb = need_c < (size_t)65536 ? (size_t)65536 : (need_c + need_c / 4 + 255) / 256 * 256;
        const size_t pb = part_bytes < (size_t)(1 << 20) ? (size_t)(1 << 20) : part_bytes + part_bytes / 4;
        const size_t bytes = cb + pb;
        void* p = nullptr;
        e = hipMallocAsync(&p, bytes, stream);
        if (e != hipSuccess) return e;
        // Every counter word of the new buffer starts at zero.
        const int64_t words = (int64_t)(cb / sizeof(uint32_t));
        zero_words<<<dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream>>>(
            static_cast<uint32_t*>(p), words);
        e = hipGetLastError();
        if (e != hipSuccess) {
            (void)hipFreeAsync(p, stream);
            return e;
        }
        en.ptr = p;
        en.bytes = bytes;
        en.cbytes = cb;
    }
    *counters = static_cast<uint32_t*>(en.ptr);
    *part = reinterpret_cast<float*>(static_cast<char*>(en.ptr) + en.cbytes);
    return hipSuccess;
}

}  // namespace wq
