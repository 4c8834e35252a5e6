/*
 * wq_probe.h — C ABI of the HBM read-stream probe (libwq_probe.so).
 *
 * A measurement aid, not part of the product: the decode product is bound by
 * the rate at which its packed weights stream from HBM ("Quantization &
 * inference optimisation", "Bandwidth, not compute"; "What actually happens
 * when you quantize a KV cache" §6, runtime = bytes / bandwidth), and this
 * load-only kernel measures that rate on the machine at hand, in the access
 * shapes the product kernels use, so their roofline fractions can be quoted
 * against it as well as against the vendor peak.
 */
#ifndef WQ_PROBE_H
#define WQ_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read a device matrix of `rows` rows of `row_bytes` bytes once with 128-bit
 * loads, and nothing else.  Each wave walks strips of 64 / lanes_per_row rows;
 * one load instruction reads lanes_per_row consecutive 16-byte vectors of each
 * row of its strip (64: 1 KB of one row; 4: 64 bytes of each of 16 rows).
 * Every wave keeps `depth` loads in flight; the grid has blocks_per_cu
 * 256-thread workgroups per compute unit and is persistent.  `order`: 0, a
 * strip's rows are adjacent and every walk starts at column 0; 1, adjacent
 * rows, wave w starts its walk at step w mod (row_bytes / (16 *
 * lanes_per_row)) and wraps; 2, a strip's rows are spread over the matrix
 * (strip s holds rows s, s + S, s + 2S, ... with S = rows * lanes_per_row / 64);
 * 3, as 1 but with the lanes of a row interleaved: lane l reads row
 * l mod (64 / lanes_per_row) of the strip, 16-byte vector l / (64 /
 * lanes_per_row) of the row's piece.
 *
 * buf            device pointer, 16-byte aligned, rows * row_bytes bytes
 *                (< 4 GiB), caller-owned, only read
 * lanes_per_row  4, 8, 16, 32 or 64; rows % (64 / lanes_per_row) == 0 and
 *                row_bytes % (16 * lanes_per_row) == 0
 * depth          2, 4, 8 or 16
 * order          0, 1, 2 or 3 (above)
 * nontemporal    nonzero: loads with the non-temporal cache policy
 * blocks_per_cu  1..32
 * sink           device pointer to one 32-bit word (4-byte aligned); written
 *                only if the XOR of everything read equals a fixed constant
 * stream         hipStream_t (NULL: default stream); enqueued, not waited for
 *
 * Returns 0 on success, 1 for an invalid argument, 2 for an unsupported
 * shape or size, 3 for a misaligned pointer (all before any launch), 4 when
 * HIP reports an error.
 */
int32_t wq_probe_read(const void* buf, int64_t rows, int64_t row_bytes, int32_t lanes_per_row,
                      int32_t depth, int32_t order, int32_t nontemporal, int32_t blocks_per_cu,
                      void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WQ_PROBE_H */
