/*
 * w12_probe.h - HBM read-bandwidth probe of libw12 (measurement only; not
 * part of the W12 format or its GEMM).
 *
 * SpecPilot (arXiv 2611.02501) section 3.1, "Ceilings": a kernel bound by
 * weight reads is judged against the bytes it must read and the bandwidth
 * the memory system actually delivers. This probe measures the second number
 * on the device at hand: it streams a buffer once with 16-byte non-temporal
 * loads (the load the W12 GEMM kernels use for records) and discards the data.
 *
 * Conventions as in w12.h: device pointers owned by the caller, asynchronous
 * on `stream`, arguments checked before any launch, negative status on error.
 */
#ifndef W12_PROBE_H
#define W12_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* work distribution of w12_probe_read */
#define W12_PROBE_STATIC 0  /* workgroup p reads the p-th of `grid` equal contiguous ranges          */
#define W12_PROBE_DYNAMIC 1 /* workgroups take 16-byte-word chunks in order from an atomic counter   */
#define W12_PROBE_STRIDE 2  /* grid-stride: consecutive waves read consecutive kilobytes             */
#define W12_PROBE_PIECES 3  /* workgroup p reads pieces p, p + grid, p + 2 grid, ... of `piece` bytes */

#define W12_PROBE_WS_BYTES 256 /* workspace: counters, zero before first use, left zero by every call */

/* Reads `bytes` (a multiple of 16, at most 2^40) from `buf` (16-byte aligned)
 * with `grid` workgroups of `block` threads (a multiple of 64, at most 1024);
 * each lane keeps `loads` 16-byte loads in flight (1, 2, 4 or 8).
 * `piece` (W12_PROBE_PIECES only): bytes of each contiguous piece, a multiple
 * of 16; the last piece may be shorter.
 * `stamps` (nullable, device, 3 * grid entries): workgroup p writes its start
 * and end times (the 100 MHz real-time counter) and the XCD it ran on.
 * `lds_bytes` (0 .. 163776): LDS each workgroup reserves and leaves unused, to
 * reproduce the occupancy of a kernel that needs that much.
 * `ws`: W12_PROBE_WS_BYTES of device memory (used by W12_PROBE_DYNAMIC).
 * The data read is folded into a value that is never stored. */
int w12_probe_read(const void* buf, size_t bytes, int grid, int block, int loads, int mode, size_t piece,
                   int lds_bytes, uint64_t* stamps, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* W12_PROBE_H */
