/*
 * qlora_read_probe.h - C ABI of libqlora_probe.so, a measurement helper that
 * ships beside the QLoRA NF4 library.
 *
 * It streams a device buffer once, as fast as a plain read can go on this
 * GPU (16-byte loads per lane, four loads in flight per lane, a grid-stride
 * walk), and throws the data away.  Timed at the size of a memory-bound
 * kernel's input, it gives the device's own read ceiling for that size, the
 * figure such a kernel is judged against beside the HBM specification.  It
 * computes nothing of the method.
 */
#ifndef QLORA_READ_PROBE_H
#define QLORA_READ_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes (a multiple of 16, >= 16) of device memory at `src`
 * (16-byte aligned) with `grid` workgroups of 256 threads (1 .. 65536),
 * enqueued on `stream` (hipStream_t as void*; NULL = the null stream).
 * `sink` is a device uint32 the kernel writes only when an impossible XOR
 * of the data comes up, so the loads cannot be optimised away.  Returns 0,
 * 1 for a bad argument (nothing launched), 8 for a launch failure. */
int qlora_read_probe(const void* src, int64_t bytes, int grid, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_READ_PROBE_H */
