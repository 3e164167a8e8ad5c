/*
 * relay_probes.h - measurement probes for gfx950 (MI355X), built as librelay_probes.so.
 *
 * Not part of the attention path.  They measure what this GPU reaches at all, the
 * ceilings that the decode kernels' roofline fractions are also reported against
 * (beside the published 8 TB/s HBM and 2.5 PFLOP/s dense bf16 peaks):
 *   - relay_probe_read: a plain streaming read of a device buffer;
 *   - relay_probe_mfma: bf16 matrix-core products on register operands only.
 *
 * Both enqueue one kernel on `stream` (a hipStream_t, NULL for the default stream) and
 * return 0, or -1 for a bad argument (nothing enqueued).  The caller times them.
 */
#ifndef RELAY_PROBES_H
#define RELAY_PROBES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads `bytes` bytes of the device buffer `buf` once (16-byte loads; each of the
 * `workgroups` workgroups of 256 threads reads one contiguous slab) and writes one
 * float per workgroup to the device array `sink` (so that no load is dead).
 * buf: 16-byte aligned, bytes a positive multiple of 16; sink: >= workgroups floats;
 * workgroups >= 1.
 */
int relay_probe_read(const void* buf, size_t bytes, float* sink, int32_t workgroups, void* stream);

/*
 * `workgroups` workgroups of four waves; every wave issues iters x 4 independent
 * v_mfma_f32_32x32x16_bf16 products (32768 flops each) on register operands, then
 * writes one float per thread to `sink` (>= 256 * workgroups floats).  Floating-point
 * work of the launch: workgroups * 4 * iters * 4 * 32768.  iters >= 1, workgroups >= 1.
 */
int relay_probe_mfma(float* sink, int32_t iters, int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RELAY_PROBES_H */
