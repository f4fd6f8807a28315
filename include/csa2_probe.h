/*
 * csa2_probe.h - peak probes for the roofline figures: plain gfx950 kernels
 * of known work whose measured rates stand beside the vendor peaks (HBM
 * 8 TB/s, dense FP8 MFMA 5.0 PFLOP/s), so a kernel's fraction can be stated
 * against both.  Separate library (libcsa2_probe.so); nothing in the layer
 * step uses it.
 *
 * Every function enqueues one kernel on stream s and returns at once; the
 * caller times it (events on s).  The return value is a hipError_t: 0 on
 * success, hipErrorInvalidValue (1) for arguments outside the stated ranges
 * (then nothing is launched), else the launch error.  Outputs are written
 * only under a condition the kernels never meet, so `sink` needs 4 bytes.
 */
#ifndef CSA2_PROBE_H
#define CSA2_PROBE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* FP8 matrix-core issue rate: `blocks` workgroups of 4 waves, each wave
 * issuing `iters` V_MFMA_SCALE_F32_16X16X128_F8F6F4 with register operands
 * into four independent accumulators (no memory traffic in the loop).
 * Work: blocks * 4 * iters * 65,536 FLOP.  epilogue = 1 adds, per MFMA, the
 * indexer's minimal score epilogue on an earlier accumulator (4 integer
 * max for the ReLU, 4 fp32 multiply-adds for the head weights, 1 add):
 * the rate the dense prefill indexer could reach if nothing but its
 * essential per-score arithmetic shared the SIMD with the matrix core.
 * 1 <= blocks <= 1<<20; iters a positive multiple of 4; epilogue 0 or 1;
 * sink: device, 4 bytes. */
int32_t csa2_probe_mfma_fp8(int32_t blocks, int32_t iters, int32_t epilogue, float* sink, hipStream_t s);

/* HBM read rate: `blocks` workgroups of 256 threads stream `bytes` from
 * device memory at `src` in 16-byte loads (grid-stride, four loads in
 * flight per thread) and fold them into a register.
 * src: device, 16-byte aligned; bytes a positive multiple of 16;
 * 1 <= blocks <= 1<<20; sink: device, 4 bytes. */
int32_t csa2_probe_stream_read(const void* src, uint64_t bytes, int32_t blocks, uint32_t* sink, hipStream_t s);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_PROBE_H */
