/*
 * rkv_probe.h -- measurement aids for MI355X (gfx950), in librkv_probe.so,
 * a library of their own beside the cache library librkv.so.
 *
 * These are not steps of the cache method: they measure the two ceilings
 * that bound its kernels on the running device, so that a benchmark can
 * report each kernel against the measured peak beside the published one.
 *
 *   rkv_probe_fp8_mfma ... dense FP8 matrix throughput: the instruction the
 *                          attention uses (32x32x64 e4m3 with E8M0 scales),
 *                          issued back to back with no memory traffic.
 *   rkv_probe_stream ..... HBM bandwidth of a streaming in-place
 *                          read-modify-write, the access pattern of the
 *                          delta rotation (nontemporal 16-byte accesses).
 *
 * The caller owns every buffer, calls only enqueue work on the given
 * stream, host-visible misuse returns RKV_PROBE_EINVAL (with a message in
 * rkv_probe_last_error()) and enqueues nothing, a failed launch returns
 * RKV_PROBE_EHIP.  Time the calls with events on the same stream.
 */
#ifndef RKV_PROBE_H
#define RKV_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { RKV_PROBE_EINVAL = -1, RKV_PROBE_EHIP = -2 };

/* Message for the last error of a probe call on the calling thread. */
const char* rkv_probe_last_error(void);

/* Runs `workgroups` workgroups of 4 waves; every wave issues `iters` rounds
 * of 4 independent v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 operands, neutral
 * scales), i.e. workgroups * 4 * iters * 4 * 131072 floating-point
 * operations.  sink: device float[workgroups], receives one accumulator
 * value per workgroup (so the work cannot be elided).  workgroups in
 * [1, 65536], iters in [1, 2^20]. */
int rkv_probe_fp8_mfma(int32_t workgroups, int32_t iters, float* sink, hipStream_t stream);

/* Reads and rewrites every 16-byte word of the device buffer `buf` once
 * (the first 4 bytes of each word are complemented, so two calls restore
 * the contents): 2 * bytes of HBM traffic.  buf 16-byte aligned, bytes a
 * positive multiple of 16. */
int rkv_probe_stream(void* buf, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RKV_PROBE_H */
