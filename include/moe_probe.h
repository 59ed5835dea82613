/*
 * moe_probe.h — peak probes of libmoe.so: measurement helpers that sit beside the MoE layer's
 * C ABI (moe.h) and are not part of the layer. They measure what one MI355X sustains, so
 * that the layer's kernels can be quoted against measured ceilings as well as against the
 * published peaks (8 TB/s HBM3E, 2.5 PFLOP/s dense bf16 MFMA).
 *
 * Conventions as in moe.h: device pointers, caller-owned, asynchronous on `stream`, arguments
 * validated before anything is enqueued, status returned, detail in moe_last_error().
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Plain device copy dst[0, bytes) = src[0, bytes) in 16-byte non-temporal vectors, one
 * contiguous chunk per workgroup (at most 16384 workgroups): bytes read + bytes written over
 * the kernel time is the sustained HBM rate of a streaming kernel. src and dst 16-byte aligned, not overlapping; bytes a multiple of 16,
 * at least 16. MOE_EINVAL otherwise; MOE_EHIP if the launch fails. */
moe_status moe_probe_copy(const void* src, void* dst, size_t bytes, moe_stream_t stream);

/* Matrix-core loop: `workgroups` workgroups of 256 threads; every wave issues MOE_PROBE_CHAINS
 * independent chains of `iters` v_mfma_f32_16x16x32_bf16 each (16*16*32*2 flops per MFMA) on
 * fixed bf16 register operands in [-0.125, 0.125], with no memory traffic; each thread then
 * writes one float to out [workgroups*256] (4-byte aligned). Flops per launch:
 * workgroups * 4 * MOE_PROBE_CHAINS * iters * 16384. MOE_EINVAL for workgroups outside
 * [1, 2^20] or iters outside [1, 2^24] or a NULL / misaligned out; MOE_EHIP if the launch fails. */
#define MOE_PROBE_CHAINS 16
moe_status moe_probe_mfma(float* out, int64_t workgroups, int64_t iters, moe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
