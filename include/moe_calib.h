/*
 * moe_calib.h -- calibration kernels of libmoe_shard.so.
 *
 * Not part of the layer: they measure what this GPU reaches outside it, so
 * that the layer's kernels can be reported as a fraction of a measured
 * ceiling beside the vendor's peak figures (HBM bandwidth, bf16 matrix
 * throughput).  Same conventions as moe_shard.h: device pointers, the
 * caller's stream, MOE_* status codes, nothing allocated.
 */
#ifndef MOE_CALIB_H
#define MOE_CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming copy of `bytes` bytes (a multiple of 16, both pointers 16-byte
 * aligned, buffers not overlapping): nontemporal 16-byte loads and stores,
 * four in flight per lane, a grid of `blocks` workgroups of 256 threads
 * striding over the buffer (8192 workgroups copy 1 GiB fastest on
 * MI355X).  HBM traffic is 2 * bytes.  MOE_EINVAL for a bad argument. */
int moe_calib_copy(const void* src, void* dst, int64_t bytes, int32_t blocks, void* stream);

/* Matrix-core peak loop: `blocks` workgroups of 8 waves, each wave issuing
 * `iters` rounds of 8 independent v_mfma_f32_16x16x32_bf16 on register
 * operands (no memory traffic).  *flops (host) receives the bf16 flops the
 * launch performs (2 * 16 * 16 * 32 per MFMA); sink (device, 512 floats)
 * receives a value that keeps the work from being optimised away. */
int moe_calib_mfma(int32_t blocks, int32_t iters, float* sink, int64_t* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_CALIB_H */
