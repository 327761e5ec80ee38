/* Measurement probes (libmoe_probe.so): the achievable HBM read rate and
 * bf16 MFMA rate of the GPU, the measured ceilings that the path's kernels
 * are reported against besides the published peaks.  Not part of the path.
 *
 * All pointers are device pointers owned by the caller; the calls enqueue on
 * `stream` (NULL = default stream) and do not synchronise.  They return 0, -1
 * for a bad argument (nothing launched), -2 if the launch failed. */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of blocks (and of block_xor entries) the read probe uses. */
int moe_probe_read_blocks(void);

/* Streams `bytes` (a positive multiple of 16; buf 16-byte aligned) once,
 * each block one contiguous chunk, each lane 32 contiguous bytes per step
 * (two 16-byte loads), and writes the XOR of every 32-bit word each block read to
 * block_xor[moe_probe_read_blocks()]; the XOR of those equals the XOR of all
 * words of the buffer. */
int moe_probe_stream_read(const void* buf, long long bytes, uint32_t* block_xor, void* stream);

/* FLOPs of one moe_probe_mfma call. */
long long moe_probe_mfma_flops(int blocks, int iters);

/* `blocks` blocks of 4 waves, each wave running `iters` rounds of 8
 * independent v_mfma_f32_32x32x16_bf16 on all-ones operands (1..2^20 each).
 * out[blocks * 4] receives, per wave, 16 * iters (exact) or -1 if any
 * accumulator lane disagreed. */
int moe_probe_mfma(int blocks, int iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
