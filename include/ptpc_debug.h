/*
 * Debug builds of libptpc -- not part of the library's ABI (include/ptpc.h);
 * for tests and measurement only.
 *
 * libptpc_lds_poison.so  (-DPTPC_LDS_POISON) Every pipelined GEMM kernel
 *     overwrites each LDS region with 0x7F bytes (E4M3 NaN) right before it
 *     issues the fills that refill the region.  Same ABI and, when the
 *     pipelines read LDS only between a fill's landing and the next refill,
 *     the same results as libptpc.so bit for bit.
 *
 * libptpc_timeline.so  (-DPTPC_TIMELINE) Wave 0 of every workgroup of the
 *     main tiled GEMM kernel (gemm16_kernel: every tile of 256 or more
 *     tokens and the 128x128 tiles of 65..255) stores the GPU's constant
 *     100 MHz clock at four points into a caller buffer:
 *       [0] workgroup start, [1] K loop entered (first operands landed),
 *       [2] K loop done, [3] last output store completed.
 *     Same ABI plus the call below; results equal libptpc.so's.
 *
 * libptpc_join_lost.so  (-DPTPC_JOIN_LOST) The two-range K join of
 *     ptpc_gemm_ws / ptpc_gemm_noalloc never raises its per-tile flag and
 *     waits only 16 sleeps for it, so every joined tile takes the path of a
 *     wait that runs out: its outputs are NaN.  Every other path equals
 *     libptpc.so bit for bit.
 */
#ifndef PTPC_DEBUG_H
#define PTPC_DEBUG_H

#ifdef __cplusplus
extern "C" {
#endif

/* libptpc_timeline.so only: buf = DEVICE buffer of [workgroups][4] uint64
 * (at least one row per workgroup of the next launches), or NULL to stop
 * recording.  Returns the hipError_t of setting it (0 = success).  Takes
 * effect for kernels launched after the call; not thread-safe. */
int ptpc_debug_set_timeline(void* buf);

#ifdef __cplusplus
}
#endif
#endif /* PTPC_DEBUG_H */
