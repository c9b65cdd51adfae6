/*
 * libptpc -- PTPC-FP8 linear-layer hot path for AMD MI355X (gfx950).
 *
 * The method: vLLM blog "PTPC-FP8: Boosting vLLM Performance on AMD ROCm"
 * (2025-02-24), cited below as [PTPC].  FP8 weights and FP8 activations,
 * one scale per token for the activations and one per output channel for
 * the weights (§What is PTPC-FP8; §PTPC: a precision-targeted scheme), with
 * the scales applied to the GEMM result on chip before it is written
 * (§The solution: fusion; §Why this matters).  The FP8 format is OCP E4M3
 * (largest finite value 448).
 *
 * Conventions shared by every call:
 *   - Every buffer pointer is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees or keeps a pointer past the call.
 *   - bf16 buffers are passed as void* holding bf16 bit patterns; E4M3
 *     buffers as uint8_t* holding E4M3 bit patterns; scales are fp32.
 *   - Matrices are row-major; leading dimensions (ld*) are in ELEMENTS.
 *   - stream is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work on it and returns without synchronising; calls are
 *     thread-safe (no global mutable state).
 *   - Arguments are validated on the host before anything is enqueued.  On
 *     any error nothing is launched and no output is touched.  A failed
 *     launch reports PTPC_ERR_HIP.  No call aborts or throws.
 *   - Supported shapes (v1): T >= 0, Ci >= 0, Co >= 0 with Ci % 16 == 0 and
 *     Co % 16 == 0; base pointers 16-byte aligned; bf16 pitches multiples of
 *     8 elements and E4M3 pitches multiples of 16 (16-byte rows).  A zero
 *     extent is a no-op returning PTPC_OK (except as noted for Ci == 0).
 *     The weight and GEMM calls also need Ci <= 2^17 (the K range in which
 *     every partial sum of E4M3 products is exact in double, the accuracy
 *     reference).  Every call needs row pitches <= 2^22 elements, row
 *     counts (T, R) and output columns (Co) <= 2^24, and a GEMM at most 2^36
 *     outputs (T * Co).
 *     Anything else returns PTPC_ERR_UNSUPPORTED / PTPC_ERR_ALIGN.
 *
 * Quantization rule (readings taken where [PTPC] is silent):
 *   Delta = amax / 448 in fp32 (an all-zero vector gets Delta = 1);
 *   code  = E4M3(x / Delta), the fp32 quotient correctly rounded, then
 *           rounded to the nearest E4M3 value, ties to even, saturating at
 *           +-448, sign kept.
 */
#ifndef PTPC_H
#define PTPC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PTPC_ABI_VERSION 1

typedef enum {
    PTPC_OK = 0,
    PTPC_ERR_NULL = 1,        /* a required pointer is NULL                 */
    PTPC_ERR_SHAPE = 2,       /* negative extent, or pitch below the extent */
    PTPC_ERR_UNSUPPORTED = 3, /* shape outside the v1 contract above         */
    PTPC_ERR_ALIGN = 4,       /* pointer or pitch not 16-byte aligned        */
    PTPC_ERR_HIP = 5          /* the HIP runtime refused a launch            */
} ptpc_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* ptpc_status_string(int status);

/* PTPC_ABI_VERSION of the built library. */
int ptpc_abi_version(void);

/*
 * Per-token activation quantization ([PTPC] §PTPC: a precision-targeted
 * scheme, "per-token activation quantization"; §Understanding the figure,
 * Delta_X of shape [T x 1]).
 *   x   [T x Ci] bf16, pitch ldx (>= Ci)         -- read
 *   qx  [T x Ci] E4M3 codes, pitch ldq (>= Ci)   -- written
 *   dx  [T] fp32, dx[t] = max_k |x[t,k]| / 448 (1 for an all-zero row)
 * Ci == 0 with T > 0 writes dx[t] = 1 and no codes.
 */
ptpc_status ptpc_quant_act(const void* x, int64_t T, int64_t Ci, int64_t ldx,
                           uint8_t* qx, int64_t ldq, float* dx, void* stream);

/*
 * Size in bytes of the packed weight buffer for a [Ci x Co] weight:
 * Co * roundup(Ci, 128).  Returns 0 for unsupported or empty shapes
 * (including Ci > 2^17).
 */
size_t ptpc_weight_packed_bytes(int64_t Ci, int64_t Co);

/*
 * Per-output-channel weight quantization and prepacking ([PTPC]
 * §PTPC: a precision-targeted scheme, "per-channel weight quantization",
 * each weight column gets its own scale; §Understanding the figure,
 * Delta_W of shape [1 x Co]; done once when the model loads, no
 * pre-quantized checkpoint -- §TL;DR / §Getting started).
 *   w         [Ci x Co] bf16, pitch ldw (>= Co)             -- read
 *   w_packed  ptpc_weight_packed_bytes(Ci, Co) bytes         -- written
 *             layout (opaque to callers; ptpc_unpack_weight inverts it):
 *             Kp = roundup(Ci, 128); 1 KB blocks, block (g, s) for
 *             g < Co/16, s < Kp/64 at byte (g*Kp/64 + s)*1024; the 16-byte
 *             unit u of a block holds the codes of w[64s+16c .. 64s+16c+15]
 *             [16g + u/4] with c = (u%4) ^ ((u/16)%4); codes for k >= Ci are
 *             zero.  This is the GEMM's LDS order for its MFMA B operand, so
 *             the GEMM streams the weight as contiguous 1 KB reads.
 *   dw        [Co] fp32, dw[o] = max_k |w[k,o]| / 448 (1 for a zero column);
 *             also used as the column-amax scratch during the call.
 */
ptpc_status ptpc_quant_weight(const void* w, int64_t Ci, int64_t Co, int64_t ldw,
                              void* w_packed, float* dw, void* stream);

/*
 * Inverse of the packing, for tests and inspection: qw [Ci x Co] E4M3 codes,
 * row-major with pitch Co, qw[k][o] = code of w[k][o].
 */
ptpc_status ptpc_unpack_weight(const void* w_packed, int64_t Ci, int64_t Co,
                               uint8_t* qw, void* stream);

/*
 * Fused PTPC-FP8 GEMM ([PTPC] §The solution: fusion -- the scaled GEMM that
 * takes the token scales and channel scales; §Why this matters -- scaling
 * happens on chip before the result is written):
 *   out[t,o] = bf16( (acc[t,o] * dx[t]) * dw[o] ),
 *   acc[t,o] = sum_k E4M3(qx[t,k]) * E4M3(qw[k,o])   (FP8 MFMA, fp32 accumulate)
 *   qx [T x Ci] pitch ldq; dx [T]; w_packed / dw from ptpc_quant_weight;
 *   out [T x Co] bf16, pitch ldo (>= Co), written once.
 * The fp32 products are rounded to bf16 with round-to-nearest-even.
 */
ptpc_status ptpc_gemm(const uint8_t* qx, int64_t ldq, const float* dx,
                      const void* w_packed, const float* dw, int64_t T,
                      int64_t Ci, int64_t Co, void* out, int64_t ldo,
                      void* stream);

/*
 * Workspace that lets ptpc_gemm_ws split K across workgroups: nonzero only
 * where output tiles are too few to occupy the GPU -- 65..255 tokens with few
 * output columns (except where ptpc_gemm already splits K inside each
 * workgroup of 64x64 tiles: up to 128 tokens when those tiles need no more
 * rounds of the GPU than larger ones; at 129..255 tokens with Ci >= 16384 or
 * where ptpc_gemm runs 128x128 tiles, one 256-row tile per weight slab), and
 * 256 tokens or more with Ci >= 16384
 * when fewer than 128 tiles of 256x256 cover the output (with 12288 <= Ci <
 * 16384 only for a split of at least 4 ranges where ptpc_gemm's own tiles
 * leave CUs idle) -- then 4 * S * T * Co bytes for S K ranges (at most
 * 64 MiB), except for splits of 2 ranges over 256x256 tiles, which need
 * n * (262144 + 16) bytes for the n = ceil(T/256) * ceil(Co/256) output
 * tiles (at most 128 tiles, 32 MiB).
 */
size_t ptpc_gemm_workspace_bytes(int64_t T, int64_t Ci, int64_t Co);

/*
 * ptpc_gemm with a caller-provided workspace (ptpc_gemm_workspace_bytes(T,
 * Ci, Co) bytes, 16-byte aligned, contents ignored and overwritten).  Where
 * that size is 0 this is exactly ptpc_gemm (workspace may be NULL).
 * Otherwise K is cut into S ranges, each workgroup writes the fp32 partial
 * sums of one range of one output tile to the workspace, and one more pass
 * adds the S partials in range order and applies the same epilogue
 * bf16((sum * dx[t]) * dw[o]).  With S = 2 over 256x256 tiles there is no
 * second pass: of the two workgroups of a tile, the one that finishes first
 * publishes its sums in the workspace, the other adds them to its own and
 * applies the epilogue (per-tile counters in the workspace, cleared by the
 * call; a workgroup only ever waits for one that is already running, and
 * its wait is bounded: sums that never arrive leave that tile NaN).  The
 * result is deterministic and the same in both forms; it can differ from
 * ptpc_gemm's in the last bf16 bit (another fp32 summation order).
 * PTPC_ERR_NULL for a missing, PTPC_ERR_SHAPE for a too small workspace.
 */
ptpc_status ptpc_gemm_ws(const uint8_t* qx, int64_t ldq, const float* dx,
                         const void* w_packed, const float* dw, int64_t T,
                         int64_t Ci, int64_t Co, void* out, int64_t ldo,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * ptpc_gemm_ws for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same kernels and the same result, bit for bit, as ptpc_gemm_ws with a
 * workspace, but the split-K partial sums go to a scratch array the library
 * holds on each GPU (PTPC_NOALLOC_SCRATCH_BYTES, kept until the process
 * ends) and nothing is allocated or freed.  The caller still passes inputs
 * and outputs; the stream must belong to the current device.  Where
 * ptpc_gemm_workspace_bytes(T, Ci, Co) is 0 this is exactly ptpc_gemm.
 * Shapes whose split needs more than PTPC_NOALLOC_SCRATCH_BYTES return
 * PTPC_ERR_UNSUPPORTED before anything is launched (the current split plan
 * never needs more: at most 64 MiB by construction).  Calls that overlap on
 * one GPU (different streams, or threads) share the scratch and race; calls
 * in one stream are ordered and safe.  The first call on a device looks up
 * the scratch's device address (PTPC_ERR_HIP if that fails).
 */
#define PTPC_NOALLOC_SCRATCH_BYTES (64u << 20)
ptpc_status ptpc_gemm_noalloc(const uint8_t* qx, int64_t ldq, const float* dx,
                              const void* w_packed, const float* dw, int64_t T,
                              int64_t Ci, int64_t Co, void* out, int64_t ldo,
                              void* stream);

/* Workspace needed by ptpc_gemm_unfused: 4 * T * Co bytes (fp32 [T x Co]). */
size_t ptpc_gemm_unfused_workspace_bytes(int64_t T, int64_t Co);

/*
 * The naive two-step form ([PTPC] §The challenge: two-step vs fused): step 1
 * is the same FP8 GEMM writing the unscaled fp32 result to `workspace`
 * ([T x Co], pitch Co, caller-allocated, at least
 * ptpc_gemm_unfused_workspace_bytes(T, Co) bytes); step 2 reads it back and
 * writes out = bf16((ws * dx[t]) * dw[o]).  Same arguments and result as
 * ptpc_gemm (bit-identical output), kept for comparison.
 */
ptpc_status ptpc_gemm_unfused(const uint8_t* qx, int64_t ldq, const float* dx,
                              const void* w_packed, const float* dw, int64_t T,
                              int64_t Ci, int64_t Co, void* out, int64_t ldo,
                              float* workspace, void* stream);

/* Workspace needed by ptpc_gemm_unfused_bf16: 2 * T * Co bytes. */
size_t ptpc_gemm_unfused_bf16_workspace_bytes(int64_t T, int64_t Co);

/*
 * The two-step form with a bf16 intermediate ([PTPC] §The challenge: two-step
 * vs fused -- the listing leaves the intermediate's type open; this is its
 * bf16 reading): step 1 writes ws = bf16(acc) unscaled ([T x Co], pitch Co,
 * caller-allocated, ptpc_gemm_unfused_bf16_workspace_bytes(T, Co) bytes, 16-
 * byte aligned), step 2 writes out = bf16((float(ws) * dx[t]) * dw[o]).
 * Rounds twice, so it differs from ptpc_gemm in the last bf16 bit at times;
 * it moves half the intermediate bytes of ptpc_gemm_unfused.
 */
ptpc_status ptpc_gemm_unfused_bf16(const uint8_t* qx, int64_t ldq, const float* dx,
                                   const void* w_packed, const float* dw, int64_t T,
                                   int64_t Ci, int64_t Co, void* out, int64_t ldo,
                                   void* workspace, void* stream);

/*
 * ---- Per-tensor ("standard") FP8, the comparator ------------------------
 * [PTPC] measures PTPC-FP8 against FP8 with one scale per tensor
 * (§PTPC: a precision-targeted scheme; §Benchmark 1 throughput,
 * §Benchmark 2.1/2.2 accuracy).  These calls give that baseline on the same
 * kernels: a scalar scale per matrix, measured (ptpc_tensor_scale) or given
 * ahead of time ("static", e.g. from calibration).  Same conventions and
 * contract as above; a scale argument is a device pointer to ONE fp32.
 */

/* d[0] = max |x| / 448 over the R x C bf16 matrix x (pitch ld), or 1 if it
 * is all zero or empty.  Works for activations ([T x Ci]) and weights
 * ([Ci x Co]) alike.  C % 16 == 0. */
ptpc_status ptpc_tensor_scale(const void* x, int64_t R, int64_t C, int64_t ld, float* d,
                              void* stream);

/* qx[t,k] = E4M3(x[t,k] / d[0]) (saturating at +-448), x [T x Ci] bf16, qx
 * E4M3 codes; d[0] > 0 is read, not written. */
ptpc_status ptpc_quant_act_static(const void* x, int64_t T, int64_t Ci, int64_t ldx,
                                  const float* d, uint8_t* qx, int64_t ldq, void* stream);

/* Quantize W [Ci x Co] with the scalar scale d[0] and prepack it into the
 * layout of ptpc_quant_weight (same size, same ptpc_unpack_weight). */
ptpc_status ptpc_quant_weight_static(const void* w, int64_t Ci, int64_t Co, int64_t ldw,
                                     const float* d, void* w_packed, void* stream);

/* ptpc_gemm with scalar scales: out[t,o] = bf16((acc[t,o] * dx[0]) * dw[0]);
 * dx and dw point to one fp32 each. */
ptpc_status ptpc_gemm_tensor(const uint8_t* qx, int64_t ldq, const float* dx,
                             const void* w_packed, const float* dw, int64_t T,
                             int64_t Ci, int64_t Co, void* out, int64_t ldo,
                             void* stream);

/*
 * ---- Diagnostics ----------------------------------------------------------
 * Which kernel a call launches for a shape (the choice is made on the host
 * from the extents alone), as a static string naming the kernel and its
 * template arguments, e.g. "gemm16_kernel<256,256,2,2>".  NULL for shapes
 * the call rejects or for which it launches nothing.  Nothing is launched.
 */

/* Kernel of ptpc_gemm, ptpc_gemm_unfused, ptpc_gemm_unfused_bf16,
 * ptpc_gemm_tensor and of ptpc_gemm_ws where it does not split K. */
const char* ptpc_gemm_kernel(int64_t T, int64_t Ci, int64_t Co);

/* Kernel of ptpc_quant_act for T rows of Ci elements. */
const char* ptpc_quant_act_kernel(int64_t T, int64_t Ci);

/* Number of K ranges ptpc_gemm_ws and ptpc_gemm_noalloc cut K into for a
 * shape (1: no split, the call is ptpc_gemm's; 0: a shape the calls reject). */
int ptpc_gemm_ws_splits(int64_t T, int64_t Ci, int64_t Co);

#ifdef __cplusplus
}
#endif
#endif /* PTPC_H */
