// Internal launchers of libptpc (host side).  Every launcher only enqueues
// kernels on the given stream and returns hipGetLastError(); argument
// validation happens before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ptpc {

// Compute units of the target GPU (MI355X): the tile rules count rounds of
// this many workgroups.
constexpr int64_t kCus = 256;

// "Long K" for the split-K choices (K = Ci bytes of FP8 per row): from here
// on the workspace form splits the K-split 64x64 tile shapes too, and its
// split kernel's weight fills carry the non-temporal hint.
constexpr int64_t kLongK = 16384;
// K from which the workspace form splits K for 256 tokens and more.
constexpr int64_t kSplitK256 = 12288;

// K extent of the packed weight: whole 128-byte K tiles.
inline int64_t round_up_k(int64_t Ci) { return (Ci + 127) / 128 * 128; }

hipError_t launch_quant_act(const uint16_t* x, int64_t T, int64_t Ci, int64_t ldx,
                            uint8_t* qx, int64_t ldq, float* dx, hipStream_t s);

hipError_t launch_quant_weight(const uint16_t* w, int64_t Ci, int64_t Co, int64_t ldw,
                               uint8_t* packed, float* dw, hipStream_t s);

// Per-tensor comparator: d[0] = amax / 448 over an R x C bf16 matrix (1 if
// all zero); static casts with the scalar scale d[0].
hipError_t launch_tensor_scale(const uint16_t* x, int64_t R, int64_t C, int64_t ld, float* d,
                               hipStream_t s);
hipError_t launch_quant_act_static(const uint16_t* x, int64_t T, int64_t Ci, int64_t ldx,
                                   const float* d, uint8_t* qx, int64_t ldq, hipStream_t s);
hipError_t launch_quant_weight_static(const uint16_t* w, int64_t Ci, int64_t Co, int64_t ldw,
                                      const float* d, uint8_t* packed, hipStream_t s);

hipError_t launch_unpack_weight(const uint8_t* packed, int64_t Ci, int64_t Co, uint8_t* qw,
                                hipStream_t s);

// The GEMM kernel and tile ptpc_gemm (and both two-step forms) launch for a
// shape, chosen on the host from T, Ci and Co alone.
enum class GemmPlan : int {
    k16_256x256, k16_192x256, k16_256x224, k16_256x160, k16_128x256, k16_128x128, k16_128x224,
    k16s_64x64, k32_64x64, k32_64x128, k32_128x128, k32_32x64,
    kDecode_2x2, kDecode_2x1, kDecode_1x2, kDecode_1x1,
};
GemmPlan gemm_plan(int64_t T, int64_t Ci, int64_t Co);
const char* gemm_plan_name(GemmPlan p);

// Launch shape of the activation quantizer for rows of Ci elements: G
// threads per row holding VPT 16-byte vectors each, or G = 0 for the two-pass
// long-row kernel; and its kernel's name (for a row count and length).
struct ActPlan {
    int G;
    int vpt;
};
ActPlan act_plan(int64_t Ci);
const char* quant_act_plan_name(int64_t T, int64_t Ci);

// fp32_out == nullptr: fused epilogue writing bf16 `out`.
// fp32_out != nullptr: the GEMM stores unscaled fp32 sums there ([T x Co],
// pitch Co), then a rescale kernel writes bf16 `out`.
// per_tensor: the fused epilogue uses dx[0] and dw[0] for every row and
// column (the two-step form is per-token / per-channel only).
hipError_t launch_gemm(const uint8_t* qx, int64_t ldq, const float* dx, const uint8_t* wp,
                       const float* dw, int64_t T, int64_t Ci, int64_t Co, uint16_t* out,
                       int64_t ldo, float* fp32_out, hipStream_t s, bool per_tensor = false);

// The bf16-intermediate two-step form: step 1 writes bf16(acc) unscaled to
// ws ([T x Co], pitch Co), step 2 scales it into bf16 `out`.
hipError_t launch_gemm_unfused_bf16(const uint8_t* qx, int64_t ldq, const float* dx,
                                    const uint8_t* wp, const float* dw, int64_t T, int64_t Ci,
                                    int64_t Co, uint16_t* out, int64_t ldo, uint16_t* ws,
                                    hipStream_t s);

// Split-K for token counts whose tiled grid leaves most CUs idle: the number
// of K ranges (1 = no split; then the call is ptpc_gemm's), and the launch
// writing S fp32 partial slices [S][T][Co] to ws before one reduce + scale
// pass into bf16 `out`.
int gemm_splitk_plan(int64_t T, int64_t Ci, int64_t Co);
bool gemm_split_tiles256(int64_t T, int64_t Ci, int64_t Co);
// Two K ranges of 256x256 tiles: the ranges are joined inside the GEMM
// kernel (the second to finish adds the first's published sums), so ws holds
// one fp32 slot per tile plus a 4-word record per tile, and no reduction
// pass follows.  Other splits write S slices [S][T][Co] and reduce them.
bool gemm_split_fixup(int64_t T, int64_t Ci, int64_t Co);
// Workspace bytes of the split plan (0: no split).
size_t gemm_splitk_workspace_bytes(int64_t T, int64_t Ci, int64_t Co);
hipError_t launch_gemm_splitk(const uint8_t* qx, int64_t ldq, const float* dx, const uint8_t* wp,
                              const float* dw, int64_t T, int64_t Ci, int64_t Co, uint16_t* out,
                              int64_t ldo, float* ws, int splits, hipStream_t s);

// The no-allocation split-K form: its scratch size, and the device address
// of the current device's copy of the scratch array (looked up once per
// device).  The split plan needs at most 64 MiB (see gemm_splitk_plan).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void** ptr);

}  // namespace ptpc
