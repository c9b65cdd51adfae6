// C ABI of libptpc: argument validation on the host, then kernel launches
// on the caller's stream.  The contract is documented in include/ptpc.h.
#include "ptpc.h"

#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>

#include "kernels.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Host-side fault injection for the error-path tests: with PTPC_FAULT=launch
// in the environment, every call that would launch work returns
// PTPC_ERR_HIP instead, without touching the GPU.
bool forced_launch_failure() {
    const char* f = std::getenv("PTPC_FAULT");
    return f != nullptr && std::strcmp(f, "launch") == 0;
}

ptpc_status from_hip(hipError_t e) { return e == hipSuccess ? PTPC_OK : PTPC_ERR_HIP; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Longest K (Ci) a weight or GEMM call accepts: the exact-sum argument of the
// contraction (every partial sum of E4M3 products a multiple of 2^-18 below
// 2^53 units) holds up to 2^17, far beyond any layer of the targeted models.
constexpr int64_t kMaxK = int64_t(1) << 17;
// Longest row pitch of any matrix: the kernels address an activation tile
// (<= 256 rows of ldq bytes), a weight slab (<= 256 columns of roundup(Ci,
// 128) bytes) and an output tile (<= 256 rows of 2*ldo bytes) with 32-bit
// buffer offsets, which holds for pitches up to 2^22 elements.
constexpr int64_t kMaxPitch = int64_t(1) << 22;
// Most rows (T, R) or output columns (Co) of one call, and most outputs T*Co
// of one GEMM: tile and workgroup counts then stay within 32-bit indices
// (at most 2^22 output tiles of 128 x 128).
constexpr int64_t kMaxExtent = int64_t(1) << 24;
constexpr int64_t kMaxOutputs = int64_t(1) << 36;

}  // namespace

extern "C" {

const char* ptpc_status_string(int status) {
    switch (status) {
        case PTPC_OK: return "PTPC_OK";
        case PTPC_ERR_NULL: return "PTPC_ERR_NULL: required pointer is NULL";
        case PTPC_ERR_SHAPE: return "PTPC_ERR_SHAPE: negative extent or pitch below extent";
        case PTPC_ERR_UNSUPPORTED:
            return "PTPC_ERR_UNSUPPORTED: shape outside the contract (Ci, Co multiples of 16)";
        case PTPC_ERR_ALIGN: return "PTPC_ERR_ALIGN: pointer or pitch not 16-byte aligned";
        case PTPC_ERR_HIP: return "PTPC_ERR_HIP: kernel launch failed";
        default: return "unknown ptpc_status";
    }
}

int ptpc_abi_version(void) { return PTPC_ABI_VERSION; }

ptpc_status ptpc_quant_act(const void* x, int64_t T, int64_t Ci, int64_t ldx, uint8_t* qx,
                           int64_t ldq, float* dx, void* stream) {
    if (T < 0 || Ci < 0 || ldx < Ci || ldq < Ci) return PTPC_ERR_SHAPE;
    if (Ci % 16 != 0 || T > kMaxExtent || ldx > kMaxPitch || ldq > kMaxPitch)
        return PTPC_ERR_UNSUPPORTED;
    if (T == 0) return PTPC_OK;
    if (dx == nullptr || (Ci > 0 && (x == nullptr || qx == nullptr))) return PTPC_ERR_NULL;
    if (!aligned16(dx) || (Ci > 0 && (!aligned16(x) || !aligned16(qx) || ldx % 8 != 0 ||
                                      ldq % 16 != 0)))
        return PTPC_ERR_ALIGN;
    if (forced_launch_failure()) return PTPC_ERR_HIP;
    return from_hip(ptpc::launch_quant_act(static_cast<const uint16_t*>(x), T, Ci, ldx, qx, ldq,
                                           dx, as_stream(stream)));
}

size_t ptpc_weight_packed_bytes(int64_t Ci, int64_t Co) {
    if (Ci <= 0 || Co <= 0 || Ci % 16 != 0 || Co % 16 != 0 || Ci > kMaxK || Co > kMaxExtent)
        return 0;
    return (size_t)Co * (size_t)ptpc::round_up_k(Ci);
}

ptpc_status ptpc_quant_weight(const void* w, int64_t Ci, int64_t Co, int64_t ldw,
                              void* w_packed, float* dw, void* stream) {
    if (Ci < 0 || Co < 0 || ldw < Co) return PTPC_ERR_SHAPE;
    if (Ci % 16 != 0 || Co % 16 != 0 || Ci > kMaxK || Co > kMaxExtent || ldw > kMaxPitch)
        return PTPC_ERR_UNSUPPORTED;
    if (Co == 0) return PTPC_OK;
    if (dw == nullptr || (Ci > 0 && (w == nullptr || w_packed == nullptr))) return PTPC_ERR_NULL;
    if (!aligned16(dw) || (Ci > 0 && (!aligned16(w) || !aligned16(w_packed) || ldw % 8 != 0)))
        return PTPC_ERR_ALIGN;
    if (forced_launch_failure()) return PTPC_ERR_HIP;
    return from_hip(ptpc::launch_quant_weight(static_cast<const uint16_t*>(w), Ci, Co, ldw,
                                              static_cast<uint8_t*>(w_packed), dw,
                                              as_stream(stream)));
}

ptpc_status ptpc_unpack_weight(const void* w_packed, int64_t Ci, int64_t Co, uint8_t* qw,
                               void* stream) {
    if (Ci < 0 || Co < 0) return PTPC_ERR_SHAPE;
    if (Ci % 16 != 0 || Co % 16 != 0 || Ci > kMaxK || Co > kMaxExtent) return PTPC_ERR_UNSUPPORTED;
    if (Ci == 0 || Co == 0) return PTPC_OK;
    if (w_packed == nullptr || qw == nullptr) return PTPC_ERR_NULL;
    if (!aligned16(w_packed) || !aligned16(qw)) return PTPC_ERR_ALIGN;
    if (forced_launch_failure()) return PTPC_ERR_HIP;
    return from_hip(ptpc::launch_unpack_weight(static_cast<const uint8_t*>(w_packed), Ci, Co, qw,
                                               as_stream(stream)));
}

static ptpc_status check_gemm(const uint8_t* qx, int64_t ldq, const float* dx,
                              const void* w_packed, const float* dw, int64_t T, int64_t Ci,
                              int64_t Co, const void* out, int64_t ldo) {
    if (T < 0 || Ci < 0 || Co < 0 || ldq < Ci || ldo < Co) return PTPC_ERR_SHAPE;
    if (Ci % 16 != 0 || Co % 16 != 0) return PTPC_ERR_UNSUPPORTED;
    if (ldq > kMaxPitch || Ci > kMaxK || ldo > kMaxPitch || T > kMaxExtent || Co > kMaxExtent ||
        T * Co > kMaxOutputs)
        return PTPC_ERR_UNSUPPORTED;
    if (T == 0 || Co == 0) return PTPC_OK;
    if (dx == nullptr || dw == nullptr || out == nullptr ||
        (Ci > 0 && (qx == nullptr || w_packed == nullptr)))
        return PTPC_ERR_NULL;
    if (!aligned16(dx) || !aligned16(dw) || !aligned16(out) || ldo % 8 != 0 ||
        (Ci > 0 && (!aligned16(qx) || !aligned16(w_packed) || ldq % 16 != 0)))
        return PTPC_ERR_ALIGN;
    return PTPC_OK;
}

ptpc_status ptpc_gemm(const uint8_t* qx, int64_t ldq, const float* dx, const void* w_packed,
                      const float* dw, int64_t T, int64_t Ci, int64_t Co, void* out, int64_t ldo,
                      void* stream) {
    ptpc_status st = check_gemm(qx, ldq, dx, w_packed, dw, T, Ci, Co, out, ldo);
    if (st != PTPC_OK || T == 0 || Co == 0) return st;
    if (forced_launch_failure()) return PTPC_ERR_HIP;
    return from_hip(ptpc::launch_gemm(qx, ldq, dx, static_cast<const uint8_t*>(w_packed), dw, T,
                                      Ci, Co, static_cast<uint16_t*>(out), ldo, nullptr,
                                      as_stream(stream)));
}

size_t ptpc_gemm_unfused_workspace_bytes(int64_t T, int64_t Co) {
    if (T <= 0 || Co <= 0 || T > kMaxExtent || Co > kMaxExtent || T * Co > kMaxOutputs) return 0;
    return (size_t)T * (size_t)Co * sizeof(float);
}

ptpc_status ptpc_gemm_unfused(const uint8_t* qx, int64_t ldq, const float* dx,
                              const void* w_packed, const float* dw, int64_t T, int64_t Ci,
                              int64_t Co, void* out, int64_t ldo, float* workspace,
                              void* stream) {
    ptpc_status st = check_gemm(qx, ldq, dx, w_packed, dw, T, Ci, Co, out, ldo);
    if (st != PTPC_OK || T == 0 || Co == 0) return st;
    if (workspace == nullptr) return PTPC_ERR_NULL;
    if (!aligned16(workspace)) return PTPC_ERR_ALIGN;
    if (forced_launch_failure()) return PTPC_ERR_HIP;
    return from_hip(ptpc::launch_gemm(qx, ldq, dx, static_cast<const uint8_t*>(w_packed), dw, T,
                                      Ci, Co, static_cast<uint16_t*>(out), ldo, workspace,
                                      as_stream(stream)));
}

size_t ptpc_gemm_workspace_bytes(int64_t T, int64_t Ci, int64_t Co) {
    if (T <= 0 || Ci <= 0 || Co <= 0 || Ci % 16 != 0 || Co % 16 != 0 || Ci > kMaxK ||
        T > kMaxExtent || Co > kMaxExtent || T * Co > kMaxOutputs)
        return 0;
    return ptpc::gemm_splitk_workspace_bytes(T, Ci, Co);
}

ptpc_status ptpc_gemm_ws(const uint8_t* qx, int64_t ldq, const float* dx, const void* w_packed,
                         const float* dw, int64_t T, int64_t Ci, int64_t Co, void* out,
                         int64_t ldo, void* workspace, size_t workspace_bytes, void* stream) {
    ptpc_status st = check_gemm(qx, ldq, dx, w_packed, dw, T, Ci, Co, out, ldo);
    if (st != PTPC_OK || T == 0 || Co == 0) return st;
    const size_t need = ptpc_gemm_workspace_bytes(T, Ci, Co);
    if (need > 0) {
        if (workspace == nullptr) return PTPC_ERR_NULL;
        if (workspace_bytes < need) return PTPC_ERR_SHAPE;
        if (!aligned16(workspace)) return PTPC_ERR_ALIGN;
    }
    if (forced_launch_failure()) return PTPC_ERR_HIP;
    if (need == 0)
        return from_hip(ptpc::launch_gemm(qx, ldq, dx, static_cast<const uint8_t*>(w_packed), dw,
                                          T, Ci, Co, static_cast<uint16_t*>(out), ldo, nullptr,
                                          as_stream(stream)));
    return from_hip(ptpc::launch_gemm_splitk(
        qx, ldq, dx, static_cast<const uint8_t*>(w_packed), dw, T, Ci, Co,
        static_cast<uint16_t*>(out), ldo, static_cast<float*>(workspace),
        ptpc::gemm_splitk_plan(T, Ci, Co), as_stream(stream)));
}

ptpc_status ptpc_gemm_noalloc(const uint8_t* qx, int64_t ldq, const float* dx,
                              const void* w_packed, const float* dw, int64_t T, int64_t Ci,
                              int64_t Co, void* out, int64_t ldo, void* stream) {
    static_assert(PTPC_NOALLOC_SCRATCH_BYTES == ptpc::kNoAllocScratchBytes, "scratch size");
    ptpc_status st = check_gemm(qx, ldq, dx, w_packed, dw, T, Ci, Co, out, ldo);
    if (st != PTPC_OK || T == 0 || Co == 0) return st;
    const size_t need = ptpc_gemm_workspace_bytes(T, Ci, Co);
    if (need > ptpc::kNoAllocScratchBytes) return PTPC_ERR_UNSUPPORTED;
    if (forced_launch_failure()) return PTPC_ERR_HIP;
    if (need == 0)
        return from_hip(ptpc::launch_gemm(qx, ldq, dx, static_cast<const uint8_t*>(w_packed), dw,
                                          T, Ci, Co, static_cast<uint16_t*>(out), ldo, nullptr,
                                          as_stream(stream)));
    void* ws = nullptr;
    if (ptpc::noalloc_scratch(&ws) != hipSuccess) return PTPC_ERR_HIP;
    return from_hip(ptpc::launch_gemm_splitk(
        qx, ldq, dx, static_cast<const uint8_t*>(w_packed), dw, T, Ci, Co,
        static_cast<uint16_t*>(out), ldo, static_cast<float*>(ws),
        ptpc::gemm_splitk_plan(T, Ci, Co), as_stream(stream)));
}

size_t ptpc_gemm_unfused_bf16_workspace_bytes(int64_t T, int64_t Co) {
    if (T <= 0 || Co <= 0 || T > kMaxExtent || Co > kMaxExtent || T * Co > kMaxOutputs) return 0;
    return (size_t)T * (size_t)Co * 2;
}

ptpc_status ptpc_gemm_unfused_bf16(const uint8_t* qx, int64_t ldq, const float* dx,
                                   const void* w_packed, const float* dw, int64_t T, int64_t Ci,
                                   int64_t Co, void* out, int64_t ldo, void* workspace,
                                   void* stream) {
    ptpc_status st = check_gemm(qx, ldq, dx, w_packed, dw, T, Ci, Co, out, ldo);
    if (st != PTPC_OK || T == 0 || Co == 0) return st;
    if (workspace == nullptr) return PTPC_ERR_NULL;
    if (!aligned16(workspace)) return PTPC_ERR_ALIGN;
    if (forced_launch_failure()) return PTPC_ERR_HIP;
    return from_hip(ptpc::launch_gemm_unfused_bf16(
        qx, ldq, dx, static_cast<const uint8_t*>(w_packed), dw, T, Ci, Co,
        static_cast<uint16_t*>(out), ldo, static_cast<uint16_t*>(workspace), as_stream(stream)));
}

// ---- per-tensor comparator ---------------------------------------------

ptpc_status ptpc_tensor_scale(const void* x, int64_t R, int64_t C, int64_t ld, float* d,
                              void* stream) {
    if (R < 0 || C < 0 || ld < C) return PTPC_ERR_SHAPE;
    if (C % 16 != 0 || R > kMaxExtent || ld > kMaxPitch) return PTPC_ERR_UNSUPPORTED;
    if (d == nullptr || (R > 0 && C > 0 && x == nullptr)) return PTPC_ERR_NULL;
    if (!aligned16(d) || (R > 0 && C > 0 && (!aligned16(x) || ld % 8 != 0)))
        return PTPC_ERR_ALIGN;
    if (forced_launch_failure()) return PTPC_ERR_HIP;
    return from_hip(ptpc::launch_tensor_scale(static_cast<const uint16_t*>(x), R, C, ld, d,
                                              as_stream(stream)));
}

ptpc_status ptpc_quant_act_static(const void* x, int64_t T, int64_t Ci, int64_t ldx,
                                  const float* d, uint8_t* qx, int64_t ldq, void* stream) {
    if (T < 0 || Ci < 0 || ldx < Ci || ldq < Ci) return PTPC_ERR_SHAPE;
    if (Ci % 16 != 0 || T > kMaxExtent || ldx > kMaxPitch || ldq > kMaxPitch)
        return PTPC_ERR_UNSUPPORTED;
    if (T == 0 || Ci == 0) return PTPC_OK;
    if (x == nullptr || d == nullptr || qx == nullptr) return PTPC_ERR_NULL;
    if (!aligned16(x) || !aligned16(d) || !aligned16(qx) || ldx % 8 != 0 || ldq % 16 != 0)
        return PTPC_ERR_ALIGN;
    if (forced_launch_failure()) return PTPC_ERR_HIP;
    return from_hip(ptpc::launch_quant_act_static(static_cast<const uint16_t*>(x), T, Ci, ldx,
                                                  d, qx, ldq, as_stream(stream)));
}

ptpc_status ptpc_quant_weight_static(const void* w, int64_t Ci, int64_t Co, int64_t ldw,
                                     const float* d, void* w_packed, void* stream) {
    if (Ci < 0 || Co < 0 || ldw < Co) return PTPC_ERR_SHAPE;
    if (Ci % 16 != 0 || Co % 16 != 0 || Ci > kMaxK || Co > kMaxExtent || ldw > kMaxPitch)
        return PTPC_ERR_UNSUPPORTED;
    if (Ci == 0 || Co == 0) return PTPC_OK;
    if (w == nullptr || d == nullptr || w_packed == nullptr) return PTPC_ERR_NULL;
    if (!aligned16(w) || !aligned16(d) || !aligned16(w_packed) || ldw % 8 != 0)
        return PTPC_ERR_ALIGN;
    if (forced_launch_failure()) return PTPC_ERR_HIP;
    return from_hip(ptpc::launch_quant_weight_static(static_cast<const uint16_t*>(w), Ci, Co,
                                                     ldw, d, static_cast<uint8_t*>(w_packed),
                                                     as_stream(stream)));
}

ptpc_status ptpc_gemm_tensor(const uint8_t* qx, int64_t ldq, const float* dx,
                             const void* w_packed, const float* dw, int64_t T, int64_t Ci,
                             int64_t Co, void* out, int64_t ldo, void* stream) {
    ptpc_status st = check_gemm(qx, ldq, dx, w_packed, dw, T, Ci, Co, out, ldo);
    if (st != PTPC_OK || T == 0 || Co == 0) return st;
    if (forced_launch_failure()) return PTPC_ERR_HIP;
    return from_hip(ptpc::launch_gemm(qx, ldq, dx, static_cast<const uint8_t*>(w_packed), dw, T,
                                      Ci, Co, static_cast<uint16_t*>(out), ldo, nullptr,
                                      as_stream(stream), true));
}

// ---- diagnostics ------------------------------------------------------------

const char* ptpc_gemm_kernel(int64_t T, int64_t Ci, int64_t Co) {
    if (T <= 0 || Ci < 0 || Co <= 0 || Ci % 16 != 0 || Co % 16 != 0 || Ci > kMaxK ||
        T > kMaxExtent || Co > kMaxExtent || T * Co > kMaxOutputs)
        return nullptr;
    return ptpc::gemm_plan_name(ptpc::gemm_plan(T, Ci, Co));
}

int ptpc_gemm_ws_splits(int64_t T, int64_t Ci, int64_t Co) {
    if (T <= 0 || Ci <= 0 || Co <= 0 || Ci % 16 != 0 || Co % 16 != 0 || Ci > kMaxK ||
        T > kMaxExtent || Co > kMaxExtent || T * Co > kMaxOutputs)
        return 0;
    return ptpc::gemm_splitk_plan(T, Ci, Co);
}

const char* ptpc_quant_act_kernel(int64_t T, int64_t Ci) {
    if (T <= 0 || Ci < 0 || Ci % 16 != 0 || T > kMaxExtent || Ci > kMaxPitch) return nullptr;
    return ptpc::quant_act_plan_name(T, Ci);
}

}  // extern "C"
