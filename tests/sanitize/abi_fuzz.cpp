// Host half of the libptpc C ABI under AddressSanitizer / UBSan.
//
// Built with g++ from ptpc_api.cpp and plan.cpp (the library's own host
// sources) plus the stub launchers below, which stand in for the GPU
// kernels: they record that a launch was requested and check the
// preconditions the real launchers rely on (what validation must guarantee
// before anything is enqueued), running the same kernel-choice code the real
// launchers run.  main() calls every entry point over a grid of extents,
// pitches and pointers that includes negative, zero, misaligned, boundary and
// extreme values, and checks that every status is a defined one, that a
// launch is requested exactly when a call reports PTPC_OK for a non-empty
// shape, and that no call launches after an error.  Any sanitizer report
// aborts the run.
#include <cinttypes>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "kernels.h"
#include "ptpc.h"

static long g_launches = 0;
static long g_fail = 0;

#define REQUIRE(c)                                                                         \
    do {                                                                                   \
        if (!(c)) {                                                                        \
            std::fprintf(stderr, "%s:%d: requirement failed: %s\n", __FILE__, __LINE__, #c); \
            ++g_fail;                                                                      \
        }                                                                                  \
    } while (0)

static bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

namespace ptpc {

hipError_t launch_quant_act(const uint16_t* x, int64_t T, int64_t Ci, int64_t ldx, uint8_t* qx,
                            int64_t ldq, float* dx, hipStream_t) {
    ++g_launches;
    REQUIRE(T >= 1 && Ci >= 0 && Ci % 16 == 0 && ldx >= Ci && ldq >= Ci && dx && al16(dx));
    if (Ci > 0) {
        REQUIRE(x && qx && al16(x) && al16(qx) && ldx % 8 == 0 && ldq % 16 == 0);
        const ActPlan p = act_plan(Ci);
        REQUIRE((p.G == 0 && p.vpt == 0) || (p.G >= 16 && p.vpt >= 1 && p.vpt <= 16));
    }
    REQUIRE(quant_act_plan_name(T, Ci) != nullptr);
    return hipSuccess;
}

hipError_t launch_quant_weight(const uint16_t* w, int64_t Ci, int64_t Co, int64_t ldw,
                               uint8_t* packed, float* dw, hipStream_t) {
    ++g_launches;
    REQUIRE(Ci >= 0 && Co >= 1 && Ci % 16 == 0 && Co % 16 == 0 && ldw >= Co && dw && al16(dw));
    if (Ci > 0) REQUIRE(w && packed && al16(w) && al16(packed) && ldw % 8 == 0);
    return hipSuccess;
}

hipError_t launch_tensor_scale(const uint16_t* x, int64_t R, int64_t C, int64_t ld, float* d,
                               hipStream_t) {
    ++g_launches;
    REQUIRE(R >= 0 && C >= 0 && C % 16 == 0 && ld >= C && d && al16(d));
    if (R > 0 && C > 0) REQUIRE(x && al16(x) && ld % 8 == 0);
    return hipSuccess;
}

hipError_t launch_quant_act_static(const uint16_t* x, int64_t T, int64_t Ci, int64_t ldx,
                                   const float* d, uint8_t* qx, int64_t ldq, hipStream_t) {
    ++g_launches;
    REQUIRE(T >= 1 && Ci >= 16 && Ci % 16 == 0 && ldx >= Ci && ldq >= Ci);
    REQUIRE(x && d && qx && al16(x) && al16(d) && al16(qx) && ldx % 8 == 0 && ldq % 16 == 0);
    return hipSuccess;
}

hipError_t launch_quant_weight_static(const uint16_t* w, int64_t Ci, int64_t Co, int64_t ldw,
                                      const float* d, uint8_t* packed, hipStream_t) {
    ++g_launches;
    REQUIRE(Ci >= 16 && Co >= 16 && Ci % 16 == 0 && Co % 16 == 0 && ldw >= Co);
    REQUIRE(w && d && packed && al16(w) && al16(d) && al16(packed) && ldw % 8 == 0);
    return hipSuccess;
}

hipError_t launch_unpack_weight(const uint8_t* packed, int64_t Ci, int64_t Co, uint8_t* qw,
                                hipStream_t) {
    ++g_launches;
    REQUIRE(Ci >= 16 && Co >= 16 && packed && qw && al16(packed) && al16(qw));
    return hipSuccess;
}

static void gemm_pre(const uint8_t* qx, int64_t ldq, const float* dx, const uint8_t* wp,
                     const float* dw, int64_t T, int64_t Ci, int64_t Co, const void* out,
                     int64_t ldo) {
    REQUIRE(T >= 1 && Co >= 16 && Ci >= 0 && Ci % 16 == 0 && Co % 16 == 0);
    REQUIRE(ldq >= Ci && ldo >= Co && ldo % 8 == 0);
    REQUIRE(dx && dw && out && al16(dx) && al16(dw) && al16(out));
    if (Ci > 0) REQUIRE(qx && wp && al16(qx) && al16(wp) && ldq % 16 == 0);
    REQUIRE(gemm_plan_name(gemm_plan(T, Ci, Co)) != nullptr);
}

hipError_t launch_gemm(const uint8_t* qx, int64_t ldq, const float* dx, const uint8_t* wp,
                       const float* dw, int64_t T, int64_t Ci, int64_t Co, uint16_t* out,
                       int64_t ldo, float* fp32_out, hipStream_t, bool) {
    ++g_launches;
    gemm_pre(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo);
    if (fp32_out) REQUIRE(al16(fp32_out));
    return hipSuccess;
}

hipError_t launch_gemm_unfused_bf16(const uint8_t* qx, int64_t ldq, const float* dx,
                                    const uint8_t* wp, const float* dw, int64_t T, int64_t Ci,
                                    int64_t Co, uint16_t* out, int64_t ldo, uint16_t* ws,
                                    hipStream_t) {
    ++g_launches;
    gemm_pre(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo);
    REQUIRE(ws && al16(ws));
    return hipSuccess;
}

hipError_t launch_gemm_splitk(const uint8_t* qx, int64_t ldq, const float* dx, const uint8_t* wp,
                              const float* dw, int64_t T, int64_t Ci, int64_t Co, uint16_t* out,
                              int64_t ldo, float* ws, int splits, hipStream_t) {
    ++g_launches;
    gemm_pre(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo);
    REQUIRE(ws && al16(ws) && splits >= 2 && splits <= 8);
    return hipSuccess;
}

hipError_t noalloc_scratch(void** ptr) {
    *ptr = reinterpret_cast<void*>(uintptr_t(0x900000));
    return hipSuccess;
}

}  // namespace ptpc

// Fake device addresses: never dereferenced (the stubs only look at them).
static uint8_t* const P0 = reinterpret_cast<uint8_t*>(uintptr_t(0x100000));
static uint8_t* const P1 = reinterpret_cast<uint8_t*>(uintptr_t(0x200000));
static uint8_t* const P2 = reinterpret_cast<uint8_t*>(uintptr_t(0x300000));
static uint8_t* const P3 = reinterpret_cast<uint8_t*>(uintptr_t(0x400000));
static uint8_t* const P4 = reinterpret_cast<uint8_t*>(uintptr_t(0x500000));

static const int64_t kVals[] = {INT64_MIN, -16, -1, 0, 1, 15, 16, 32, 48, 256, 4096,
                                (1 << 17), (1 << 17) + 16, (1 << 22), (1 << 22) + 16,
                                (1 << 24), (1 << 24) + 16, (int64_t(1) << 36) + 16, INT64_MAX};
static const int kN = sizeof(kVals) / sizeof(kVals[0]);

// Pointer variant v: all valid, one null, one misaligned.
static uint8_t* ptr(uint8_t* base, int v, int which) {
    if (v == 1 + which) return nullptr;
    if (v == 6 + which) return base + 8;
    return base;
}

static void check(int st, long before, bool empty) {
    REQUIRE(st >= 0 && st <= 5);
    if (st != PTPC_OK) REQUIRE(g_launches == before);          // nothing launched on error
    if (st == PTPC_OK && !empty) REQUIRE(g_launches > before);
    REQUIRE(ptpc_status_string(st) != nullptr);
}

int main() {
    long calls = 0;
    for (int v = 0; v < 11; ++v)
        for (int a = 0; a < kN; ++a)
            for (int b = 0; b < kN; ++b)
                for (int c = 0; c < kN; ++c) {
                    const int64_t T = kVals[a], Ci = kVals[b], ld = kVals[c];
                    long n0 = g_launches;
                    int st = ptpc_quant_act(ptr(P0, v, 0), T, Ci, ld, ptr(P1, v, 1), ld,
                                            reinterpret_cast<float*>(ptr(P2, v, 2)), nullptr);
                    check(st, n0, T == 0);
                    n0 = g_launches;
                    st = ptpc_quant_act_static(ptr(P0, v, 0), T, Ci, ld,
                                               reinterpret_cast<float*>(ptr(P2, v, 2)),
                                               ptr(P1, v, 1), ld, nullptr);
                    check(st, n0, T == 0 || Ci == 0);
                    n0 = g_launches;
                    st = ptpc_tensor_scale(ptr(P0, v, 0), T, Ci, ld,
                                           reinterpret_cast<float*>(ptr(P2, v, 2)), nullptr);
                    check(st, n0, false);
                    // weights: (Ci, Co, ldw) = (T, Ci, ld) of this loop
                    n0 = g_launches;
                    st = ptpc_quant_weight(ptr(P0, v, 0), T, Ci, ld, ptr(P1, v, 1),
                                           reinterpret_cast<float*>(ptr(P2, v, 2)), nullptr);
                    check(st, n0, Ci == 0);
                    n0 = g_launches;
                    st = ptpc_quant_weight_static(ptr(P0, v, 0), T, Ci, ld,
                                                  reinterpret_cast<float*>(ptr(P2, v, 2)),
                                                  ptr(P1, v, 1), nullptr);
                    check(st, n0, T == 0 || Ci == 0);
                    n0 = g_launches;
                    st = ptpc_unpack_weight(ptr(P0, v, 0), T, Ci, ptr(P1, v, 1), nullptr);
                    check(st, n0, T == 0 || Ci == 0);
                    (void)ptpc_weight_packed_bytes(T, Ci);
                    (void)ptpc_gemm_unfused_workspace_bytes(T, Ci);
                    (void)ptpc_gemm_unfused_bf16_workspace_bytes(T, Ci);
                    (void)ptpc_quant_act_kernel(T, Ci);
                    calls += 6;
                }
    // GEMM calls over (T, Ci, Co, ldq, ldo), pitches tied to the extents or
    // taken from the grid.
    for (int v = 0; v < 11; ++v)
        for (int a = 0; a < kN; ++a)
            for (int b = 0; b < kN; ++b)
                for (int c = 0; c < kN; ++c)
                    for (int d = 0; d < 3; ++d) {
                        const int64_t T = kVals[a], Ci = kVals[b], Co = kVals[c];
                        const int64_t ldq = d == 0 ? Ci : d == 1 ? kVals[(b + 1) % kN] : 8192;
                        const int64_t ldo = d == 0 ? Co : d == 1 ? kVals[(c + 1) % kN] : 8192;
                        const uint8_t* qx = ptr(P0, v, 0);
                        const float* dx = reinterpret_cast<const float*>(ptr(P1, v, 1));
                        const void* wp = ptr(P2, v, 2);
                        const float* dw = reinterpret_cast<const float*>(ptr(P3, v, 3));
                        void* out = ptr(P4, v, 4);
                        const bool empty = T == 0 || Co == 0;
                        long n0 = g_launches;
                        int st = ptpc_gemm(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, nullptr);
                        check(st, n0, empty);
                        n0 = g_launches;
                        st = ptpc_gemm_tensor(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, nullptr);
                        check(st, n0, empty);
                        n0 = g_launches;
                        st = ptpc_gemm_unfused(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo,
                                               reinterpret_cast<float*>(P1 + 0x10000), nullptr);
                        check(st, n0, empty);
                        n0 = g_launches;
                        st = ptpc_gemm_unfused_bf16(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo,
                                                    P1 + 0x10000, nullptr);
                        check(st, n0, empty);
                        const size_t need = ptpc_gemm_workspace_bytes(T, Ci, Co);
                        n0 = g_launches;
                        st = ptpc_gemm_ws(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo,
                                          P3 + 0x10000, need, nullptr);
                        check(st, n0, empty);
                        n0 = g_launches;
                        st = ptpc_gemm_noalloc(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, nullptr);
                        check(st, n0, empty);
                        if (st == PTPC_OK) REQUIRE(need <= PTPC_NOALLOC_SCRATCH_BYTES);
                        (void)ptpc_gemm_kernel(T, Ci, Co);
                        calls += 6;
                    }
    std::printf("abi_fuzz: %ld calls, %ld launches, %ld failures\n", calls, g_launches, g_fail);
    return g_fail == 0 ? 0 : 1;
}
