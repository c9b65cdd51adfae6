// Exhaustive check of the epilogue's fp32 -> bf16 pair conversion
// (f32x2_to_bf16x2_rne in device_common.h, one v_cvt_pk_bf16_f32 on gfx950)
// against round-to-nearest-even written with integer arithmetic: every fp32
// bit pattern goes through the low half, and (an odd multiplier permutes the
// 2^32 patterns) every pattern through the high half too.  NaN inputs must
// give a NaN of the same sign; every other input the exact RNE result,
// subnormals, overflow to infinity and signed zeros included.
#include "device_common.h"

namespace {

__device__ __forceinline__ uint32_t rne_ref(uint32_t u) {
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ bool same(uint32_t in, uint32_t got) {
    const bool nan_in = (in & 0x7F800000u) == 0x7F800000u && (in & 0x007FFFFFu) != 0;
    if (nan_in) return (got & 0x7F80u) == 0x7F80u && (got & 0x7Fu) != 0 && (got >> 15) == (in >> 31);
    return got == rne_ref(in);
}

__global__ __launch_bounds__(256) void cvt_check_kernel(unsigned long long* __restrict__ res) {
    unsigned long long bad = 0;
    const uint64_t stride = (uint64_t)gridDim.x * 256;
    for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < (1ull << 32); i += stride) {
        const uint32_t lo = (uint32_t)i;
        const uint32_t hi = lo * 2654435761u + 0x9E3779B9u;   // a bijection of the 2^32 patterns
        const uint32_t r = ptpc::f32x2_to_bf16x2_rne(__uint_as_float(lo), __uint_as_float(hi));
        const bool ok = same(lo, r & 0xFFFFu) && same(hi, r >> 16);
        if (!ok) {
            ++bad;
            atomicMin(res + 1, (unsigned long long)lo);
        }
    }
    if (bad) atomicAdd(res, bad);
}

}  // namespace

// res[0] = number of mismatching pairs, res[1] = smallest low-half pattern of
// a mismatch (initialise it to ~0).  Returns the launch status.
extern "C" int cvt_bf16_check(unsigned long long* res, void* stream) {
    hipLaunchKernelGGL(cvt_check_kernel, dim3(8192), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), res);
    return (int)hipGetLastError();
}
