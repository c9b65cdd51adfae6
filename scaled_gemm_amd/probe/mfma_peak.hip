// Register-only FP8 MFMA throughput on the whole chip: the ceiling the
// GEMM's MFMA-bound roofline is measured against, under the chip's power
// limit.  Not part of the library: built as its own shared object and used
// only by `bench.py --mfma-ceiling`.
//
// One workgroup of 4 waves per CU (one wave per SIMD, 256 accumulator
// registers each, the GEMM's 256x256-tile occupancy); every wave multiplies
// random finite E4M3 operands held in registers into a 128x128 fp32
// accumulator, in the two MFMA forms the GEMM kernels use.  No memory
// traffic inside the loop.  Each accumulator is next written 16 or 64 MFMAs
// later (an accumulation chain), the operands are written 8 wait states
// before the first MFMA and the accumulators read 24 after the last (the
// 16x16x128 form is issued from inline asm with the accumulators tied to
// AGPRs, as in the GEMM; the 32x32x64 form through the builtin, as in the
// GEMM's other kernels, with the compiler's hazard handling).
#include <hip/hip_runtime.h>
#include <cstdint>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

namespace {

__device__ __forceinline__ v8i random_codes(uint32_t& x) {
    v8i r;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t w = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x = x * 1664525u + 1013904223u;
            uint32_t b = x >> 24;
            if ((b & 0x7Fu) == 0x7Fu) b ^= 1u;        // no NaN codes
            w |= b << (8 * k);
        }
        r[i] = (int)w;
    }
    return r;
}

template <int FORM>
__global__ __launch_bounds__(256, 1) void mfma_peak_kernel(int64_t iters, float* sink,
                                                           uint32_t seed) {
    uint32_t x = seed ^ ((uint32_t)(blockIdx.x * 256 + threadIdx.x) * 2654435761u);
    v8i a0 = random_codes(x), a1 = random_codes(x);
    v8i b0 = random_codes(x), b1 = random_codes(x);
    // The operands are complete before the wait states that precede the
    // first MFMA (the empty asm orders every write ahead of the nops).
    asm volatile("" : "+v"(a0), "+v"(a1), "+v"(b0), "+v"(b1));
    asm volatile("s_nop 7");
    float total = 0.0f;
    if constexpr (FORM == 16) {
        v4f acc[8][8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
                asm volatile("" : "+a"(acc[i][j]));
            }
        asm volatile("s_nop 4");
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0"
                                 : "+a"(acc[i][j])
                                 : "v"((j & 1) ? b1 : b0), "v"((i & 1) ? a1 : a0));
        }
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                asm volatile("" : "+a"(acc[i][j]));
                total += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
            }
    } else {
        v16f acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
                asm volatile("" : "+a"(acc[i][j]));
            }
        asm volatile("s_nop 4");
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        (j & 1) ? b1 : b0, (i & 1) ? a1 : a0, acc[i][j], 0, 0, 0, 0, 0, 0);
        }
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                asm volatile("" : "+a"(acc[i][j]));
#pragma unroll
                for (int e = 0; e < 16; ++e) total += acc[i][j][e];
            }
    }
    sink[blockIdx.x * 256 + threadIdx.x] = total;
}

}  // namespace

// form 16: v_mfma_f32_16x16x128_f8f6f4; form 32: v_mfma_f32_32x32x64_f8f6f4.
// Launches `blocks` workgroups of 256 threads; sink holds blocks * 256 floats.
// Flops per launch: blocks * 4 waves * iters * 2 * 128 * 128 * K, K = 128
// (form 16) or 64 (form 32).
extern "C" int mfma_peak(int form, int blocks, int64_t iters, float* sink, void* stream) {
    if ((form != 16 && form != 32) || blocks <= 0 || iters <= 0 || sink == nullptr) return 1;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (form == 16)
        hipLaunchKernelGGL(mfma_peak_kernel<16>, dim3((unsigned)blocks), dim3(256), 0, s, iters,
                           sink, 12345u);
    else
        hipLaunchKernelGGL(mfma_peak_kernel<32>, dim3((unsigned)blocks), dim3(256), 0, s, iters,
                           sink, 12345u);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
