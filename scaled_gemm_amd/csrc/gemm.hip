// FP8 x FP8 GEMM with the PTPC scale epilogue, gfx950 MFMA.
//
// Method: vLLM blog "PTPC-FP8: Boosting vLLM Performance on AMD ROCm",
// §The solution: fusion (the scaled GEMM takes the per-token and
// per-channel scales) and §Why this matters (scaling is done on chip,
// before the result is written); §The challenge: two-step vs fused gives
// the unfused form kept for comparison (GEMM, write, read back, scale).
//
// out[t,o] = bf16((acc[t,o] * dx[t]) * dw[o]),
// acc[t,o] = sum_k qx[t,k] * qw[k,o] on OCP E4M3 values, fp32 accumulation
// in v_mfma_f32_32x32x64_f8f6f4.
//
// Data layout: qx is [T x Ci] row-major (K contiguous); the packed weight is
// [Co x Kp] (K contiguous, Kp = roundup(Ci, 128), zero codes past Ci), so A
// and B tiles are both "rows of 128 K bytes" and both MFMA operands are read
// from LDS the same way: lane l takes row l % 32 of a 32-row slab and 32
// consecutive K bytes starting at 32 * (l / 32) within a 64-byte K step.
// Each LDS row is 128 bytes = 8 chunks of 16 bytes, stored at chunk
// position c ^ swz(row) so that the 32 rows one MFMA operand read touches
// fall on different banks.
#include "device_common.h"
#include "kernels.h"

namespace ptpc {

constexpr int BK = 128;

__device__ __forceinline__ int swz(int row) { return row & 7; }

template <int BM, int BN, int WM, int WN, bool FUSED>
__global__ __launch_bounds__(WM * WN * 64) void gemm_kernel(
    const uint8_t* __restrict__ qx, int64_t ldq, const float* __restrict__ dx,
    const uint8_t* __restrict__ wp, int64_t Kp, const float* __restrict__ dw,
    int64_t T, int64_t Ci, int64_t Co, void* __restrict__ out, int64_t ldo) {
    constexpr int NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int MT = WTM / 32, NTL = WTN / 32;
    constexpr int AV = BM * 8 / NT;      // 16-byte vectors of the A tile per thread
    constexpr int BV = BN * 8 / NT;
    static_assert(AV * NT == BM * 8 && BV * NT == BN * 8, "tile/threads mismatch");
    constexpr int TILE_VECS = (BM + BN) * 8;
    __shared__ uint4 smem[2 * TILE_VECS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int64_t nk = Kp / BK;

    uint4 ra[AV], rb[BV];

    auto load_tile = [&](int64_t kt) {
        const int64_t k0 = kt * BK;
#pragma unroll
        for (int p = 0; p < AV; ++p) {
            const int i = tid + p * NT;
            const int row = i >> 3, c = i & 7;
            const int64_t gr = m0 + row;
            const int64_t gk = k0 + c * 16;
            ra[p] = (gr < T && gk < Ci)
                        ? *reinterpret_cast<const uint4*>(qx + gr * ldq + gk)
                        : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int p = 0; p < BV; ++p) {
            const int i = tid + p * NT;
            const int row = i >> 3, c = i & 7;
            const int64_t gn = n0 + row;
            rb[p] = (gn < Co) ? *reinterpret_cast<const uint4*>(wp + gn * Kp + k0 + c * 16)
                              : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_tile = [&](int buf) {
        uint4* sa = smem + buf * TILE_VECS;
        uint4* sb = sa + BM * 8;
#pragma unroll
        for (int p = 0; p < AV; ++p) {
            const int i = tid + p * NT;
            const int row = i >> 3, c = i & 7;
            sa[row * 8 + (c ^ swz(row))] = ra[p];
        }
#pragma unroll
        for (int p = 0; p < BV; ++p) {
            const int i = tid + p * NT;
            const int row = i >> 3, c = i & 7;
            sb[row * 8 + (c ^ swz(row))] = rb[p];
        }
    };

    v16f acc[MT][NTL];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NTL; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    if (nk > 0) {
        load_tile(0);
        store_tile(0);
        __syncthreads();
    }
    const int lr = lane & 31;
    const int lg = lane >> 5;
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = (int)(kt & 1);
        if (kt + 1 < nk) load_tile(kt + 1);
        const uint4* sa = smem + cur * TILE_VECS;
        const uint4* sb = sa + BM * 8;
#pragma unroll
        for (int s = 0; s < BK / 64; ++s) {
            const int c0 = s * 4 + lg * 2;
            v8i af[MT], bf[NTL];
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int row = wm * WTM + i * 32 + lr;
                uint4 lo = sa[row * 8 + (c0 ^ swz(row))];
                uint4 hi = sa[row * 8 + ((c0 + 1) ^ swz(row))];
                af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                            (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
#pragma unroll
            for (int j = 0; j < NTL; ++j) {
                const int row = wn * WTN + j * 32 + lr;
                uint4 lo = sb[row * 8 + (c0 ^ swz(row))];
                uint4 hi = sb[row * 8 + ((c0 + 1) ^ swz(row))];
                bf[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                            (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NTL; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        af[i], bf[j], acc[i][j], 0, 0, 0, 0, 0, 0);
        }
        if (kt + 1 < nk) store_tile(cur ^ 1);
        __syncthreads();
    }

    // Epilogue.  Accumulator element e of a 32x32 tile in lane l sits at
    // row 8*(e/4) + 4*(l/32) + e%4, column l%32.
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int j = 0; j < NTL; ++j) {
            const int64_t col = n0 + wn * WTN + j * 32 + lr;
            if (col >= Co) continue;
            const float sw = FUSED ? dw[col] : 0.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = m0 + wm * WTM + i * 32 + 8 * (e >> 2) + 4 * lg + (e & 3);
                if (row >= T) continue;
                if constexpr (FUSED) {
                    const float v = (acc[i][j][e] * dx[row]) * sw;
                    reinterpret_cast<uint16_t*>(out)[row * ldo + col] = f32_to_bf16_rne(v);
                } else {
                    reinterpret_cast<float*>(out)[row * Co + col] = acc[i][j][e];
                }
            }
        }
    }
}

// Step 2 of the two-step form: read the fp32 GEMM result back and scale.
__global__ __launch_bounds__(256) void rescale_kernel(const float* __restrict__ ws,
                                                      const float* __restrict__ dx,
                                                      const float* __restrict__ dw, int64_t T,
                                                      int64_t Co, uint16_t* __restrict__ out,
                                                      int64_t ldo) {
    const int64_t per_row = Co / 4;
    const int64_t n = T * per_row;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = i / per_row;
        const int64_t o = (i - t * per_row) * 4;
        const float4 a = *reinterpret_cast<const float4*>(ws + t * Co + o);
        const float4 s = *reinterpret_cast<const float4*>(dw + o);
        const float st = dx[t];
        uint16_t* dst = out + t * ldo + o;
        dst[0] = f32_to_bf16_rne((a.x * st) * s.x);
        dst[1] = f32_to_bf16_rne((a.y * st) * s.y);
        dst[2] = f32_to_bf16_rne((a.z * st) * s.z);
        dst[3] = f32_to_bf16_rne((a.w * st) * s.w);
    }
}

template <int BM, int BN, int WM, int WN>
static hipError_t launch_tiles(const uint8_t* qx, int64_t ldq, const float* dx, const uint8_t* wp,
                               const float* dw, int64_t T, int64_t Ci, int64_t Co, uint16_t* out,
                               int64_t ldo, float* fp32_out, hipStream_t s) {
    const dim3 grid((unsigned)((Co + BN - 1) / BN), (unsigned)((T + BM - 1) / BM));
    const int64_t Kp = round_up_k(Ci);
    if (fp32_out == nullptr) {
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, true>), grid, dim3(WM * WN * 64), 0, s,
                           qx, ldq, dx, wp, Kp, dw, T, Ci, Co, (void*)out, ldo);
    } else {
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, false>), grid, dim3(WM * WN * 64), 0, s,
                           qx, ldq, dx, wp, Kp, dw, T, Ci, Co, (void*)fp32_out, Co);
    }
    return hipGetLastError();
}

hipError_t launch_gemm(const uint8_t* qx, int64_t ldq, const float* dx, const uint8_t* wp,
                       const float* dw, int64_t T, int64_t Ci, int64_t Co, uint16_t* out,
                       int64_t ldo, float* fp32_out, hipStream_t s) {
    hipError_t e;
    if (T >= 512 && Co >= 2048)
        e = launch_tiles<256, 256, 2, 2>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s);
    else if (T > 32)
        e = launch_tiles<128, 128, 2, 2>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s);
    else
        e = launch_tiles<32, 64, 1, 2>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s);
    if (e != hipSuccess || fp32_out == nullptr) return e;
    const int64_t n = T * (Co / 4);
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(rescale_kernel, dim3((unsigned)blocks), dim3(256), 0, s, fp32_out, dx, dw,
                       T, Co, out, ldo);
    return hipGetLastError();
}

}  // namespace ptpc
