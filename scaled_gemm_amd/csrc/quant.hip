// Per-token activation quantization and per-channel weight quantization +
// prepacking for gfx950.
//
// Method: vLLM blog "PTPC-FP8: Boosting vLLM Performance on AMD ROCm",
// §PTPC: a precision-targeted scheme (one scale per token, one per weight
// column) and §Understanding the figure (Delta_X is [T x 1], Delta_W is
// [1 x Co]).  Scale = amax / 448 (1 for an all-zero vector); code =
// OCP E4M3(x / scale), round to nearest even.
//
// Both quantizers are HBM-bound streams (2 bytes read, 1 byte written per
// element).  The activation kernel keeps each row in registers between the
// amax pass and the cast, so X is read from HBM exactly once.
#include "device_common.h"
#include "kernels.h"

namespace ptpc {

// ---------------------------------------------------------------------------
// quant_act: a group of G threads owns one row; each thread holds VPT
// 16-byte vectors (8 bf16 each) of the row in registers.  Vector j of thread
// g is chunk j*G + g, so a group's loads for one j are contiguous.
// ---------------------------------------------------------------------------
// A 16-byte load with the non-temporal cache hint.
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

// 8- and 16-byte stores with the non-temporal cache hint.
__device__ __forceinline__ void store_nt(uint2* p, uint2 v) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(u32x2{v.x, v.y}, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void store_nt(uint4* p, uint4 v) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

// Loads of rows held as 8 or more vectors per thread carry the non-temporal
// hint (X is read once); measured faster there, slower for short rows.
template <int VPT>
__device__ __forceinline__ uint4 load_row_vec(const uint4* p) {
    if constexpr (VPT >= 8) {
        return load_nt(p);
    } else {
        return *p;
    }
}

template <int G, int VPT>
__global__ __launch_bounds__(256) void quant_act_kernel(
    const uint16_t* __restrict__ x, int64_t T, int64_t Ci, int64_t ldx,
    uint8_t* __restrict__ qx, int64_t ldq, float* __restrict__ dx) {
    constexpr int ROWS = 256 / G;
    __shared__ uint32_t red[256 / 64];
    const int tid = threadIdx.x;
    const int g = tid % G;
    const int64_t t = (int64_t)blockIdx.x * ROWS + tid / G;
    const bool row_ok = t < T;
    const int64_t nchunk = Ci / 8;
    const uint4* xr = reinterpret_cast<const uint4*>(x + (row_ok ? t : 0) * ldx);

    uint4 v[VPT];
    us2 m = {0, 0};
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int64_t c = (int64_t)j * G + g;
        if (row_ok && c < nchunk) {
            v[j] = load_row_vec<VPT>(xr + c);
        } else {
            v[j] = make_uint4(0, 0, 0, 0);
        }
        m = max2(m, abs_bits2(v[j].x));
        m = max2(m, abs_bits2(v[j].y));
        m = max2(m, abs_bits2(v[j].z));
        m = max2(m, abs_bits2(v[j].w));
    }
    uint32_t amax_bits;
    if constexpr (G <= 64) {
        amax_bits = group_max_u32<G>(hmax(m));
    } else {
        uint32_t w = wave_max_u32(hmax(m));
        if ((tid & 63) == 0) red[tid >> 6] = w;
        __syncthreads();
        amax_bits = 0;
#pragma unroll
        for (int i = 0; i < G / 64; ++i) {
            uint32_t o = red[(tid / G) * (G / 64) + i];
            amax_bits = amax_bits > o ? amax_bits : o;
        }
    }
    if (!row_ok) return;
    const float d = scale_from_amax(__uint_as_float(amax_bits << 16));
    const Divisor dv = make_divisor(d);
    uint2* qr = reinterpret_cast<uint2*>(qx + t * ldq);
    // Rows of 256 or more vectors (128 or 256 threads per row) store their
    // codes with the non-temporal hint: 4-8% faster with every input and
    // output streamed from HBM (rows of 4096-28672 elements); with an output
    // buffer the memory-side cache already holds, it was 0.5-4% slower.
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int64_t c = (int64_t)j * G + g;
        if (c < nchunk) {
            if constexpr (G >= 128)
                store_nt(qr + c, quantize8(v[j], dv));
            else
                qr[c] = quantize8(v[j], dv);
        }
    }
    if (g == 0) dx[t] = d;
}

// Rows longer than 256 threads x 32 vectors: amax pass, then a second read.
__global__ __launch_bounds__(256) void quant_act_long_kernel(
    const uint16_t* __restrict__ x, int64_t Ci, int64_t ldx,
    uint8_t* __restrict__ qx, int64_t ldq, float* __restrict__ dx) {
    __shared__ uint32_t red[4];
    const int tid = threadIdx.x;
    const int64_t t = blockIdx.x;
    const int64_t nchunk = Ci / 8;
    const uint4* xr = reinterpret_cast<const uint4*>(x + t * ldx);
    us2 m = {0, 0};
    for (int64_t c = tid; c < nchunk; c += 256) {
        uint4 v = xr[c];
        m = max2(m, abs_bits2(v.x));
        m = max2(m, abs_bits2(v.y));
        m = max2(m, abs_bits2(v.z));
        m = max2(m, abs_bits2(v.w));
    }
    uint32_t w = wave_max_u32(hmax(m));
    if ((tid & 63) == 0) red[tid >> 6] = w;
    __syncthreads();
    uint32_t a = red[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) a = a > red[i] ? a : red[i];
    const float d = scale_from_amax(__uint_as_float(a << 16));
    const Divisor dv = make_divisor(d);
    uint2* qr = reinterpret_cast<uint2*>(qx + t * ldq);
    for (int64_t c = tid; c < nchunk; c += 256) qr[c] = quantize8(xr[c], dv);
    if (tid == 0) dx[t] = d;
}

__global__ void fill_f32_kernel(float* __restrict__ p, int64_t n, float v) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

template <int G, int VPT>
static hipError_t launch_act(const uint16_t* x, int64_t T, int64_t Ci, int64_t ldx,
                             uint8_t* qx, int64_t ldq, float* dx, hipStream_t s) {
    constexpr int ROWS = 256 / G;
    const int64_t blocks = (T + ROWS - 1) / ROWS;
    hipLaunchKernelGGL((quant_act_kernel<G, VPT>), dim3((unsigned)blocks), dim3(256), 0, s,
                       x, T, Ci, ldx, qx, ldq, dx);
    return hipGetLastError();
}

hipError_t launch_quant_act(const uint16_t* x, int64_t T, int64_t Ci, int64_t ldx,
                            uint8_t* qx, int64_t ldq, float* dx, hipStream_t s) {
    if (Ci == 0) {
        hipLaunchKernelGGL(fill_f32_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, s,
                           dx, T, 1.0f);
        return hipGetLastError();
    }
    const ActPlan p = act_plan(Ci);
    if (p.G == 0) {
        hipLaunchKernelGGL(quant_act_long_kernel, dim3((unsigned)T), dim3(256), 0, s,
                           x, Ci, ldx, qx, ldq, dx);
        return hipGetLastError();
    }
    if (p.G == 16) {
        switch (p.vpt) {
            case 1: return launch_act<16, 1>(x, T, Ci, ldx, qx, ldq, dx, s);
            case 2: return launch_act<16, 2>(x, T, Ci, ldx, qx, ldq, dx, s);
            case 4: return launch_act<16, 4>(x, T, Ci, ldx, qx, ldq, dx, s);
            default: return launch_act<16, 8>(x, T, Ci, ldx, qx, ldq, dx, s);
        }
    }
    if (p.G == 32) return launch_act<32, 8>(x, T, Ci, ldx, qx, ldq, dx, s);
    if (p.G == 128) return launch_act<128, 8>(x, T, Ci, ldx, qx, ldq, dx, s);
    switch (p.vpt) {
        case 1: return launch_act<256, 1>(x, T, Ci, ldx, qx, ldq, dx, s);
        case 2: return launch_act<256, 2>(x, T, Ci, ldx, qx, ldq, dx, s);
        case 8: return launch_act<256, 8>(x, T, Ci, ldx, qx, ldq, dx, s);
        case 16: return launch_act<256, 16>(x, T, Ci, ldx, qx, ldq, dx, s);
        default: return launch_act<256, 32>(x, T, Ci, ldx, qx, ldq, dx, s);
    }
}

// ---------------------------------------------------------------------------
// quant_weight.  W is [Ci x Co] row-major; the per-column amax runs down the
// long K direction, so it is split over row blocks and merged with integer
// atomicMax on the fp32 bit patterns (non-negative floats order like their
// bits) held in dw; a second kernel turns amax into the scale in place; the
// third quantizes and writes the K-contiguous packed layout through an LDS
// transpose.  Both reads of W carry the non-temporal hint (measured 12%
// faster on the 70B down weight, 3-7% on the gate_up weights, level on the
// 8192 x 8192 one), and so do the packed weight's stores (another 1-5%,
// every weight and packed copy streamed from HBM).
// ---------------------------------------------------------------------------
constexpr int kColsPerBlock = 512;   // 64 lanes x 8 columns

__global__ void zero_u32_kernel(uint32_t* __restrict__ p, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

__global__ __launch_bounds__(256) void weight_colamax_kernel(
    const uint16_t* __restrict__ w, int64_t Ci, int64_t Co, int64_t ldw,
    int64_t rows_per_split, uint32_t* __restrict__ amax_bits) {
    __shared__ us2 red[4][64][4];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t col0 = (int64_t)blockIdx.x * kColsPerBlock + lane * 8;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_split;
    int64_t r1 = r0 + rows_per_split;
    if (r1 > Ci) r1 = Ci;
    us2 m0 = {0, 0}, m1 = {0, 0}, m2 = {0, 0}, m3 = {0, 0};
    if (col0 < Co) {
        // Eight rows' loads in flight per wave before their maxes; rows past
        // the split re-read its last row (the max is unchanged), so the loads
        // need no branch.
        constexpr int U = 8;
        for (int64_t r = r0 + wave; r < r1; r += 4 * U) {
            uint4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t rr = r + 4 * u < r1 ? r + 4 * u : r1 - 1;
                v[u] = load_nt(reinterpret_cast<const uint4*>(w + rr * ldw + col0));
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                m0 = max2(m0, abs_bits2(v[u].x));
                m1 = max2(m1, abs_bits2(v[u].y));
                m2 = max2(m2, abs_bits2(v[u].z));
                m3 = max2(m3, abs_bits2(v[u].w));
            }
        }
    }
    red[wave][lane][0] = m0;
    red[wave][lane][1] = m1;
    red[wave][lane][2] = m2;
    red[wave][lane][3] = m3;
    __syncthreads();
    if (wave == 0 && col0 < Co) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            us2 a = max2(max2(red[0][lane][q], red[1][lane][q]), max2(red[2][lane][q], red[3][lane][q]));
            if (a.x) atomicMax(amax_bits + col0 + 2 * q, (uint32_t)a.x << 16);
            if (a.y) atomicMax(amax_bits + col0 + 2 * q + 1, (uint32_t)a.y << 16);
        }
    }
}

__global__ void weight_scale_kernel(float* __restrict__ dw, int64_t Co) {
    int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (o < Co) dw[o] = scale_from_amax(dw[o]);
}

// Packed weight layout (what the GEMM streams): 1 KB blocks of 16 columns x
// 64 K bytes, block (g, s) at byte ((g * Kp/64) + s) * 1024.  Inside a block
// the 16-byte unit u holds column 16g + u/4, K bytes 64s + 16c .. +15 with
// c = (u % 4) ^ ((u / 16) % 4): the GEMM's LDS row order with its bank
// swizzle already applied, so one load instruction copies a block verbatim.
__device__ __forceinline__ int pack_chunk_of_unit(int u) { return (u & 3) ^ ((u >> 4) & 3); }

// Tile: 128 rows of K x 64 columns.  Each thread loads 16 bytes (8 columns)
// of one row per pass, quantizes them with its 8 column divisors and drops
// the codes transposed into LDS; the tile then leaves as 8 packed blocks.
constexpr int kPackK = 128;
constexpr int kPackN = 64;
constexpr int kPackPitch = kPackK + 16;   // keeps 16-byte alignment of rows

// dw_step = 1: column o uses dw[o] (per-channel); 0: every column uses dw[0]
// (per-tensor).
__global__ __launch_bounds__(256) void weight_pack_kernel(
    const uint16_t* __restrict__ w, int64_t Ci, int64_t Co, int64_t ldw,
    const float* __restrict__ dw, int64_t dw_step, uint8_t* __restrict__ packed, int64_t Kp) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[kPackN * kPackPitch];
    const int tid = threadIdx.x;
    const int cg = tid & 7;            // 8-column group within the tile
    const int rr = tid >> 3;           // row within a 32-row pass
    const int64_t o0 = (int64_t)blockIdx.x * kPackN;
    const int64_t k0 = (int64_t)blockIdx.y * kPackK;
    const int64_t col = o0 + cg * 8;
    const bool col_ok = col < Co;      // Co % 16 == 0: 8-column groups are whole

    Divisor dv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float d = dw[(col_ok ? col + j : 0) * dw_step];   // in bounds, no branch
        dv[j] = make_divisor(col_ok ? d : 1.0f);
    }

    // All four rows' loads are issued before any is used: rows past Ci and
    // columns past Co read a valid element (clamped address) and are then
    // replaced by zero, so the loads need no branch.
    uint4 vin[kPackK / 32];
#pragma unroll
    for (int p = 0; p < kPackK / 32; ++p) {
        const int64_t k = k0 + p * 32 + rr;
        const int64_t kc = k < Ci ? k : Ci - 1;
        vin[p] = load_nt(reinterpret_cast<const uint4*>(w + kc * ldw + (col_ok ? col : 0)));
    }
#pragma unroll
    for (int p = 0; p < kPackK / 32; ++p) {
        const int kl = p * 32 + rr;
        const int64_t k = k0 + kl;
        const uint4 v = (col_ok && k < Ci) ? vin[p] : make_uint4(0, 0, 0, 0);
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            uint32_t c = cvt_e4m3x2<false>(sat448(divide(bf16lo_to_f32(wd[h]), dv[2 * h])),
                                           sat448(divide(bf16hi_to_f32(wd[h]), dv[2 * h + 1])),
                                           0u);
            tile[(cg * 8 + 2 * h) * kPackPitch + kl] = (uint8_t)(c & 0xFF);
            tile[(cg * 8 + 2 * h + 1) * kPackPitch + kl] = (uint8_t)((c >> 8) & 0xFF);
        }
    }
    __syncthreads();
    // 4 column groups x 2 K steps = 8 blocks = 512 units of 16 bytes.
    const int64_t kblocks = Kp / 64;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int i = p * 256 + tid;
        const int b = i >> 6, u = i & 63;
        const int g = b >> 1, ks = b & 1;
        const int n = g * 16 + (u >> 2);
        if (o0 + n < Co) {
            const uint4 val = *reinterpret_cast<const uint4*>(
                tile + n * kPackPitch + ks * 64 + pack_chunk_of_unit(u) * 16);
            const int64_t blk = ((o0 >> 4) + g) * kblocks + (k0 >> 6) + ks;
            store_nt(reinterpret_cast<uint4*>(packed + blk * 1024 + u * 16), val);
        }
    }
}

hipError_t launch_quant_weight(const uint16_t* w, int64_t Ci, int64_t Co, int64_t ldw,
                               uint8_t* packed, float* dw, hipStream_t s) {
    const int64_t Kp = round_up_k(Ci);
    uint32_t* amax_bits = reinterpret_cast<uint32_t*>(dw);
    hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((Co + 255) / 256)), dim3(256), 0, s,
                       amax_bits, Co);
    if (Ci > 0) {
        const int64_t colblocks = (Co + kColsPerBlock - 1) / kColsPerBlock;
        // About 256 workgroups in all (one per CU): fewer, longer row splits
        // than 2048 were 6-12% faster over the whole weight quantization
        // (fewer atomics per column, less tail); 128 was slower again.
        int64_t splits = 256 / colblocks;
        if (splits < 1) splits = 1;
        int64_t max_splits = (Ci + 31) / 32;    // at least 32 rows per split
        if (splits > max_splits) splits = max_splits;
        if (splits > 65535) splits = 65535;
        int64_t rows_per_split = (Ci + splits - 1) / splits;
        rows_per_split = (rows_per_split + 3) / 4 * 4;
        splits = (Ci + rows_per_split - 1) / rows_per_split;
        hipLaunchKernelGGL(weight_colamax_kernel, dim3((unsigned)colblocks, (unsigned)splits),
                           dim3(256), 0, s, w, Ci, Co, ldw, rows_per_split, amax_bits);
    }
    hipLaunchKernelGGL(weight_scale_kernel, dim3((unsigned)((Co + 255) / 256)), dim3(256), 0, s,
                       dw, Co);
    if (Kp > 0) {
        hipLaunchKernelGGL(weight_pack_kernel,
                           dim3((unsigned)((Co + kPackN - 1) / kPackN), (unsigned)(Kp / kPackK)),
                           dim3(256), 0, s, w, Ci, Co, ldw, dw, (int64_t)1, packed, Kp);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-tensor ("standard") FP8, the comparator: one scale for a whole matrix.
// The amax pass gives each wave whole rows (16-byte loads along the row),
// reduces the workgroup in LDS and merges workgroups with one integer
// atomicMax on the fp32 bit pattern; the scale kernel then converts it in
// place.  The static casts are plain streams with a scalar divisor.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tensor_amax_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t C, int64_t ld, int64_t rows_per_block,
    uint32_t* __restrict__ amax_bits) {
    __shared__ uint32_t red[4];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t nvec = C / 8;
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
    int64_t r1 = r0 + rows_per_block;
    if (r1 > R) r1 = R;
    us2 m = {0, 0};
    for (int64_t r = r0 + wave; r < r1; r += 4) {
        const uint4* xr = reinterpret_cast<const uint4*>(x + r * ld);
        for (int64_t c = lane; c < nvec; c += 64) {
            const uint4 v = xr[c];
            m = max2(m, abs_bits2(v.x));
            m = max2(m, abs_bits2(v.y));
            m = max2(m, abs_bits2(v.z));
            m = max2(m, abs_bits2(v.w));
        }
    }
    const uint32_t w = wave_max_u32(hmax(m));
    if (lane == 0) red[wave] = w;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t a = red[0];
#pragma unroll
        for (int i = 1; i < 4; ++i) a = a > red[i] ? a : red[i];
        if (a) atomicMax(amax_bits, a << 16);
    }
}

// code = E4M3(x / d[0]) for an R x C bf16 matrix, row pitches ld / ldq.
__global__ __launch_bounds__(256) void quant_static_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t C, int64_t ld,
    const float* __restrict__ d, uint8_t* __restrict__ q, int64_t ldq, int64_t rows_per_block) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t nvec = C / 8;
    const Divisor dv = make_divisor(d[0]);
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
    int64_t r1 = r0 + rows_per_block;
    if (r1 > R) r1 = R;
    for (int64_t r = r0 + wave; r < r1; r += 4) {
        const uint4* xr = reinterpret_cast<const uint4*>(x + r * ld);
        uint2* qr = reinterpret_cast<uint2*>(q + r * ldq);
        for (int64_t c = lane; c < nvec; c += 64) qr[c] = quantize8<true>(xr[c], dv);
    }
}

// Rows per workgroup for the row-streaming kernels: about 2048 workgroups,
// at least 4 rows (one per wave).
static int64_t rows_per_block_for(int64_t R) {
    int64_t rpb = (R + 2047) / 2048;
    if (rpb < 4) rpb = 4;
    return rpb;
}

hipError_t launch_tensor_scale(const uint16_t* x, int64_t R, int64_t C, int64_t ld, float* d,
                               hipStream_t s) {
    uint32_t* amax_bits = reinterpret_cast<uint32_t*>(d);
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, s, amax_bits, (int64_t)1);
    if (R > 0 && C > 0) {
        const int64_t rpb = rows_per_block_for(R);
        hipLaunchKernelGGL(tensor_amax_kernel, dim3((unsigned)((R + rpb - 1) / rpb)), dim3(256),
                           0, s, x, R, C, ld, rpb, amax_bits);
    }
    hipLaunchKernelGGL(weight_scale_kernel, dim3(1), dim3(64), 0, s, d, (int64_t)1);
    return hipGetLastError();
}

hipError_t launch_quant_act_static(const uint16_t* x, int64_t T, int64_t Ci, int64_t ldx,
                                   const float* d, uint8_t* qx, int64_t ldq, hipStream_t s) {
    const int64_t rpb = rows_per_block_for(T);
    hipLaunchKernelGGL(quant_static_kernel, dim3((unsigned)((T + rpb - 1) / rpb)), dim3(256), 0,
                       s, x, T, Ci, ldx, d, qx, ldq, rpb);
    return hipGetLastError();
}

hipError_t launch_quant_weight_static(const uint16_t* w, int64_t Ci, int64_t Co, int64_t ldw,
                                      const float* d, uint8_t* packed, hipStream_t s) {
    const int64_t Kp = round_up_k(Ci);
    hipLaunchKernelGGL(weight_pack_kernel,
                       dim3((unsigned)((Co + kPackN - 1) / kPackN), (unsigned)(Kp / kPackK)),
                       dim3(256), 0, s, w, Ci, Co, ldw, d, (int64_t)0, packed, Kp);
    return hipGetLastError();
}

__global__ void unpack_kernel(const uint8_t* __restrict__ packed, int64_t Ci, int64_t Co,
                              int64_t Kp, uint8_t* __restrict__ qw) {
    const int64_t n = Ci * Co;
    const int64_t kblocks = Kp / 64;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t k = i / Co, o = i - k * Co;
        const int row = (int)(o & 15), chunk = (int)((k & 63) >> 4);
        const int u = row * 4 + (chunk ^ ((row >> 2) & 3));    // inverse of the packing
        const int64_t blk = (o >> 4) * kblocks + (k >> 6);
        qw[i] = packed[blk * 1024 + u * 16 + (k & 15)];
    }
}

hipError_t launch_unpack_weight(const uint8_t* packed, int64_t Ci, int64_t Co, uint8_t* qw,
                                hipStream_t s) {
    const int64_t n = Ci * Co;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)blocks), dim3(256), 0, s, packed, Ci, Co,
                       round_up_k(Ci), qw);
    return hipGetLastError();
}

}  // namespace ptpc
