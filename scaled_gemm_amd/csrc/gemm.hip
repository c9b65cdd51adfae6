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
// Data layout: qx is [T x Ci] row-major (K contiguous).  The packed weight
// is a sequence of 1 KB blocks, [Co/16][Kp/64] of them (Kp = roundup(Ci,
// 128), zero codes past Ci): block (g, s) holds columns 16g..16g+15 for K
// bytes 64s..64s+63, laid out exactly as one load instruction drops it into
// LDS (16 rows of 64 bytes, chunks in swizzled slots), so B tiles stream as
// contiguous 1 KB reads.  In LDS both operands are "rows of 64 K bytes" and
// both MFMA operands are read the same way: lane l takes row l % 32 of a
// 32-row slab and 32 consecutive K bytes starting at 32 * (l / 32).
//
// Pipeline: tiles move HBM/L2 -> LDS with buffer_load_dwordx4 ... lds (no
// staging registers, no ds_write); the buffer descriptor's range check
// turns rows past T / Co and K past Ci into zeros.  LDS holds two stages;
// while the MFMAs consume stage k, the loads for stage k+1 are in flight.
// One LDS row is 128 bytes = 8 chunks of 16 bytes; chunk c of row r is
// stored at slot c ^ swz(r), so the 32 rows an operand read touches spread
// over the banks.  A load instruction fills 1 KB of LDS (64 lanes x 16 B,
// i.e. 8 rows), so each lane fetches the global chunk that belongs in its
// fixed LDS slot.
#include "device_common.h"
#include "kernels.h"

namespace ptpc {

#ifndef PTPC_NSTAGE
#define PTPC_NSTAGE 4
#endif

constexpr int BK = 64;          // K bytes per pipeline stage (one MFMA K step)
constexpr int kBufferDword3 = 0x00020000;   // raw buffer, 32-bit data format
constexpr uint32_t kOutOfRange = 0x80000000u;

// Chunk slot of logical 16-byte chunk c in LDS row r.  A row is 64 bytes
// (4 chunks); an operand read has 16 consecutive rows of one logical chunk in
// flight per LDS cycle on the 64-bank LDS, and rows r, r+4, r+8, r+12 share
// banks unless their slots differ.
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kBufferDword3);
}

// Workgroup barrier without the release/acquire fences of __syncthreads():
// the fence would wait for every load in flight into LDS (vmcnt 0), which
// would drain the prefetch ring.  Callers wait for exactly the fills they
// need with wait_counts first; the memory clobber keeps the compiler from
// moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt with vmcnt <= VM and lgkmcnt <= LGKM (expcnt not waited on).
template <int VM, int LGKM>
__device__ __forceinline__ void wait_counts() {
    static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "waitcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8));
}

template <int BM, int BN, int WM, int WN, int NSTAGE, bool FUSED>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_kernel(
    const uint8_t* __restrict__ qx, int64_t ldq, const float* __restrict__ dx,
    const uint8_t* __restrict__ wp, int64_t Kp, const float* __restrict__ dw,
    int64_t T, int64_t Ci, int64_t Co, void* __restrict__ out, int64_t ldo) {
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int MT = WTM / 32, NTL = WTN / 32;
    constexpr int ROWS_PER_BLK = 1024 / BK;                   // rows one load instruction fills
    constexpr int A_BLK = BM / ROWS_PER_BLK, B_BLK = BN / ROWS_PER_BLK;
    constexpr int A_PER_W = A_BLK / NW, B_PER_W = B_BLK / NW;
    constexpr int DPW = A_PER_W + B_PER_W;                    // load instructions per wave per stage
    static_assert(A_PER_W * NW == A_BLK && B_PER_W * NW == B_BLK, "tile/waves mismatch");
    static_assert(2 * DPW < 64, "vmcnt range");
    constexpr int A_BYTES = BM * BK;
    constexpr int STAGE = (BM + BN) * BK;
    // Distinct LDS objects per stage (not one array indexed by stage) so
    // that the compiler can tell the stage being filled from the stage being
    // read and does not wait for the fills before the reads.
    static_assert(NSTAGE >= 2 && NSTAGE <= 5, "ring depth");
    __shared__ __attribute__((aligned(1024))) uint8_t stage0[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t stage1[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t stage2[NSTAGE > 2 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t stage3[NSTAGE > 3 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t stage4[NSTAGE > 4 ? STAGE : 16];
    uint8_t* const stages[5] = {stage0, stage1, stage2, stage3, stage4};

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wm = wave / WN, wn = wave % WN;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int nks = (int)(Kp / BK);                           // K steps with data

    // Buffer descriptors based at this tile's first row; rows past the end
    // and K past the data land beyond num_records and read as zero.
    const int64_t a_rows = (T - m0 < BM) ? (T - m0) : BM;
    const int64_t b_rows = (Co - n0 < BN) ? (Co - n0) : BN;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(qx + m0 * ldq, (uint32_t)(a_rows * ldq));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(wp + n0 * Kp, (uint32_t)(b_rows * Kp));

    // A load instruction fills ROWS_PER_BLK rows: lane L owns LDS row L/4,
    // slot L%4, and fetches the logical chunk that belongs in that slot.
    const int lrow = lane >> 2;
    const int slot = lane & 3;
    uint32_t a_off[A_PER_W], b_off[B_PER_W];
    int a_chunk[A_PER_W];
#pragma unroll
    for (int p = 0; p < A_PER_W; ++p) {
        const int r = (wave + p * NW) * ROWS_PER_BLK + lrow;
        const int c = slot ^ swz(r);
        a_chunk[p] = c;
        a_off[p] = (r < a_rows) ? (uint32_t)(r * ldq + c * 16) : kOutOfRange;
    }
    // The packed weight is already in LDS order: 1 KB blocks of 16 columns x
    // one 64-byte K step, lane L's 16 bytes at L*16 (see the packing kernel).
    const int kblocks = (int)(Kp / BK);
#pragma unroll
    for (int p = 0; p < B_PER_W; ++p) {
        const int blk = wave + p * NW;                      // 16-column group in the tile
        b_off[p] = (blk * ROWS_PER_BLK < b_rows) ? (uint32_t)(blk * kblocks * 1024 + lane * 16)
                                                 : kOutOfRange;
    }

    auto issue_stage = [&](int ks, uint8_t* sa) {
        const int k0 = ks * BK;
        uint8_t* sb = sa + A_BYTES;
#pragma unroll
        for (int p = 0; p < A_PER_W; ++p) {
            const bool kin = (int64_t)(k0 + a_chunk[p] * 16) < Ci;
            const uint32_t off = (a_off[p] != kOutOfRange && kin) ? a_off[p] + k0 : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (lds_ptr_t)(sa + (wave + p * NW) * 1024), 16, off, 0, 0, 0);
        }
        const bool kin_b = k0 < Kp;
#pragma unroll
        for (int p = 0; p < B_PER_W; ++p) {
            const uint32_t off =
                (b_off[p] != kOutOfRange && kin_b) ? b_off[p] + (uint32_t)ks * 1024u : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (lds_ptr_t)(sb + (wave + p * NW) * 1024), 16, off, 0, 0, 0);
        }
    };

    v16f acc[MT][NTL];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NTL; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int lr = lane & 31;
    const int lg = lane >> 5;
    // MFMA operands: lane l reads row l%32 of a 32-row slab, logical chunks
    // 2*(l/32) and 2*(l/32)+1 of the 64-byte K step.
    int a_lo[MT], a_hi[MT], b_lo[NTL], b_hi[NTL];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int r = wm * WTM + i * 32 + lr;
        a_lo[i] = r * BK + (((2 * lg) ^ swz(r)) << 4);
        a_hi[i] = r * BK + (((2 * lg + 1) ^ swz(r)) << 4);
    }
#pragma unroll
    for (int j = 0; j < NTL; ++j) {
        const int r = wn * WTN + j * 32 + lr;
        b_lo[j] = A_BYTES + r * BK + (((2 * lg) ^ swz(r)) << 4);
        b_hi[j] = A_BYTES + r * BK + (((2 * lg + 1) ^ swz(r)) << 4);
    }
    auto read_frags = [&](const uint8_t* st, v8i (&a)[MT], v8i (&b)[NTL]) {
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const uint4 lo = *reinterpret_cast<const uint4*>(st + a_lo[i]);
            const uint4 hi = *reinterpret_cast<const uint4*>(st + a_hi[i]);
            a[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int j = 0; j < NTL; ++j) {
            const uint4 lo = *reinterpret_cast<const uint4*>(st + b_lo[j]);
            const uint4 hi = *reinterpret_cast<const uint4*>(st + b_hi[j]);
            b[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
    };
    // One K step: its MFMAs, with the next step's operand reads and the
    // loads that refill the just-freed stage threaded between them (the
    // reads fill the other fragment registers).  Issuing the loads in one
    // burst would hold back the first MFMA until the texture unit accepted
    // them all.
    constexpr int NMFMA = MT * NTL;
    constexpr int NREAD = 2 * (MT + NTL);
    auto step = [&](int s, const v8i (&a)[MT], const v8i (&b)[NTL], const uint8_t* nxt,
                    v8i (&na)[MT], v8i (&nb)[NTL], uint8_t* refill) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NTL; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    b[j], a[i], acc[i][j], 0, 0, 0, 0, 0, 0);
        read_frags(nxt, na, nb);
        issue_stage(s + NSTAGE, refill);
        constexpr int NQ = NMFMA > NREAD ? NMFMA : NREAD;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if (q < NMFMA) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            if (q < NREAD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
            if (q < DPW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // VMEM read
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // Top of K step s: the stage s+1 fill has landed (the fills of the
    // NSTAGE-2 later steps may still be in flight) and every wave has read
    // stage s into registers, so stage s%NSTAGE is free for the fill of step
    // s+NSTAGE (issued inside step s).
    auto top = [&]() {
        wait_counts<(NSTAGE - 2) * DPW, 0>();
        lds_barrier();
    };

    // Ring of NSTAGE stages; K steps past the data are filled with zeros
    // (every offset out of range) so the loop needs no branch; fewer than
    // U extra zero steps are multiplied.  The loop is unrolled so that every
    // access names its stage and fragment set statically.
    constexpr int U = (NSTAGE % 2) ? 2 * NSTAGE : NSTAGE;
    v8i fr_a[2][MT], fr_b[2][NTL];
    if (nks > 0) {
#pragma unroll
        for (int u = 0; u < NSTAGE; ++u) issue_stage(u, stages[u]);
        wait_counts<(NSTAGE - 1) * DPW, 15>();   // stage 0 landed
        lds_barrier();
        read_frags(stage0, fr_a[0], fr_b[0]);
        for (int s = 0; s < nks; s += U) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                top();
                step(s + u, fr_a[u & 1], fr_b[u & 1], stages[(u + 1) % NSTAGE],
                     fr_a[(u + 1) & 1], fr_b[(u + 1) & 1], stages[u % NSTAGE]);
            }
        }
        wait_counts<0, 0>();            // no fill may land after the loop
        lds_barrier();
    }

    // Epilogue.  The weight slab is the MFMA's first operand, so the 32x32
    // accumulator tile is out^T: in lane l, element e holds output row
    // (token) l%32 of the slab and output column 8*(e/4) + 4*(l/32) + e%4.
    // Each lane therefore owns runs of 4 consecutive columns of one row:
    // 8-byte bf16 stores (16-byte fp32 stores in the two-step form).
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int64_t row = m0 + wm * WTM + i * 32 + lr;
        if (row >= T) continue;
        const float sx = FUSED ? dx[row] : 0.0f;
#pragma unroll
        for (int j = 0; j < NTL; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t col = n0 + wn * WTN + j * 32 + 8 * g + 4 * lg;
                if (col >= Co) continue;                  // Co % 16 == 0: runs are whole
                const float a0 = acc[i][j][4 * g + 0], a1 = acc[i][j][4 * g + 1];
                const float a2 = acc[i][j][4 * g + 2], a3 = acc[i][j][4 * g + 3];
                if constexpr (FUSED) {
                    const float4 sw = *reinterpret_cast<const float4*>(dw + col);
                    uint2 pk;
                    pk.x = (uint32_t)f32_to_bf16_rne((a0 * sx) * sw.x) |
                           ((uint32_t)f32_to_bf16_rne((a1 * sx) * sw.y) << 16);
                    pk.y = (uint32_t)f32_to_bf16_rne((a2 * sx) * sw.z) |
                           ((uint32_t)f32_to_bf16_rne((a3 * sx) * sw.w) << 16);
                    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + row * ldo + col) =
                        pk;
                } else {
                    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + row * Co + col) =
                        make_float4(a0, a1, a2, a3);
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
        uint2 packed;
        packed.x = (uint32_t)f32_to_bf16_rne((a.x * st) * s.x) |
                   ((uint32_t)f32_to_bf16_rne((a.y * st) * s.y) << 16);
        packed.y = (uint32_t)f32_to_bf16_rne((a.z * st) * s.z) |
                   ((uint32_t)f32_to_bf16_rne((a.w * st) * s.w) << 16);
        *reinterpret_cast<uint2*>(out + t * ldo + o) = packed;
    }
}

template <int BM, int BN, int WM, int WN, int NS>
static hipError_t launch_tiles(const uint8_t* qx, int64_t ldq, const float* dx, const uint8_t* wp,
                               const float* dw, int64_t T, int64_t Ci, int64_t Co, uint16_t* out,
                               int64_t ldo, float* fp32_out, hipStream_t s) {
    const dim3 grid((unsigned)((Co + BN - 1) / BN), (unsigned)((T + BM - 1) / BM));
    const int64_t Kp = round_up_k(Ci);
    if (fp32_out == nullptr) {
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, NS, true>), grid, dim3(WM * WN * 64), 0, s,
                           qx, ldq, dx, wp, Kp, dw, T, Ci, Co, (void*)out, ldo);
    } else {
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, NS, false>), grid, dim3(WM * WN * 64), 0, s,
                           qx, ldq, dx, wp, Kp, dw, T, Ci, Co, (void*)fp32_out, Co);
    }
    return hipGetLastError();
}

hipError_t launch_gemm(const uint8_t* qx, int64_t ldq, const float* dx, const uint8_t* wp,
                       const float* dw, int64_t T, int64_t Ci, int64_t Co, uint16_t* out,
                       int64_t ldo, float* fp32_out, hipStream_t s) {
    hipError_t e;
    if (T >= 512 && Co >= 2048)
        e = launch_tiles<256, 256, 2, 2, PTPC_NSTAGE>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s);
    else if (T > 32)
        e = launch_tiles<128, 128, 2, 2, 4>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s);
    else
        e = launch_tiles<32, 64, 1, 2, 4>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s);
    if (e != hipSuccess || fp32_out == nullptr) return e;
    const int64_t n = T * (Co / 4);
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(rescale_kernel, dim3((unsigned)blocks), dim3(256), 0, s, fp32_out, dx, dw,
                       T, Co, out, ldo);
    return hipGetLastError();
}

}  // namespace ptpc
