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
// in v_mfma_f32_16x16x128_f8f6f4 (gemm16_kernel, gemm16s_kernel) or
// v_mfma_f32_32x32x64_f8f6f4 (the other kernels).
//
// Data layout: qx is [T x Ci] row-major (K contiguous).  The packed weight
// is a sequence of 1 KB blocks, [Co/16][Kp/64] of them (Kp = roundup(Ci,
// 128), zero codes past Ci): block (g, s) holds columns 16g..16g+15 for K
// bytes 64s..64s+63, laid out exactly as one load instruction drops it into
// LDS (16 rows of 64 bytes, chunks in swizzled slots), so B tiles stream as
// contiguous 1 KB reads.  In LDS both operands are "rows of 64 K bytes" and
// both MFMA operands are read the same way: lane l takes row l % 32 of a
// 32-row slab and 32 consecutive K bytes starting at 32 * (l / 32) of a
// 64-byte step (32x32x64), or row l % 16 of a 16-row slab and K bytes
// 32 * (l / 16) .. +31 of a 128-byte step (16x16x128).
//
// Pipeline (details above gemm_kernel): operand tiles move HBM/L2 -> LDS
// with buffer_load_dwordx4 ... lds (no staging registers, no ds_write); the
// buffer descriptor's range check turns rows past T / Co and K past Ci into
// zeros.  LDS holds a ring of A and B slots several K steps deep.  Within an
// LDS row, 16-byte chunk c of row r is stored at slot c ^ swz(r), so the 32
// rows an operand read touches spread over the banks; a load instruction
// fills 1 KB of LDS (64 lanes x 16 B), each lane fetching the global chunk
// that belongs in its fixed LDS slot.
//
// Kernels: gemm16_kernel (tiled, 128..256-row x 128..256-column tiles,
// 16x16x128 MFMAs; also the two-range split of 256x256 tiles, joined inside
// the kernel), gemm16s_kernel (64x64 tiles of 65..128 tokens, the K
// steps split between the waves, each on its own LDS ring), gemm_kernel
// (tiled, 32x64 and 64-row tiles -- also from 256 tokens where 128x128 tiles
// would leave CUs idle -- and the split-K form, 32x32x64 MFMAs),
// gemm_decode_kernel (up to 64 tokens: K split across the waves of a
// workgroup, operands loaded straight into registers), and the second
// passes of the two-step forms and of split-K with more than two ranges.
#include <mutex>
#include <utility>

#include "device_common.h"
#include "kernels.h"

namespace ptpc {

constexpr int BK = 64;          // K bytes per step (one MFMA K step)
constexpr uint32_t kOutOfRange = 0x80000000u;
// Bound on the sleeps of the two-range fix-up's wait (gemm16_kernel): about
// 2^20 x 64 clocks, far beyond the microseconds the other range needs to
// publish its sums.  The lost-flag debug build (-DPTPC_JOIN_LOST,
// libptpc_join_lost.so) never raises the flag and waits 16 sleeps, so that
// every joined tile takes the path of a wait that runs out.
#ifdef PTPC_JOIN_LOST
constexpr int kFixupSpins = 16;
constexpr bool kRaiseJoinFlag = false;
#else
constexpr int kFixupSpins = 1 << 20;
constexpr bool kRaiseJoinFlag = true;
#endif
// Cache-policy bits of a buffer load: sc1, device-coherent (reads memory,
// not a stale line of this XCD's L2).
constexpr int kSc1 = 16;

// LDS bank swizzles (64 banks of 4 bytes; an operand read has 16 consecutive
// rows of one logical 16-byte chunk in flight per LDS cycle).
//   B rows are 64 bytes (4 chunks): rows r, r+4, r+8, r+12 share banks
//   unless their slots differ -> slot = c ^ ((r >> 2) & 3).
//   A rows are 128 bytes (8 chunks, two K steps): rows r and r+2 share
//   banks unless their slots differ -> slot = c ^ ((r >> 1) & 7).
__device__ __forceinline__ int swz_b(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int swz_a(int row) { return (row >> 1) & 7; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Scales the fused epilogue applies: per token and per output column (the
// method), one scalar each (the per-tensor comparator), or none (step 1 of
// the bf16-intermediate two-step form: acc rounded to bf16 unscaled).
constexpr int kTokenChannelScales = 0;
constexpr int kTensorScales = 1;
constexpr int kUnitScales = 2;

__device__ __forceinline__ float4 scale_of_cols(const float* dw, int64_t col, int mode) {
    if (mode == kTokenChannelScales) return *reinterpret_cast<const float4*>(dw + col);
    const float v = (mode == kTensorScales) ? dw[0] : 1.0f;
    return make_float4(v, v, v, v);
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

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

// LDS-poison debug build (-DPTPC_LDS_POISON, libptpc_lds_poison.so): right
// before a wave issues the fills that refill an LDS region, it overwrites the
// region with 0x7F bytes -- NaN as E4M3 -- and waits for those writes.  The
// pipelines below issue a fill only once every wave's last read of the region
// is done (behind a barrier, or the wave's own wait where a wave owns its
// slots); a read that came too late, or one that came before its fill
// landed, would now see NaN and turn the outputs it feeds into NaN, whatever
// the data.  The parity tests compare the two builds bit for bit.
#ifdef PTPC_LDS_POISON
constexpr bool kLdsPoison = true;
#else
constexpr bool kLdsPoison = false;
#endif
__device__ __forceinline__ void poison_block(uint8_t* blk) {
    const uint32_t nan4 = 0x7F7F7F7Fu;
    *reinterpret_cast<uint4*>(blk + (threadIdx.x & 63) * 16) = make_uint4(nan4, nan4, nan4, nan4);
}
__device__ __forceinline__ void poison_done() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Timeline debug build (-DPTPC_TIMELINE, libptpc_timeline.so): wave 0 of
// every workgroup of gemm16_kernel records the GPU's constant 100 MHz clock
// (s_memrealtime) at four points -- start, K loop entered (first operands
// landed), K loop done, last output store completed -- into the buffer set
// with ptpc_debug_set_timeline ([workgroups][4] uint64, or NULL for none).
#ifdef PTPC_TIMELINE
__device__ unsigned long long* g_timeline = nullptr;
#endif
__device__ __forceinline__ void timeline_mark(int k) {
#ifdef PTPC_TIMELINE
    if (k == 3) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (threadIdx.x == 0 && g_timeline != nullptr)
        g_timeline[(size_t)blockIdx.x * 4 + k] = __builtin_amdgcn_s_memrealtime();
#else
    (void)k;
#endif
}

// Tile order.  Workgroups are dealt round-robin to the 8 XCDs, each with its
// own L2.  The linear id is remapped so that XCD x owns a contiguous chunk of
// the logical order, and the logical order walks groups of kGroupN column
// blocks, every row block of a group before the next group: a weight block
// is streamed from HBM once, the activation blocks re-read per group stay in
// the MALL, and the 32 tiles an XCD holds at once (4 row x 8 column blocks)
// share 12 operand blocks per K step.
constexpr int kXcds = 8;
constexpr int kGroupN = 8;
// Tiles of fewer than 256 rows and 256 columns (128x256, 192x256: the
// one-round grids of 1024-token layers) walk groups of 4 columns instead:
// at 1024 tokens an XCD then holds 8 row x 4 column tiles of 128x256, 256 KB
// of distinct operand bytes per K step instead of 320 KB (the 70B O / QKV /
// down layers at 1024 tokens 1-2% faster; on 256x224 and 256x256 tiles groups
// of 4 were level or up to 1% slower).
template <int BM, int BN>
constexpr int group_n_of() { return BM < 256 && BN == 256 ? 4 : kGroupN; }
__device__ __forceinline__ void tile_group_of(int i, int gm, int gn, int& tm, int& tn,
                                              int group_n = kGroupN) {
    const int group = i / (group_n * gm);
    const int first_n = group * group_n;
    const int width = (gn - first_n < group_n) ? gn - first_n : group_n;
    const int r = i - group * group_n * gm;
    // The divisions run on the vector ALU; say that the results are the same
    // in every lane so that the buffer descriptors built from them stay
    // scalar (a descriptor in vector registers costs a loop per load).
    tm = __builtin_amdgcn_readfirstlane(r / width);
    tn = __builtin_amdgcn_readfirstlane(first_n + r % width);
}
__device__ __forceinline__ void tile_of(int i, int gm, int gn, int& tm, int& tn) {
    const int n = gm * gn;
    if (n % kXcds == 0) i = (i % kXcds) * (n / kXcds) + i / kXcds;
    tile_group_of(i, gm, gn, tm, tn);
}
// Split-K grids of the 16x16x128 kernel (S K ranges of every tile): the XCD
// remap runs over all S x tiles workgroups, range-major, so that an XCD's
// share is a run of consecutive tiles of one K range, grouped as in an
// unsplit grid (range-minor, an XCD held tiles of every range, which share
// no operand blocks: the 70B down projection at 512 / 1024 tokens, 4 / 2
// ranges, ran 11% / 3% slower).  S = 1 gives tile_of's mapping.  Returns the
// range; `tile` gets the tile's index in the group order.
__device__ __forceinline__ int split_of(int b, int splits, int ntiles, int& tile) {
    const int total = ntiles * splits;
    int L = b;
    if (total % kXcds == 0) L = (b % kXcds) * (total / kXcds) + b / kXcds;
    const int split = __builtin_amdgcn_readfirstlane(L / ntiles);
    tile = __builtin_amdgcn_readfirstlane(L - split * ntiles);
    return split;
}

// The pipeline.  K advances in 64-byte steps; each step is one MFMA K
// step for every accumulator tile.
//   A (token rows of qx, row-major in HBM) is staged in "pair slots": one
//   slot holds two consecutive K steps as 128-byte LDS rows, so every A load
//   fetches whole 128-byte lines.  Three pair slots.
//   B (the packed weight) is staged one step per slot, NB slots of 64-byte
//   rows, filled by verbatim 1 KB block copies.
// Each step issues the same number of loads: the B fill for step s+NB and
// half (by rows) of the A pair that is two pairs ahead: at an even step s the
// second half of pair (s+4, s+5), at an odd step s the first half of pair
// (s+5, s+6).  At the top of step t the fills read during step t (operands
// of step t+1) were issued at the top of step t-2 or earlier (t+1-NB or
// earlier for B), so with uniform issue counts one "vmcnt <= loads issued
// in the last NB-2 steps" wait covers both.
// NTB: the B fills carry the non-temporal cache hint.  Used where every
// weight byte is read by one workgroup only (one row tile) -- up to 64
// tokens, and the split-K ranges of long K: 11-13% faster on the 70B gate_up
// layer at 16-64 tokens and 7% on the split 70B down projection at 72-128
// tokens; where row tiles share the weight, or the split ranges are short
// (K = 8192), it was level or up to 5% slower.
template <int BM, int BN, int WM, int WN, int NB, bool FUSED, bool NTB>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_kernel(
    const uint8_t* __restrict__ qx, int64_t ldq, const float* __restrict__ dx,
    const uint8_t* __restrict__ wp, int64_t Kp, const float* __restrict__ dw,
    int64_t T, int64_t Ci, int64_t Co, void* __restrict__ out, int64_t ldo, int scale_mode,
    int splits) {
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int MT = WTM / 32, NTL = WTN / 32;
    constexpr int A_BLK = BM / 8;                    // A pair: 8 rows x 128 B per load
    constexpr int B_BLK = BN / 16;                   // B step: 16 rows x 64 B per load
    constexpr int A_HALF_PER_W = A_BLK / 2 / NW;     // loads per wave per half pair
    // When the B blocks do not split evenly over the waves, every wave still
    // issues B_PER_W loads (the extra ones out of range, into padding at the
    // end of the slot), so that all waves count the same loads.
    constexpr int B_PER_W = (B_BLK + NW - 1) / NW;
    constexpr int DPW = A_HALF_PER_W + B_PER_W;      // loads per wave per step
    static_assert(A_HALF_PER_W * 2 * NW == A_BLK, "tile/waves");
    static_assert((NB - 2) * DPW < 64, "vmcnt range");
    constexpr int A_SLOT = BM * 2 * BK;              // one pair slot
    constexpr int B_SLOT = B_PER_W * NW * 1024;      // BN * BK, padded to whole wave loads
    // Distinct LDS objects per slot (not one array indexed by slot) so that
    // the compiler can tell the slot being filled from the slot being read
    // and does not wait for fills before reads.
    __shared__ __attribute__((aligned(1024))) uint8_t a_s0[A_SLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t a_s1[A_SLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t a_s2[A_SLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t b_s0[B_SLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t b_s1[B_SLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t b_s2[B_SLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t b_s3[NB > 3 ? B_SLOT : 16];
    uint8_t* const a_slots[3] = {a_s0, a_s1, a_s2};
    uint8_t* const b_slots[4] = {b_s0, b_s1, b_s2, b_s3};

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int wm = wave / WN, wn = wave % WN;
    const int lr = lane & 31;
    const int lg = lane >> 5;
    // Split K (splits > 1, two-step form only): workgroup b takes K range
    // b / ntiles of tile b % ntiles and writes its partial sums to slice
    // b / ntiles of the fp32 output.  Ranges are whole A pairs (even steps).
    const int gm = (int)((T + BM - 1) / BM), gn = (int)((Co + BN - 1) / BN);
    const int ntiles = gm * gn;
    const int split = (int)blockIdx.x / ntiles;
    const int nks = (int)(Kp / BK);                  // K steps of the packed weight (even)
    const int per = ((nks + splits - 1) / splits + 1) & ~1;
    const int ks0 = split * per < nks ? split * per : nks;
    const int nsteps = (ks0 + per < nks ? ks0 + per : nks) - ks0;
    const int64_t k_end = (int64_t)(ks0 + nsteps) * BK < Ci ? (int64_t)(ks0 + nsteps) * BK : Ci;

    // Per-tile state.  Buffer descriptors are based at the tile's first row
    // and the split's first K step; rows past the end and K past the range
    // land beyond num_records or are sent there, and read as zero.
    // A pair load: lane L owns LDS row L/8 of its 8-row block, slot L%8, and
    // fetches the logical chunk that belongs in that slot.  The packed
    // weight is already in LDS order: 1 KB blocks of 16 columns x one 64-byte
    // K step, lane L's 16 bytes at L*16 (see the packing kernel).
    int64_t m0 = 0, n0 = 0, a_rows = 0;
    __amdgpu_buffer_rsrc_t ra, rb;
    uint32_t a_off[2][A_HALF_PER_W];
    int a_chunk[2][A_HALF_PER_W];
    uint32_t b_off[B_PER_W];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int p = 0; p < A_HALF_PER_W; ++p) {
            const int r = (h * (A_BLK / 2) + wave + p * NW) * 8 + (lane >> 3);
            a_chunk[h][p] = (lane & 7) ^ swz_a(r);
        }
    auto setup = [&](int tile) {
        int tm, tn;
        tile_of(tile, gm, gn, tm, tn);
        m0 = (int64_t)tm * BM;
        n0 = (int64_t)tn * BN;
        a_rows = (T - m0 < BM) ? (T - m0) : BM;
        const int64_t b_rows = (Co - n0 < BN) ? (Co - n0) : BN;
        ra = make_rsrc(qx + m0 * ldq + (int64_t)ks0 * BK, (uint32_t)(a_rows * ldq));
        rb = make_rsrc(wp + n0 * Kp + (int64_t)ks0 * 1024, (uint32_t)(b_rows * Kp));
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int p = 0; p < A_HALF_PER_W; ++p) {
                const int r = (h * (A_BLK / 2) + wave + p * NW) * 8 + (lane >> 3);
                a_off[h][p] = (r < a_rows) ? (uint32_t)(r * ldq + a_chunk[h][p] * 16) : kOutOfRange;
            }
#pragma unroll
        for (int p = 0; p < B_PER_W; ++p) {
            const int blk = wave + p * NW;           // 16-column group in the tile
            b_off[p] =
                (blk * 16 < b_rows) ? (uint32_t)(blk * nks * 1024 + lane * 16) : kOutOfRange;
        }
    };

    // Loads of one half (h) of the A pair holding steps 2q, 2q+1.
    auto issue_a_half = [&](int q, int h, uint8_t* slot) {
        const int k0 = q * 2 * BK;
#pragma unroll
        for (int p = 0; p < A_HALF_PER_W; ++p) {
            const bool kin = (int64_t)ks0 * BK + k0 + a_chunk[h][p] * 16 < k_end;
            const uint32_t off = (a_off[h][p] != kOutOfRange && kin) ? a_off[h][p] + k0
                                                                     : kOutOfRange;
            const int blk = h * (A_BLK / 2) + wave + p * NW;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(slot + blk * 1024), 16, off,
                                                     0, 0, 0);
        }
    };
    // Loads of B for step ks.
    auto issue_b = [&](int ks, uint8_t* slot) {
        const bool kin = ks < nsteps;
#pragma unroll
        for (int p = 0; p < B_PER_W; ++p) {
            const uint32_t off =
                (b_off[p] != kOutOfRange && kin) ? b_off[p] + (uint32_t)ks * 1024u : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (lds_ptr_t)(slot + (wave + p * NW) * 1024), 16, off, 0, 0,
                NTB ? kCacheNonTemporal : 0);
        }
    };
    // The fills before step 0: A pairs 0 and 1, the first NB B steps and the
    // first half of A pair 2, in the order they are needed, so that step 0
    // can start once the first three have landed: with a and b loads per A
    // half and per B step, the ones still allowed in flight then are the
    // last 3a + 3b, and the K loop's own "all but the last 2 steps' loads"
    // waits then see every later fill land before it is read (the loop's
    // first three tops each retire a + b more of them in order).
    static_assert(NB == 4, "fill order below is written for four B slots");
    // (sched_barrier keeps the scheduler from reordering the groups.)
    auto fill_prologue = [&]() {
        issue_a_half(0, 0, a_slots[0]);
        issue_a_half(0, 1, a_slots[0]);
        __builtin_amdgcn_sched_barrier(0);
        issue_b(0, b_slots[0]);
        __builtin_amdgcn_sched_barrier(0);
        issue_b(1, b_slots[1]);
        __builtin_amdgcn_sched_barrier(0);
        issue_b(2, b_slots[2]);
        __builtin_amdgcn_sched_barrier(0);
        issue_a_half(1, 0, a_slots[1]);
        issue_a_half(1, 1, a_slots[1]);
        __builtin_amdgcn_sched_barrier(0);
        issue_b(3, b_slots[3]);
        __builtin_amdgcn_sched_barrier(0);
        issue_a_half(2, 0, a_slots[2]);
        __builtin_amdgcn_sched_barrier(0);
    };

    v16f acc[MT][NTL];
    auto zero_acc = [&]() {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NTL; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    };

    // MFMA operands: lane l reads row l%32 of a 32-row slab and logical
    // chunks 2*(l/32), 2*(l/32)+1 of the 64-byte K step (for A, of the step's
    // half of the 128-byte pair row).
    int a_row[MT], a_sw[MT], b_lo[NTL], b_hi[NTL];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int r = wm * WTM + i * 32 + lr;
        a_row[i] = r * 2 * BK;
        a_sw[i] = swz_a(r);
    }
#pragma unroll
    for (int j = 0; j < NTL; ++j) {
        const int r = wn * WTN + j * 32 + lr;
        b_lo[j] = r * BK + (((2 * lg) ^ swz_b(r)) << 4);
        b_hi[j] = r * BK + (((2 * lg + 1) ^ swz_b(r)) << 4);
    }
    auto read_frags = [&](const uint8_t* as, int half, const uint8_t* bs, v8i (&a)[MT],
                          v8i (&b)[NTL]) {
        const int c0 = half * 4 + 2 * lg;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const uint4 lo = *reinterpret_cast<const uint4*>(as + a_row[i] + ((c0 ^ a_sw[i]) << 4));
            const uint4 hi =
                *reinterpret_cast<const uint4*>(as + a_row[i] + (((c0 + 1) ^ a_sw[i]) << 4));
            a[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int j = 0; j < NTL; ++j) {
            const uint4 lo = *reinterpret_cast<const uint4*>(bs + b_lo[j]);
            const uint4 hi = *reinterpret_cast<const uint4*>(bs + b_hi[j]);
            b[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                       (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
    };

    // Step s: its MFMAs, with the operand reads of step s+1 and the step's
    // loads threaded between them (the reads fill the other fragment
    // registers; issuing the loads in one burst would hold back the MFMAs).
    constexpr int NMFMA = MT * NTL;
    constexpr int NREAD = 2 * (MT + NTL);
    v8i fr_a[2][MT], fr_b[2][NTL];
    auto step = [&](auto U, int s) {
        constexpr int u = decltype(U)::value;        // s % period, static
        // operands of step s+1
        constexpr int n = u + 1;
        const uint8_t* na = a_slots[(n / 2) % 3];
        const uint8_t* nb = b_slots[n % NB];
        if constexpr (kLdsPoison) {
            // the regions this step refills: B slot u % NB and one half of an
            // A pair slot (see the fills below)
#pragma unroll
            for (int p = 0; p < B_PER_W; ++p) poison_block(b_slots[u % NB] + (wave + p * NW) * 1024);
            constexpr int h = (u & 1) ? 0 : 1;
            uint8_t* const as = a_slots[(u & 1) ? ((u + 5) / 2) % 3 : ((u + 4) / 2) % 3];
#pragma unroll
            for (int p = 0; p < A_HALF_PER_W; ++p)
                poison_block(as + (h * (A_BLK / 2) + wave + p * NW) * 1024);
            poison_done();
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NTL; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    fr_b[u & 1][j], fr_a[u & 1][i], acc[i][j], 0, 0, 0, 0, 0, 0);
        read_frags(na, n & 1, nb, fr_a[n & 1], fr_b[n & 1]);
        issue_b(s + NB, b_slots[u % NB]);
        if constexpr ((u & 1) == 0) {
            issue_a_half((s + 4) / 2, 1, a_slots[((u + 4) / 2) % 3]);
        } else {
            issue_a_half((s + 5) / 2, 0, a_slots[((u + 5) / 2) % 3]);
        }
        constexpr int NQ = NMFMA > NREAD ? NMFMA : NREAD;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if (q < NMFMA) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            if (q < NREAD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
            if (q < DPW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // VMEM read
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto top = [&]() {
        wait_counts<(NB - 2) * DPW, 0>();
        lds_barrier();
    };

    // The K loop.  Steps past the data are zero fills (every offset out of
    // range), so the loop needs no branch; it runs whole periods of P steps
    // (fewer than P extra zero steps are multiplied).  Unrolled by the period
    // so that every slot and fragment set is named statically.  On entry the
    // operands of step 0 are in fr_a[0] / fr_b[0]; on exit no fill is in
    // flight and every wave is past its last LDS read.
    constexpr int P = 6 * NB / gcd_c(6, NB);
    auto k_loop = [&]() {
        for (int s0 = 0; s0 < nsteps; s0 += P) {
            [&]<int... Us>(std::integer_sequence<int, Us...>) {
                ((top(), step(std::integral_constant<int, Us>{}, s0 + Us)), ...);
            }(std::make_integer_sequence<int, P>{});
        }
        wait_counts<0, 0>();
        lds_barrier();
    };

    // Epilogue.  The weight slab is the MFMA's first operand, so the 32x32
    // accumulator tile is out^T: in lane l, element e holds output row
    // (token) l%32 of the slab and output column 8*(e/4) + 4*(l/32) + e%4.
    // Each lane therefore owns runs of 4 consecutive columns of one row.
    //
    // Fused: the bf16 results of one 32-row slab of the wave tile go to a
    // wave-private LDS region (in the A slots, idle now, from the last one
    // down) and come back as 16-byte row chunks, so that every store
    // instruction writes whole row segments of WTN*2 bytes.  The 8-byte
    // writes of one instruction (32 rows, one column run) are spread over all
    // banks: with a power-of-two chunk count chunk c of slab row r sits at
    // chunk c ^ ((r / RB) % NC) of its LDS row (RB rows span the 64 banks);
    // otherwise rows are padded by 16 bytes.  All scales are loaded up front
    // (one latency instead of one per slab) and the stores go through a
    // range-checked descriptor (rows past T land beyond it, columns past Co
    // are sent there) instead of branches.
    constexpr int P2 = WTN * 2;                      // bytes per slab row
    constexpr int NC = WTN / 8;                      // 16-byte chunks per row
    constexpr bool POW2 = (NC & (NC - 1)) == 0;
    constexpr int PITCH = POW2 ? P2 : P2 + 16;
    constexpr int RB = POW2 ? 256 / P2 : 1;
    constexpr int NCHUNK = 32 * NC;                  // chunks per slab
    constexpr int NSTORE = (NCHUNK + 63) / 64;       // store instructions per slab
    constexpr int RPS = A_SLOT / (32 * PITCH);       // regions per A slot
    static_assert(!FUSED || (RPS >= 1 && NW <= 3 * RPS && RB >= 1), "staging");
    auto slot_of = [](int r, int c) { return POW2 ? (c ^ ((r / RB) % NC)) : c; };
    float sxv[MT];
    float4 swv[NTL][4];
    auto load_scales = [&]() {
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int64_t row = m0 + wm * WTM + i * 32 + lr;
            sxv[i] = (scale_mode == kUnitScales || row >= T) ? 1.0f : dx[scale_mode ? 0 : row];
        }
#pragma unroll
        for (int j = 0; j < NTL; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t col = n0 + wn * WTN + j * 32 + 8 * g + 4 * lg;
                swv[j][g] = col < Co ? scale_of_cols(dw, col, scale_mode)
                                     : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
            }
    };
    auto epilogue = [&](int64_t em0, int64_t en0) {
        if constexpr (FUSED) {
            const int sl = wave / RPS;
            uint8_t* const stage =
                (sl == 0 ? a_s2 : sl == 1 ? a_s1 : a_s0) + (wave - sl * RPS) * (32 * PITCH);
            const int64_t e_rows = (T - em0 < BM) ? (T - em0) : BM;
            const __amdgpu_buffer_rsrc_t ro =
                make_rsrc(reinterpret_cast<uint16_t*>(out) + em0 * ldo, (uint32_t)(e_rows * ldo * 2));
#pragma unroll
            for (int i = 0; i < MT; ++i) {
#pragma unroll
                for (int j = 0; j < NTL; ++j) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const float sx = sxv[i];
                        const float4 sw = swv[j][g];
                        uint2 pk;
                        pk.x = f32x2_to_bf16x2_rne((acc[i][j][4 * g + 0] * sx) * sw.x,
                               (acc[i][j][4 * g + 1] * sx) * sw.y);
                        pk.y = f32x2_to_bf16x2_rne((acc[i][j][4 * g + 2] * sx) * sw.z,
                               (acc[i][j][4 * g + 3] * sx) * sw.w);
                        *reinterpret_cast<uint2*>(stage + lr * PITCH +
                                                  (slot_of(lr, 4 * j + g) << 4) + lg * 8) = pk;
                    }
                }
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
                for (int q = 0; q < NSTORE; ++q) {
                    const int idx = q * 64 + lane;
                    const int rr = idx / NC, cc = idx % NC;
                    const bool in = idx < NCHUNK;
                    const uint4 v = *reinterpret_cast<const uint4*>(
                        stage + (in ? rr * PITCH + (slot_of(rr, cc) << 4) : 0));
                    const int64_t lrow = wm * WTM + i * 32 + rr;      // row within the tile
                    const int64_t gcol = en0 + wn * WTN + cc * 8;
                    const uint32_t off = (in && gcol < Co)
                                             ? (uint32_t)((lrow * ldo + gcol) * 2)
                                             : kOutOfRange;
                    __builtin_amdgcn_raw_buffer_store_b128(
                        v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w}, ro, off, 0, 0);
                }
                __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            }
        } else {
            // Two-step form: unscaled fp32 runs of 4 columns, 16-byte stores.
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int64_t row = em0 + wm * WTM + i * 32 + lr;
                if (row >= T) continue;
#pragma unroll
                for (int j = 0; j < NTL; ++j) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int64_t col = en0 + wn * WTN + j * 32 + 8 * g + 4 * lg;
                        if (col >= Co) continue;
                        *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) +
                                                   (int64_t)split * T * Co + row * Co + col) =
                            make_float4(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1],
                                        acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
                    }
                }
            }
        }
    };

    setup((int)blockIdx.x - split * ntiles);
    zero_acc();
    if (nsteps > 0) {
        fill_prologue();
        wait_counts<3 * A_HALF_PER_W + 3 * B_PER_W, 0>();   // A pair 0 and B step 0
        lds_barrier();
        read_frags(a_slots[0], 0, b_slots[0], fr_a[0], fr_b[0]);
        k_loop();
    }
    if constexpr (FUSED) load_scales();
    epilogue(m0, n0);
}

// The 16x16x128 form of the tiled kernel, used for the 256-token tiles.
// Same operands, layouts and epilogue arithmetic as gemm_kernel, but every
// MFMA is v_mfma_f32_16x16x128_f8f6f4: for the same work that form holds a
// higher clock under the chip's power limit than the 32x32x64 one.  One MFMA
// spans 128 K bytes, so a step is 128 K bytes: one A pair row (both halves)
// and two 64-byte B blocks per 16 columns.
//   LDS: 2 A slots (BM x 128 B) and 3 B slots (two 64-byte half steps of BN
//   columns each); the weight, streamed from HBM, gets the deeper ring.
//   Operand lanes: lane l takes row l % 16 of a 16-row slab and K bytes
//   32 * (l / 16) .. +31 of the step (for B: from half step l / 32).
//   A step runs over the wave's 16-column slabs j, each against all its
//   16-row slabs (MT MFMAs).  The A fragments of step s+1 are read during
//   step s (two register sets); the B fragment of slab j is read two slabs
//   ahead of its use into a ring of three (the last two slabs of step s read
//   step s+1's first two).  The pieces of this side work (operand reads and
//   fills) are spread evenly between the slab's MFMAs, so that their issue
//   hides under the running MFMAs.
//   Two barriers per step.  At the top of step s, A of step s+1 has landed
//   (it is read during step s) and A slot s%2 is free: A of step s+2 is
//   filled into it.  Before slab NT-2 ("mid"), B of step s+1 has landed (its
//   first fragments are read next) and every read of B slot s%3 is done: the
//   first half of B of step s+3 is filled into it during the last two slabs,
//   the second half during the first NT-2 slabs of step s+1 (the slot is
//   next read in step s+2).  The fills are spread evenly over the slabs (A
//   of step s+2, then the second half of B of step s+2, before mid; the
//   first half of B of step s+3 after it): the address unit takes a 1 KB LDS
//   load in several cycles, and four waves issuing their fills in bursts
//   stalled their MFMA issue (on the 70B down projection the even spread is
//   8% faster than fills confined to four of the eight slabs).  With loads
//   issued in that order the waits are "all but the last step's B fills" at
//   the top and "all but the last A and B step's worth" at mid.
//   The MFMAs are issued from inline asm with the accumulators tied to AGPRs:
//   with the builtin, the register allocator moved 64 four-register
//   accumulators between AGPRs, VGPRs and scratch inside the K loop.  Inline
//   asm hides the MFMAs from the compiler's hazard tracking, so the kernel
//   keeps every dependence on an accumulator far apart by construction: in
//   the K loop an accumulator is next used a full step later, the zeroing
//   before the loop is pinned ahead of an explicit wait, and the epilogue
//   reads the accumulators only after the loop's final wait and barrier.
//   Operand registers are only read by the MFMAs (LDS loads may overwrite
//   them right after issue, as in compiler-scheduled code).
// The K loop runs whole periods of 6 steps, then the remaining 0-5 steps,
// each behind a uniform branch; fills for steps past the data read zeros.
template <int BM, int BN, int WM, int WN, bool FUSED, bool FIXUP = false>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm16_kernel(
    const uint8_t* __restrict__ qx, int64_t ldq, const float* __restrict__ dx,
    const uint8_t* __restrict__ wp, int64_t Kp, const float* __restrict__ dw,
    int64_t T, int64_t Ci, int64_t Co, void* __restrict__ out, int64_t ldo, int scale_mode,
    int splits, float* __restrict__ part) {
    static_assert(!FIXUP || FUSED, "the two-range fix-up ends in the fused epilogue");
    constexpr int KS = 128;                          // K bytes per step
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int MT = WTM / 16, NT = WTN / 16;
    constexpr int A_BLK = BM / 8;                    // A: 8 rows x 128 B per load
    constexpr int BH = BN / 16;                      // B: 1 KB blocks per half step
    constexpr int B_BLK = 2 * BH;
    constexpr int A_PER_W = A_BLK / NW;
    constexpr int B_PER_W = (B_BLK + NW - 1) / NW;   // padded: extra loads out of range
    constexpr int RING = 3;                          // B fragment ring, read 2 slabs ahead
    static_assert(A_PER_W * NW == A_BLK && NT >= 4, "tile/waves");
    static_assert(2 * A_PER_W + 2 * B_PER_W < 64, "vmcnt range");
    // B fills of step s+3: the first B1 loads go out in the last two slabs
    // of step s, the other B2 in the first NT-2 slabs of step s+1, after
    // that step's A fills (NEARLY fills spread over those slabs).  B1 makes
    // the busier of the two windows as light as it can be (fills per slab),
    // the larger B1 on a tie.
    constexpr int B1 = [] {
        int best = B_PER_W, cost = 1 << 30;
        for (int b = B_PER_W; b >= 1; --b) {
            const int early = 2 * (A_PER_W + B_PER_W - b), late = b * (NT - 2);
            const int c = early > late ? early : late;
            if (c < cost) { cost = c; best = b; }
        }
        return best;
    }();
    constexpr int B2 = B_PER_W - B1;
    constexpr int NEARLY = A_PER_W + B2;
    constexpr int A_SLOT = BM * KS;
    constexpr int B_SLOT = B_PER_W * NW * 1024;
    __shared__ __attribute__((aligned(1024))) uint8_t a_s0[A_SLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t a_s1[A_SLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t b_s0[B_SLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t b_s1[B_SLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t b_s2[B_SLOT];
    auto a_slot = [&](int k) __attribute__((always_inline)) -> uint8_t* {
        return k == 0 ? a_s0 : a_s1;
    };
    auto b_slot = [&](int k) __attribute__((always_inline)) -> uint8_t* {
        return k == 0 ? b_s0 : k == 1 ? b_s1 : b_s2;
    };

    timeline_mark(0);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    const int gm = (int)((T + BM - 1) / BM), gn = (int)((Co + BN - 1) / BN);
    const int ntiles = gm * gn;
    int tile_lin;
    const int split = split_of((int)blockIdx.x, splits, ntiles, tile_lin);
    const int nks = (int)(Kp / KS);
    const int per = (nks + splits - 1) / splits;
    const int ks0 = split * per < nks ? split * per : nks;
    const int nsteps = (ks0 + per < nks ? ks0 + per : nks) - ks0;
    const int64_t k_end = (int64_t)(ks0 + nsteps) * KS < Ci ? (int64_t)(ks0 + nsteps) * KS : Ci;

    // Loads.  A: load p of a wave covers the 8-row block wave + p * NW; lane
    // L owns LDS row L/8 of it, slot L%8, and fetches the logical chunk that
    // belongs there.  B: load p copies 1 KB packed block bl = wave + p * NW
    // of the step (16-column group bl % BH, half step bl / BH) to LDS offset
    // bl * 1024.  Offsets are 32-bit (the descriptors span less than 4 GB)
    // and branch-free.
    int tm, tn;
    tile_group_of(tile_lin, gm, gn, tm, tn, group_n_of<BM, BN>());
    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * BN;
    const int64_t a_rows = (T - m0 < BM) ? (T - m0) : BM;
    const int64_t b_rows = (Co - n0 < BN) ? (Co - n0) : BN;
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(qx + m0 * ldq + (int64_t)ks0 * KS, (uint32_t)(a_rows * ldq));
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(wp + n0 * Kp + (int64_t)ks0 * 2048, (uint32_t)(b_rows * Kp));
    const int k_lim = (int)(k_end - (int64_t)ks0 * KS);  // K bytes of this range
    // With an even number of waves, the A rows of load p are those of load 0
    // plus p * NW * 8 and their chunk swizzle is the same, so the per-lane
    // part of every A offset is one register; the rest is wave-uniform.
    static_assert(NW % 2 == 0, "A chunk swizzle shared by all loads of a wave");
    const int a_r0 = wave * 8 + (lane >> 3);
    const int a_c16 = ((lane & 7) ^ swz_a(a_r0)) * 16;
    const uint32_t a_lane = (uint32_t)a_r0 * (uint32_t)ldq + (uint32_t)a_c16;
    const uint32_t b_lane = (uint32_t)lane * 16u;
    // LDS offset of this wave's fills, re-defined at every step (an empty
    // asm) so that the compiler forms each fill's LDS address with one add
    // instead of holding one register per fill and slot across the loop.
    int wlds = wave * 1024;
    // Rows past the tile's last row need no test of their own: the
    // descriptors span exactly a_rows rows of A and b_rows columns of the
    // packed weight, so their offsets fall outside and read as zero.
    auto issue_a = [&](int ks, int p, uint8_t* slot) __attribute__((always_inline)) {
        const int k0 = ks * KS;
        const bool in = k0 + a_c16 < k_lim;
        const uint32_t off =
            in ? a_lane + (uint32_t)(p * NW * 8) * (uint32_t)ldq + (uint32_t)k0 : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(slot + wlds + p * NW * 1024),
                                                 16, off, 0, 0, 0);
    };
    auto issue_b = [&](int ks, int p, uint8_t* slot) __attribute__((always_inline)) {
        const int bl = wave + p * NW;
        const int blk = bl % BH, h = bl / BH;
        const bool in = (bl < B_BLK) & (ks < nsteps);
        const uint32_t off =
            in ? b_lane + ((uint32_t)(blk * 16) * (uint32_t)Kp + (uint32_t)(h * 1024 + ks * 2048))
               : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(slot + wlds + p * NW * 1024), 16,
                                                 off, 0, 0, 0);
    };

    // Operand reads (see the layout above); the swizzle of a 16-row slab
    // depends only on the lane, slabs are fixed offsets apart.
    const int a_lo = (wm * WTM + l16) * KS + (((2 * lg) ^ swz_a(l16)) << 4);
    const int a_hi = (wm * WTM + l16) * KS + (((2 * lg + 1) ^ swz_a(l16)) << 4);
    const int b_base = (lg >> 1) * BH * 1024 + (wn * WTN + l16) * 64;
    const int b_lo = b_base + (((2 * (lg & 1)) ^ swz_b(l16)) << 4);
    const int b_hi = b_base + (((2 * (lg & 1) + 1) ^ swz_b(l16)) << 4);
    auto read_a = [&](const uint8_t* as, int i) __attribute__((always_inline)) {
        const uint4 lo = *reinterpret_cast<const uint4*>(as + a_lo + i * 16 * KS);
        const uint4 hi = *reinterpret_cast<const uint4*>(as + a_hi + i * 16 * KS);
        return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    auto read_b = [&](const uint8_t* bs, int j) __attribute__((always_inline)) {
        const uint4 lo = *reinterpret_cast<const uint4*>(bs + b_lo + j * 1024);
        const uint4 hi = *reinterpret_cast<const uint4*>(bs + b_hi + j * 1024);
        return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };

    // Accumulators: zeroed, pinned (the empty asm makes every zero write
    // happen before it) and followed by a wait before any MFMA reads them.
    v4f acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
            asm volatile("" : "+a"(acc[i][j]));
        }
    asm volatile("s_nop 4");
    v8i fr_a[2][MT], fr_b[RING];

    auto sync = [&](auto VM) __attribute__((always_inline)) {
        wait_counts<decltype(VM)::value, 0>();
        lds_barrier();
    };
    // Step s = s0 + u (u = s % 6 static): slab by slab, each slab's MFMAs with
    // its side work threaded between them (see above).
    auto step = [&](auto U, int s) __attribute__((always_inline)) {
        constexpr int u = decltype(U)::value;
        asm volatile("" : "+s"(wlds));
        constexpr int cur = u & 1;
        const uint8_t* const na = a_slot((u + 1) % 2);
        const uint8_t* const cb = b_slot(u % 3);
        const uint8_t* const nb = b_slot((u + 1) % 3);
        uint8_t* const fa = a_slot(u % 2);
        uint8_t* const fb = b_slot(u % 3);
        uint8_t* const fc = b_slot((u + 2) % 3);
        if constexpr (kLdsPoison) {
            // A slot u % 2 (A of step s, read during step s - 1) is refilled
            // with A of step s + 2 from here on
#pragma unroll
            for (int p = 0; p < A_PER_W; ++p) poison_block(fa + wave * 1024 + p * NW * 1024);
            poison_done();
        }
        [&]<int... Js>(std::integer_sequence<int, Js...>) __attribute__((always_inline)) {
            ([&]() __attribute__((always_inline)) {
                constexpr int j = Js;
                constexpr int g = u * NT + j;                 // global slab index
                constexpr int ia0 = j * MT / NT, ia1 = (j + 1) * MT / NT;  // A frags read
                constexpr int NE = NT - 2;                    // slabs before mid
                // Early slabs (before mid): fill items e0..e1 of the
                // NEARLY spread evenly over them, A of step s+2 first, then
                // the last B2 loads of B of step s+2.
                constexpr int e0 = j < NE ? (j * NEARLY + NE - 1) / NE : 0;
                constexpr int e1 = j < NE ? ((j + 1) * NEARLY + NE - 1) / NE : 0;
                constexpr int pa0 = e0 < A_PER_W ? e0 : A_PER_W;
                constexpr int pa1 = e1 < A_PER_W ? e1 : A_PER_W;
                constexpr int pc0 = (e0 > A_PER_W ? e0 : A_PER_W) - A_PER_W + B1;
                constexpr int pc1 = (e1 > A_PER_W ? e1 : A_PER_W) - A_PER_W + B1;
                // Late slabs (from mid): the first B1 loads of B of step s+3.
                constexpr int pb0 = j < NE ? 0 : (j - NE) * B1 / 2;
                constexpr int pb1 = j < NE ? 0 : (j - NE + 1) * B1 / 2;
                if constexpr (j == NE) {
                    sync(std::integral_constant<int, A_PER_W + B_PER_W>{});
                    if constexpr (kLdsPoison) {
                        // B slot u % 3 (B of step s, read up to here) takes
                        // B of step s + 3 from here on, in both its parts
#pragma unroll
                        for (int p = 0; p < B_PER_W; ++p)
                            poison_block(fb + wave * 1024 + p * NW * 1024);
                        poison_done();
                    }
                }
                // Side work of the slab in issue order: the A fragments and
                // the B fragment first, then the fills.
                constexpr int NIA = ia1 - ia0, NPA = pa1 - pa0, NPC = pc1 - pc0, NPB = pb1 - pb0;
                constexpr int NITEM = NIA + 1 + NPA + NPC + NPB;
                auto side = [&](auto Q) __attribute__((always_inline)) {
                    constexpr int q = decltype(Q)::value;
                    if constexpr (q < NIA) {
                        fr_a[cur ^ 1][ia0 + q] = read_a(na, ia0 + q);
                    } else if constexpr (q == NIA) {
                        if constexpr (j + 2 < NT)
                            fr_b[(g + 2) % RING] = read_b(cb, j + 2);
                        else
                            fr_b[(g + 2) % RING] = read_b(nb, j + 2 - NT);
                    } else if constexpr (q < NIA + 1 + NPA) {
                        issue_a(s + 2, pa0 + q - NIA - 1, fa);
                    } else if constexpr (q < NIA + 1 + NPA + NPC) {
                        issue_b(s + 2, pc0 + q - NIA - 1 - NPA, fc);
                    } else if constexpr (q < NITEM) {
                        issue_b(s + 3, pb0 + q - NIA - 1 - NPA - NPC, fb);
                    }
                };
                __builtin_amdgcn_sched_barrier(0);
                [&]<int... Qs>(std::integer_sequence<int, Qs...>) __attribute__((always_inline)) {
                    ([&]() __attribute__((always_inline)) {
                        constexpr int q = Qs;
                        if constexpr (q < MT)
                            asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0"
                                         : "+a"(acc[q][j])
                                         : "v"(fr_b[g % RING]), "v"(fr_a[cur][q]));
                        __builtin_amdgcn_sched_barrier(0);
                        // The slab's side items, spread evenly between
                        // its MFMAs.
                        if constexpr (NITEM <= MT) {
                            constexpr int i0 = (q * NITEM + MT - 1) / MT;
                            constexpr int i1 = ((q + 1) * NITEM + MT - 1) / MT;
                            [&]<int... Is>(std::integer_sequence<int, Is...>)
                                __attribute__((always_inline)) {
                                    (side(std::integral_constant<int, i0 + Is>{}), ...);
                                }(std::make_integer_sequence<int, i1 - i0>{});
                        } else {
                            side(std::integral_constant<int, q>{});
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }(), ...);
                }(std::make_integer_sequence<int, (MT > NITEM ? MT : NITEM)>{});
                __builtin_amdgcn_sched_barrier(0);
            }(), ...);
        }(std::make_integer_sequence<int, NT>{});
    };

    if (nsteps > 0) {
        // Fills in steady-state order: B0, A0, B1 (first B1 loads), A1,
        // B1 (the rest), B2 (first B1 loads).
#pragma unroll
        for (int p = 0; p < B_PER_W; ++p) issue_b(0, p, b_s0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < A_PER_W; ++p) issue_a(0, p, a_s0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < B1; ++p) issue_b(1, p, b_s1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < A_PER_W; ++p) issue_a(1, p, a_s1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = B1; p < B_PER_W; ++p) issue_b(1, p, b_s1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < B1; ++p) issue_b(2, p, b_s2);
        __builtin_amdgcn_sched_barrier(0);
        sync(std::integral_constant<int, A_PER_W + B_PER_W + B1>{});   // A0, B0
        timeline_mark(1);
#pragma unroll
        for (int i = 0; i < MT; ++i) fr_a[0][i] = read_a(a_s0, i);
        fr_b[0] = read_b(b_s0, 0);
        fr_b[1] = read_b(b_s0, 1);
        constexpr int P = 6;
        int s0 = 0;
        for (; s0 + P <= nsteps; s0 += P) {
            [&]<int... Us>(std::integer_sequence<int, Us...>) __attribute__((always_inline)) {
                ((sync(std::integral_constant<int, B_PER_W>{}),
                  step(std::integral_constant<int, Us>{}, s0 + Us)),
                 ...);
            }(std::make_integer_sequence<int, P>{});
        }
        const int rem = __builtin_amdgcn_readfirstlane(nsteps - s0);
        [&]<int... Us>(std::integer_sequence<int, Us...>) __attribute__((always_inline)) {
            (([&]() __attribute__((always_inline)) {
                 if (Us < rem) {
                     sync(std::integral_constant<int, B_PER_W>{});
                     step(std::integral_constant<int, Us>{}, s0 + Us);
                 }
             }()),
             ...);
        }(std::make_integer_sequence<int, P - 1>{});
        wait_counts<0, 0>();
        lds_barrier();
        // The MFMAs are inline asm, invisible to the compiler's hazard
        // tracking: 24 wait states after the last one, and every accumulator
        // pinned behind them, so that no read of an accumulator (the
        // epilogue's, or a copy the register allocator makes) comes sooner.
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j) asm volatile("" : "+a"(acc[i][j]));
        timeline_mark(2);
    }

    // Published sums of the other K range (two-range fix-up), read with
    // device-coherent loads (unused otherwise).
    float* const tslot = FIXUP ? part + (int64_t)tile_lin * BM * BN : part;
    const __amdgpu_buffer_rsrc_t rpart =
        make_rsrc(tslot, FIXUP ? (uint32_t)(BM * BN * sizeof(float)) : 0u);
    uint32_t fix_lost = 0;      // the other range's flag never came: NaN output
    if constexpr (FIXUP) {
        // Two K ranges per tile, joined without a second pass.  Each
        // workgroup takes a ticket on its tile's record once its K loop is
        // done.  Ticket 0 publishes its fp32 sums in the tile's slot of
        // `part` (lane order: one 1 KB run per wave and accumulator tile),
        // writes them back from its XCD's L2 to memory, raises the record's
        // flag and exits.  Ticket 1 waits for that flag -- set by a
        // workgroup that is already past its own K loop, so the wait ends
        // whatever the order of dispatch -- and its epilogue adds the
        // published sums, read with device-coherent (sc1) loads, to its own.
        // No L2 invalidation: that would drop the operand lines of the
        // workgroups of its XCD still in their K loops (with one, the 70B O
        // projection at 1024 tokens ran 1.4x slower).  With two terms the sum
        // does not depend on which range arrives first (IEEE addition
        // commutes): the result is range 0 + range 1 in any timing.  The wait
        // is bounded (kFixupSpins sleeps of ~64 clocks) so that no fault
        // elsewhere can keep the kernel from exiting; should it run out, the
        // tile's outputs are written as NaN instead of a sum with stale
        // partials.  Records are 4 words per tile after the slots, cleared
        // before the launch.
        uint32_t* const rec = reinterpret_cast<uint32_t*>(part + (int64_t)ntiles * BM * BN) +
                              4 * tile_lin;
        volatile uint32_t* const bcast = reinterpret_cast<volatile uint32_t*>(b_s2);
        if (tid == 0)
            *bcast = __hip_atomic_fetch_add(rec, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const uint32_t ticket = __builtin_amdgcn_readfirstlane(*bcast);
        if (ticket == 0) {
            float* const slot = tslot + wave * (MT * NT * 256) + lane * 4;
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    *reinterpret_cast<v4f*>(slot + (i * NT + j) * 256) = acc[i][j];
            // every wave's stores have reached its L2 before the one
            // write-back that the flag's release makes
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (tid == 0 && kRaiseJoinFlag)
                __hip_atomic_store(rec + 1, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        if (tid == 0) {
            int spins = 0;
            while (__hip_atomic_load(rec + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0 &&
                   ++spins < kFixupSpins)
                __builtin_amdgcn_s_sleep(1);
            bcast[1] = __hip_atomic_load(rec + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0;
        }
        __syncthreads();
        fix_lost = __builtin_amdgcn_readfirstlane(bcast[1]);
    }

    // Epilogue.  The weight slab is the MFMA's first operand, so the 16x16
    // accumulator tile is out^T: in lane l, element e holds token row l % 16
    // of the slab and column 4 * (l / 16) + e.  As in gemm_kernel, the bf16
    // results of one 16-row slab go through a wave-private LDS region (in
    // A slot 0) and leave as 16-byte row chunks through a range-checked
    // descriptor.
    constexpr int P2 = WTN * 2;
    constexpr int NC = WTN / 8;
    constexpr bool POW2 = (NC & (NC - 1)) == 0;
    constexpr int PITCH = POW2 ? P2 : P2 + 16;
    constexpr int RB = POW2 ? (256 / P2 > 0 ? 256 / P2 : 1) : 1;
    constexpr int NCHUNK = 16 * NC;
    constexpr int NSTORE = (NCHUNK + 63) / 64;
    static_assert(!FUSED || NW * 16 * PITCH <= A_SLOT, "staging");
    auto slot_of = [](int r, int c) { return POW2 ? (c ^ ((r / RB) % NC)) : c; };
    if constexpr (FUSED) {
        // Lane coordinates re-derived here (the empty asm hides where they
        // come from), so that nothing the epilogue computes from them is
        // hoisted above the K loop and held through it.
        int elane = (int)threadIdx.x;
        asm volatile("" : "+v"(elane));
        const int lane = elane & 63, l16 = elane & 15, lg = (elane >> 4) & 3;
        float sxv[MT];
        float4 swv[NT];
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int64_t row = m0 + wm * WTM + i * 16 + l16;
            sxv[i] = (scale_mode == kUnitScales || row >= T) ? 1.0f : dx[scale_mode ? 0 : row];
            if constexpr (FIXUP) sxv[i] = fix_lost ? __builtin_nanf("") : sxv[i];
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int64_t col = n0 + wn * WTN + j * 16 + 4 * lg;
            swv[j] = col < Co ? scale_of_cols(dw, col, scale_mode)
                              : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
        }
        uint8_t* const stage = a_s0 + wave * (16 * PITCH);
        const int64_t e_rows = (T - m0 < BM) ? (T - m0) : BM;
        const __amdgpu_buffer_rsrc_t ro =
            make_rsrc(reinterpret_cast<uint16_t*>(out) + m0 * ldo, (uint32_t)(e_rows * ldo * 2));
        // Two-range fix-up: the other range's sums of slab i, loaded one
        // slab ahead of their use.
        v4f pv[2][FIXUP ? NT : 1];
        auto load_pv = [&](int i, int b) __attribute__((always_inline)) {
            if constexpr (FIXUP) {
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const uint32_t off =
                        (uint32_t)((wave * (MT * NT * 256) + (i * NT + j) * 256 + lane * 4) * 4);
                    const v4i v = __builtin_amdgcn_raw_buffer_load_b128(rpart, off, 0, kSc1);
                    pv[b][j] = v4f{__int_as_float(v.x), __int_as_float(v.y),
                                   __int_as_float(v.z), __int_as_float(v.w)};
                }
            }
        };
        load_pv(0, 0);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            if (i + 1 < MT) load_pv(i + 1, (i + 1) & 1);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const float sx = sxv[i];
                const float4 sw = swv[j];
                v4f a = acc[i][j];
                if constexpr (FIXUP) a += pv[i & 1][j];
                uint2 pk;
                pk.x = f32x2_to_bf16x2_rne((a[0] * sx) * sw.x,
                       (a[1] * sx) * sw.y);
                pk.y = f32x2_to_bf16x2_rne((a[2] * sx) * sw.z,
                       (a[3] * sx) * sw.w);
                *reinterpret_cast<uint2*>(stage + l16 * PITCH +
                                          (slot_of(l16, 2 * j + (lg >> 1)) << 4) +
                                          (lg & 1) * 8) = pk;
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
            for (int q = 0; q < NSTORE; ++q) {
                const int idx = q * 64 + lane;
                const int rr = idx / NC, cc = idx % NC;
                const bool in = idx < NCHUNK;
                const uint4 v = *reinterpret_cast<const uint4*>(
                    stage + (in ? rr * PITCH + (slot_of(rr, cc) << 4) : 0));
                const int64_t lrow = wm * WTM + i * 16 + rr;
                const int64_t gcol = n0 + wn * WTN + cc * 8;
                const uint32_t off =
                    (in && gcol < Co) ? (uint32_t)((lrow * ldo + gcol) * 2) : kOutOfRange;
                __builtin_amdgcn_raw_buffer_store_b128(v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w},
                                                       ro, off, 0, 0);
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        }
    } else {
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int64_t row = m0 + wm * WTM + i * 16 + l16;
            if (row >= T) continue;
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int64_t col = n0 + wn * WTN + j * 16 + 4 * lg;
                if (col >= Co) continue;
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) +
                                           (int64_t)split * T * Co + row * Co + col) =
                    make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
            }
        }
    }
    timeline_mark(3);
}

// 65..128 tokens on 64x64 tiles: the 16x16x128 pipeline with the K steps dealt to the four
// waves of a workgroup (wave w takes steps w, w+4, w+8, ...).  A workgroup
// owns a 64x64 output tile; every wave multiplies the whole tile over its
// steps through its own LDS slots (2 A + 3 B, 8 KB each, the same ring and
// fill order as gemm16_kernel), so the waves never wait for each other in
// the K loop: their syncs are waits on their own loads, no barriers.  With
// 64x64 tiles a 128-token layer of 8192 columns fills all 256 CUs once,
// each CU running four independent streams instead of one small tile split
// four ways with a barrier per step.  The four partial tiles are added in
// LDS in wave order (deterministic), then each wave stores 16 rows through
// the epilogue of gemm16_kernel.
template <bool FUSED>
__global__ __launch_bounds__(256, 1) void gemm16s_kernel(
    const uint8_t* __restrict__ qx, int64_t ldq, const float* __restrict__ dx,
    const uint8_t* __restrict__ wp, int64_t Kp, const float* __restrict__ dw,
    int64_t T, int64_t Ci, int64_t Co, void* __restrict__ out, int64_t ldo, int scale_mode) {
    constexpr int KS = 128;                          // K bytes per step
    constexpr int NW = 4;
    constexpr int BM = 64, BN = 64, MT = 4, NT = 4;
    constexpr int NA = BM / 8;                       // A loads per step (8 rows x 128 B)
    constexpr int BH = BN / 16;                      // 1 KB B blocks per half step
    constexpr int NB = 2 * BH;                       // B loads per step
    constexpr int RING = 3;
    constexpr int SLOT = BM * KS;
    static_assert(NB * 1024 == SLOT && NA + NB < 32, "slots");
    __shared__ __attribute__((aligned(1024))) uint8_t a_s0[NW][SLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t a_s1[NW][SLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t b_s0[NW][SLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t b_s1[NW][SLOT];
    __shared__ __attribute__((aligned(1024))) uint8_t b_s2[NW][SLOT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    const int gm = (int)((T + BM - 1) / BM), gn = (int)((Co + BN - 1) / BN);
    int tm, tn;
    tile_of((int)blockIdx.x, gm, gn, tm, tn);
    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * BN;
    const int a_rows = (int)((T - m0 < BM) ? (T - m0) : BM);
    const int b_rows = (int)((Co - n0 < BN) ? (Co - n0) : BN);
    const int nks = (int)(Kp / KS);
    const int nsteps = (nks - wave + NW - 1) / NW;   // this wave's steps
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(qx + m0 * ldq, (uint32_t)(a_rows * ldq));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(wp + n0 * Kp, (uint32_t)(b_rows * Kp));
    auto a_slot = [&](int k) __attribute__((always_inline)) -> uint8_t* {
        return k == 0 ? a_s0[wave] : a_s1[wave];
    };
    auto b_slot = [&](int k) __attribute__((always_inline)) -> uint8_t* {
        return k == 0 ? b_s0[wave] : k == 1 ? b_s1[wave] : b_s2[wave];
    };

    // Loads of local step i (global step wave + NW * i).  A: load p covers
    // rows 8p .. 8p+7; lane L owns LDS row 8p + L/8, slot L%8, and fetches
    // the logical chunk that belongs there (the swizzle alternates with p).
    // B: load p copies packed block p of the step (16-column group p % BH,
    // half step p / BH) to LDS offset p * 1024.
    const int a_r = lane >> 3;
    const int a_c16e = ((lane & 7) ^ swz_a(a_r)) * 16;
    const int a_c16o = ((lane & 7) ^ swz_a(a_r + 8)) * 16;
    const uint32_t b_lane = (uint32_t)lane * 16u;
    auto issue_a = [&](int i, int p, uint8_t* slot) __attribute__((always_inline)) {
        const int k0 = (wave + NW * i) * KS;
        const int row = 8 * p + a_r;
        const int c16 = (p & 1) ? a_c16o : a_c16e;
        const bool in = (row < a_rows) & (k0 + c16 < (int)Ci);
        const uint32_t off =
            in ? (uint32_t)row * (uint32_t)ldq + (uint32_t)(k0 + c16) : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(slot + p * 1024), 16, off, 0,
                                                 0, 0);
    };
    auto issue_b = [&](int i, int p, uint8_t* slot) __attribute__((always_inline)) {
        const int ks = wave + NW * i;
        const int blk = p % BH, h = p / BH;
        const bool in = (blk * 16 < b_rows) & (ks < nks);
        const uint32_t off =
            in ? b_lane + ((uint32_t)(blk * 16) * (uint32_t)Kp + (uint32_t)(h * 1024 + ks * 2048))
               : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(slot + p * 1024), 16, off, 0,
                                                 0, 0);
    };

    // Operand reads, as in gemm16_kernel for a wave covering the whole tile.
    const int a_lo = l16 * KS + (((2 * lg) ^ swz_a(l16)) << 4);
    const int a_hi = l16 * KS + (((2 * lg + 1) ^ swz_a(l16)) << 4);
    const int b_base = (lg >> 1) * BH * 1024 + l16 * 64;
    const int b_lo = b_base + (((2 * (lg & 1)) ^ swz_b(l16)) << 4);
    const int b_hi = b_base + (((2 * (lg & 1) + 1) ^ swz_b(l16)) << 4);
    auto read_a = [&](const uint8_t* as, int i) __attribute__((always_inline)) {
        const uint4 lo = *reinterpret_cast<const uint4*>(as + a_lo + i * 16 * KS);
        const uint4 hi = *reinterpret_cast<const uint4*>(as + a_hi + i * 16 * KS);
        return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    auto read_b = [&](const uint8_t* bs, int j) __attribute__((always_inline)) {
        const uint4 lo = *reinterpret_cast<const uint4*>(bs + b_lo + j * 1024);
        const uint4 hi = *reinterpret_cast<const uint4*>(bs + b_hi + j * 1024);
        return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                   (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };

    v4f acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
            asm volatile("" : "+a"(acc[i][j]));
        }
    asm volatile("s_nop 4");
    v8i fr_a[2][MT], fr_b[RING];

    // One wave's step u of the 6-step period: A of local step i+2 goes out
    // in the first two slabs, B of step i+3 in the last two (after the
    // "mid" wait, once this wave's reads of that slot are done).
    auto step = [&](auto U, int i) __attribute__((always_inline)) {
        constexpr int u = decltype(U)::value;
        constexpr int cur = u & 1;
        const uint8_t* const na = a_slot((u + 1) % 2);
        const uint8_t* const cb = b_slot(u % 3);
        const uint8_t* const nb = b_slot((u + 1) % 3);
        uint8_t* const fa = a_slot(u % 2);
        uint8_t* const fb = b_slot(u % 3);
        if constexpr (kLdsPoison) {
            // this wave's A slot u % 2 (read during its previous step) takes
            // A of its step i + 2 from here on
#pragma unroll
            for (int p = 0; p < NA; ++p) poison_block(fa + p * 1024);
            poison_done();
        }
        [&]<int... Js>(std::integer_sequence<int, Js...>) __attribute__((always_inline)) {
            ([&]() __attribute__((always_inline)) {
                constexpr int j = Js;
                constexpr int g = u * NT + j;
                constexpr int NE = NT - 2;
                constexpr int pa0 = j < NE ? j * NA / NE : 0;
                constexpr int pa1 = j < NE ? (j + 1) * NA / NE : 0;
                constexpr int pb0 = j < NE ? 0 : (j - NE) * NB / 2;
                constexpr int pb1 = j < NE ? 0 : (j - NE + 1) * NB / 2;
                if constexpr (j == NE) {
                    wait_counts<NA + NB, 0>();
                    if constexpr (kLdsPoison) {
                        // this wave's B slot u % 3 (read up to here) takes B
                        // of its step i + 3 from here on
#pragma unroll
                        for (int p = 0; p < NB; ++p) poison_block(fb + p * 1024);
                        poison_done();
                    }
                }
                constexpr int NPA = pa1 - pa0, NPB = pb1 - pb0;
                constexpr int NITEM = 1 + 1 + NPA + NPB;
                auto side = [&](auto Q) __attribute__((always_inline)) {
                    constexpr int q = decltype(Q)::value;
                    if constexpr (q == 0) {
                        fr_a[cur ^ 1][j] = read_a(na, j);
                    } else if constexpr (q == 1) {
                        if constexpr (j + 2 < NT)
                            fr_b[(g + 2) % RING] = read_b(cb, j + 2);
                        else
                            fr_b[(g + 2) % RING] = read_b(nb, j + 2 - NT);
                    } else if constexpr (q < 2 + NPA) {
                        issue_a(i + 2, pa0 + q - 2, fa);
                    } else if constexpr (q < NITEM) {
                        issue_b(i + 3, pb0 + q - 2 - NPA, fb);
                    }
                };
                __builtin_amdgcn_sched_barrier(0);
                [&]<int... Qs>(std::integer_sequence<int, Qs...>) __attribute__((always_inline)) {
                    ([&]() __attribute__((always_inline)) {
                        constexpr int q = Qs;
                        if constexpr (q < MT)
                            asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0"
                                         : "+a"(acc[q][j])
                                         : "v"(fr_b[g % RING]), "v"(fr_a[cur][q]));
                        __builtin_amdgcn_sched_barrier(0);
                        side(std::integral_constant<int, q>{});
                        __builtin_amdgcn_sched_barrier(0);
                    }(), ...);
                }(std::make_integer_sequence<int, (MT > NITEM ? MT : NITEM)>{});
                __builtin_amdgcn_sched_barrier(0);
            }(), ...);
        }(std::make_integer_sequence<int, NT>{});
    };
    static_assert(MT == NT, "one A fragment read per slab");

    if (nsteps > 0) {
#pragma unroll
        for (int p = 0; p < NB; ++p) issue_b(0, p, b_slot(0));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < NA; ++p) issue_a(0, p, a_slot(0));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < NB; ++p) issue_b(1, p, b_slot(1));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < NA; ++p) issue_a(1, p, a_slot(1));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < NB; ++p) issue_b(2, p, b_slot(2));
        __builtin_amdgcn_sched_barrier(0);
        wait_counts<NA + 2 * NB, 0>();                 // A0, B0
#pragma unroll
        for (int i = 0; i < MT; ++i) fr_a[0][i] = read_a(a_slot(0), i);
        fr_b[0] = read_b(b_slot(0), 0);
        fr_b[1] = read_b(b_slot(0), 1);
        constexpr int P = 6;
        int i0 = 0;
        for (; i0 + P <= nsteps; i0 += P) {
            [&]<int... Us>(std::integer_sequence<int, Us...>) __attribute__((always_inline)) {
                ((wait_counts<NB, 0>(), step(std::integral_constant<int, Us>{}, i0 + Us)), ...);
            }(std::make_integer_sequence<int, P>{});
        }
        const int rem = __builtin_amdgcn_readfirstlane(nsteps - i0);
        [&]<int... Us>(std::integer_sequence<int, Us...>) __attribute__((always_inline)) {
            (([&]() __attribute__((always_inline)) {
                 if (Us < rem) {
                     wait_counts<NB, 0>();
                     step(std::integral_constant<int, Us>{}, i0 + Us);
                 }
             }()),
             ...);
        }(std::make_integer_sequence<int, P - 1>{});
    }
    wait_counts<0, 0>();
    lds_barrier();
    // The accumulators are read right below: keep 24 wait states between
    // the last MFMA and the first read (the reads follow the empty asms,
    // which follow the nops).
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) asm volatile("" : "+a"(acc[i][j]));

    // Partial tiles to LDS (over the B slots of all waves: 16 KB per wave),
    // then row slab v of the sum for wave v, added in wave order.
    auto red = [&](int w) __attribute__((always_inline)) -> float* {
        return reinterpret_cast<float*>(w < 2 ? &b_s0[0][0] + w * 16384
                                              : &b_s1[0][0] + (w - 2) * 16384);
    };
    {
        float* const r = red(wave);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) r[((i * NT + j) * 4 + e) * 64 + lane] = acc[i][j][e];
    }
    __syncthreads();
    float sum[NT][4];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int idx = ((wave * NT + j) * 4 + e) * 64 + lane;
            float v = red(0)[idx];
#pragma unroll
            for (int w = 1; w < NW; ++w) v += red(w)[idx];
            sum[j][e] = v;
        }

    // Epilogue of row slab `wave` (lane l: token row l%16, columns
    // 16j + 4(l/16) .. +3), as in gemm16_kernel.
    const int64_t row = m0 + wave * 16 + l16;
    if constexpr (FUSED) {
        constexpr int PITCH = BN * 2;                 // 128-byte staged rows
        constexpr int NC = BN / 8;                    // 16-byte chunks per row
        constexpr int RB = 256 / PITCH;
        constexpr int NSTORE = 16 * NC / 64;
        auto slot_of = [](int r, int c) { return c ^ ((r / RB) % NC); };
        const float sx =
            (scale_mode == kUnitScales || row >= T) ? 1.0f : dx[scale_mode ? 0 : row];
        uint8_t* const stage = a_s0[wave];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int64_t col = n0 + j * 16 + 4 * lg;
            const float4 sw = col < Co ? scale_of_cols(dw, col, scale_mode)
                                       : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
            uint2 pk;
            pk.x = f32x2_to_bf16x2_rne((sum[j][0] * sx) * sw.x,
                   (sum[j][1] * sx) * sw.y);
            pk.y = f32x2_to_bf16x2_rne((sum[j][2] * sx) * sw.z,
                   (sum[j][3] * sx) * sw.w);
            *reinterpret_cast<uint2*>(stage + l16 * PITCH + (slot_of(l16, 2 * j + (lg >> 1)) << 4) +
                                      (lg & 1) * 8) = pk;
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        const __amdgpu_buffer_rsrc_t ro =
            make_rsrc(reinterpret_cast<uint16_t*>(out) + m0 * ldo, (uint32_t)(a_rows * ldo * 2));
#pragma unroll
        for (int q = 0; q < NSTORE; ++q) {
            const int idx = q * 64 + lane;
            const int rr = idx / NC, cc = idx % NC;
            const uint4 v = *reinterpret_cast<const uint4*>(stage + rr * PITCH +
                                                            (slot_of(rr, cc) << 4));
            const int64_t lrow = wave * 16 + rr;
            const int64_t gcol = n0 + cc * 8;
            const uint32_t off = gcol < Co ? (uint32_t)((lrow * ldo + gcol) * 2) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b128(v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w},
                                                   ro, off, 0, 0);
        }
    } else {
        if (row < T) {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int64_t col = n0 + j * 16 + 4 * lg;
                if (col < Co)
                    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + row * Co + col) =
                        make_float4(sum[j][0], sum[j][1], sum[j][2], sum[j][3]);
            }
        }
    }
}

// Few tokens (T <= 64): the GEMM is a weight stream, bound by HBM.  A
// workgroup owns NT*32 output columns and all T rows (MT = ceil(T/32) row
// tiles of 32); its NWAVE waves split the K steps (wave w takes steps w,
// w+NWAVE, ...), each loading its share of the 2*NT packed 1 KB blocks per
// step straight into MFMA operand registers (no LDS), DEPTH steps ahead.  The
// partial sums meet in LDS and are added in wave order, then the epilogue is
// the one of the tiled kernel: scales in registers, one store per output.
// Operand loads past the data (rows >= T, K >= Ci, columns >= Co, steps >=
// the last) are range-checked to zero.
template <int MT, int NT, int NWAVE, int DEPTH, bool FUSED>
__global__ __launch_bounds__(NWAVE * 64, 1) void gemm_decode_kernel(
    const uint8_t* __restrict__ qx, int64_t ldq, const float* __restrict__ dx,
    const uint8_t* __restrict__ wp, int64_t Kp, const float* __restrict__ dw,
    int64_t T, int64_t Ci, int64_t Co, void* __restrict__ out, int64_t ldo, int scale_mode) {
    static_assert(NWAVE * NT * MT * 16 * 64 * 4 <= 160 * 1024, "partial sums exceed LDS");
    __shared__ float red[NWAVE][NT * MT][16][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 31, lg = lane >> 5;
    const int64_t n0 = (int64_t)blockIdx.x * (32 * NT);
    const int nks = (int)(Kp / BK);
    const int g0 = (int)(n0 >> 4);                      // first 16-column block

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(qx, (uint32_t)(T * ldq));
    const int64_t gblocks = (Co >> 4) - g0;             // packed blocks left from g0
    const int gb = gblocks < 2 * NT ? (int)gblocks : 2 * NT;
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(wp + (int64_t)g0 * nks * 1024, (uint32_t)(gb * nks * 1024));

    // B operand of column tile j: column l%32 -> block 2j + l%32/16, row r in
    // the block; logical chunks 2*(l/32) and 2*(l/32)+1 of the step, at their
    // packed units.
    const int r = lr & 15;
    uint32_t b_lo[NT], b_hi[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int blk = 2 * j + (lr >> 4);
        b_lo[j] = (uint32_t)(blk * nks * 1024 + (4 * r + ((2 * lg) ^ ((r >> 2) & 3))) * 16);
        b_hi[j] = (uint32_t)(blk * nks * 1024 + (4 * r + ((2 * lg + 1) ^ ((r >> 2) & 3))) * 16);
    }
    // A operand: token row i*32 + l%32, 32 bytes at 32*(l/32) of the step.
    uint32_t a_base[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int64_t t = i * 32 + lr;
        a_base[i] = (t < T) ? (uint32_t)(t * ldq + 32 * lg) : kOutOfRange;
    }

    v4i fb[DEPTH][NT][2], fa[DEPTH][MT][2];
    auto load = [&](int slot_u, int ks) {
        const bool kin = ks < nks;
        const uint32_t kb = (uint32_t)ks * 1024u;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            fb[slot_u][j][0] =
                __builtin_amdgcn_raw_buffer_load_b128(rb, kin ? b_lo[j] + kb : kOutOfRange, 0, 0);
            fb[slot_u][j][1] =
                __builtin_amdgcn_raw_buffer_load_b128(rb, kin ? b_hi[j] + kb : kOutOfRange, 0, 0);
        }
        const int64_t k = (int64_t)ks * BK + 32 * lg;    // this lane's 32 A bytes start here
        const bool ain = kin && k < Ci;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const bool ok = ain && a_base[i] != kOutOfRange;
            const uint32_t off = ok ? a_base[i] + (uint32_t)ks * BK : kOutOfRange;
            fa[slot_u][i][0] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
            fa[slot_u][i][1] = __builtin_amdgcn_raw_buffer_load_b128(
                ra, (ok && k + 16 < Ci) ? off + 16 : kOutOfRange, 0, 0);
        }
    };

    v16f acc[NT][MT];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.0f;

    // The scales of the runs this wave stores at the end (see the epilogue),
    // loaded before the K loop so that their latency hides behind it.
    constexpr int NPW = (NT * MT * 4 + NWAVE - 1) / NWAVE;   // runs per wave
    float sxp[NPW];
    float4 swp[NPW];
#pragma unroll
    for (int k = 0; k < NPW; ++k) {
        const int p = wave + k * NWAVE;
        const int ji = p >> 2, g = p & 3;
        const int j = ji / MT, i = ji - j * MT;
        const int64_t row = i * 32 + lr;
        const int64_t c = n0 + 32 * j + 8 * g + 4 * lg;
        const bool ok = FUSED && p < NT * MT * 4 && row < T && c < Co;
        sxp[k] = (!ok || scale_mode == kUnitScales) ? 1.0f : dx[scale_mode ? 0 : row];
        swp[k] = ok ? scale_of_cols(dw, c, scale_mode) : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
    }
    const int count = (nks - wave + NWAVE - 1) / NWAVE;  // steps of this wave
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) load(u, wave + NWAVE * u);
    for (int it = 0; it < count; it += DEPTH) {
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const v8i bf = v8i{fb[u][j][0].x, fb[u][j][0].y, fb[u][j][0].z, fb[u][j][0].w,
                                   fb[u][j][1].x, fb[u][j][1].y, fb[u][j][1].z, fb[u][j][1].w};
#pragma unroll
                for (int i = 0; i < MT; ++i) {
                    const v8i af =
                        v8i{fa[u][i][0].x, fa[u][i][0].y, fa[u][i][0].z, fa[u][i][0].w,
                            fa[u][i][1].x, fa[u][i][1].y, fa[u][i][1].z, fa[u][i][1].w};
                    acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        bf, af, acc[j][i], 0, 0, 0, 0, 0, 0);
                }
            }
            load(u, wave + NWAVE * (it + u + DEPTH));
        }
    }

    // Sum the partials in wave order.  The (column tile, row tile, 4-column
    // run) triples are dealt round-robin to the waves: run g of tile (j, i)
    // covers columns 32j + 8g + 4*(l/32) + 0..3 of the workgroup's, token
    // row 32i + l%32.
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) red[wave][j * MT + i][e][lane] = acc[j][i][e];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NPW; ++k) {
        const int p = wave + k * NWAVE;
        if (p >= NT * MT * 4) break;
        const int ji = p >> 2, g = p & 3;
        const int j = ji / MT, i = ji - j * MT;
        const int64_t row = i * 32 + lr;
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = 4 * g + q;
            float sum = red[0][ji][e][lane];
#pragma unroll
            for (int w = 1; w < NWAVE; ++w) sum += red[w][ji][e][lane];
            v[q] = sum;
        }
        const int64_t c = n0 + 32 * j + 8 * g + 4 * lg;
        if (row >= T || c >= Co) continue;
        if constexpr (FUSED) {
            const float sx = sxp[k];
            const float4 sw = swp[k];
            uint2 pk;
            pk.x = f32x2_to_bf16x2_rne((v[0] * sx) * sw.x,
                   (v[1] * sx) * sw.y);
            pk.y = f32x2_to_bf16x2_rne((v[2] * sx) * sw.z,
                   (v[3] * sx) * sw.w);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + row * ldo + c) = pk;
        } else {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + row * Co + c) =
                make_float4(v[0], v[1], v[2], v[3]);
        }
    }
}

template <int MT, int NT, int NWAVE, int DEPTH>
static hipError_t launch_decode(const uint8_t* qx, int64_t ldq, const float* dx, const uint8_t* wp,
                                const float* dw, int64_t T, int64_t Ci, int64_t Co, uint16_t* out,
                                int64_t ldo, float* fp32_out, hipStream_t s, int mode) {
    const dim3 grid((unsigned)((Co + 32 * NT - 1) / (32 * NT)));
    const int64_t Kp = round_up_k(Ci);
    if (fp32_out == nullptr) {
        hipLaunchKernelGGL((gemm_decode_kernel<MT, NT, NWAVE, DEPTH, true>), grid,
                           dim3(NWAVE * 64), 0, s, qx, ldq, dx, wp, Kp, dw, T, Ci, Co, (void*)out,
                           ldo, mode);
    } else {
        hipLaunchKernelGGL((gemm_decode_kernel<MT, NT, NWAVE, DEPTH, false>), grid,
                           dim3(NWAVE * 64), 0, s, qx, ldq, dx, wp, Kp, dw, T, Ci, Co,
                           (void*)fp32_out, Co, 0);
    }
    return hipGetLastError();
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
        packed.x = f32x2_to_bf16x2_rne((a.x * st) * s.x,
                   (a.y * st) * s.y);
        packed.y = f32x2_to_bf16x2_rne((a.z * st) * s.z,
                   (a.w * st) * s.w);
        *reinterpret_cast<uint2*>(out + t * ldo + o) = packed;
    }
}

// Step 2 of the bf16-intermediate two-step form: the unscaled result was
// rounded to bf16 by step 1; scale it and round again.
__global__ __launch_bounds__(256) void rescale_bf16_kernel(const uint16_t* __restrict__ ws,
                                                           const float* __restrict__ dx,
                                                           const float* __restrict__ dw,
                                                           int64_t T, int64_t Co,
                                                           uint16_t* __restrict__ out,
                                                           int64_t ldo) {
    const int64_t per_row = Co / 4;
    const int64_t n = T * per_row;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = i / per_row;
        const int64_t o = (i - t * per_row) * 4;
        const uint2 a = *reinterpret_cast<const uint2*>(ws + t * Co + o);
        const float4 sc = *reinterpret_cast<const float4*>(dw + o);
        const float st = dx[t];
        uint2 packed;
        packed.x = f32x2_to_bf16x2_rne((bf16lo_to_f32(a.x) * st) * sc.x,
                   (bf16hi_to_f32(a.x) * st) * sc.y);
        packed.y = f32x2_to_bf16x2_rne((bf16lo_to_f32(a.y) * st) * sc.z,
                   (bf16hi_to_f32(a.y) * st) * sc.w);
        *reinterpret_cast<uint2*>(out + t * ldo + o) = packed;
    }
}

// Split-K epilogue: the partial sums of the S K ranges, added in range order
// (so the result does not depend on timing), then scaled and rounded once.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws,
                                                            int splits,
                                                            const float* __restrict__ dx,
                                                            const float* __restrict__ dw,
                                                            int64_t T, int64_t Co,
                                                            uint16_t* __restrict__ out,
                                                            int64_t ldo) {
    const int64_t per_row = Co / 4;
    const int64_t n = T * per_row;
    const int64_t slice = T * Co;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = i / per_row;
        const int64_t o = (i - t * per_row) * 4;
        float4 a = *reinterpret_cast<const float4*>(ws + t * Co + o);
        for (int k = 1; k < splits; ++k) {
            const float4 b = *reinterpret_cast<const float4*>(ws + k * slice + t * Co + o);
            a.x += b.x;
            a.y += b.y;
            a.z += b.z;
            a.w += b.w;
        }
        const float4 sc = *reinterpret_cast<const float4*>(dw + o);
        const float st = dx[t];
        uint2 packed;
        packed.x = f32x2_to_bf16x2_rne((a.x * st) * sc.x,
                   (a.y * st) * sc.y);
        packed.y = f32x2_to_bf16x2_rne((a.z * st) * sc.z,
                   (a.w * st) * sc.w);
        *reinterpret_cast<uint2*>(out + t * ldo + o) = packed;
    }
}

template <int BM, int BN, int WM, int WN, int NB, bool NTB = false>
static hipError_t launch_tiles(const uint8_t* qx, int64_t ldq, const float* dx, const uint8_t* wp,
                               const float* dw, int64_t T, int64_t Ci, int64_t Co, uint16_t* out,
                               int64_t ldo, float* fp32_out, hipStream_t s, int mode,
                               int splits = 1) {
    const dim3 grid((unsigned)(((Co + BN - 1) / BN) * ((T + BM - 1) / BM) * splits));
    const int64_t Kp = round_up_k(Ci);
    if (fp32_out == nullptr) {
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, NB, true, NTB>), grid, dim3(WM * WN * 64), 0, s,
                           qx, ldq, dx, wp, Kp, dw, T, Ci, Co, (void*)out, ldo, mode, 1);
    } else {
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, NB, false, NTB>), grid, dim3(WM * WN * 64), 0, s,
                           qx, ldq, dx, wp, Kp, dw, T, Ci, Co, (void*)fp32_out, Co, 0, splits);
    }
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
static hipError_t launch_tiles16(const uint8_t* qx, int64_t ldq, const float* dx, const uint8_t* wp,
                                 const float* dw, int64_t T, int64_t Ci, int64_t Co, uint16_t* out,
                                 int64_t ldo, float* fp32_out, hipStream_t s, int mode,
                                 int splits = 1) {
    const dim3 grid((unsigned)(((Co + BN - 1) / BN) * ((T + BM - 1) / BM) * splits));
    const int64_t Kp = round_up_k(Ci);
    if (fp32_out == nullptr) {
        hipLaunchKernelGGL((gemm16_kernel<BM, BN, WM, WN, true>), grid, dim3(WM * WN * 64), 0, s,
                           qx, ldq, dx, wp, Kp, dw, T, Ci, Co, (void*)out, ldo, mode, 1,
                           (float*)nullptr);
    } else {
        hipLaunchKernelGGL((gemm16_kernel<BM, BN, WM, WN, false>), grid, dim3(WM * WN * 64), 0, s,
                           qx, ldq, dx, wp, Kp, dw, T, Ci, Co, (void*)fp32_out, Co, 0, splits,
                           (float*)nullptr);
    }
    return hipGetLastError();
}

// Clears the tile records of the two-range fix-up.
__global__ __launch_bounds__(256) void clear_records_kernel(uint32_t* __restrict__ p, int n) {
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n) p[i] = 0u;
}

static hipError_t launch_tiles16s(const uint8_t* qx, int64_t ldq, const float* dx,
                                  const uint8_t* wp, const float* dw, int64_t T, int64_t Ci,
                                  int64_t Co, uint16_t* out, int64_t ldo, float* fp32_out,
                                  hipStream_t s, int mode) {
    const dim3 grid((unsigned)(((Co + 63) / 64) * ((T + 63) / 64)));
    const int64_t Kp = round_up_k(Ci);
    if (fp32_out == nullptr) {
        hipLaunchKernelGGL((gemm16s_kernel<true>), grid, dim3(256), 0, s, qx, ldq, dx, wp, Kp,
                           dw, T, Ci, Co, (void*)out, ldo, mode);
    } else {
        hipLaunchKernelGGL((gemm16s_kernel<false>), grid, dim3(256), 0, s, qx, ldq, dx, wp, Kp,
                           dw, T, Ci, Co, (void*)fp32_out, Co, 0);
    }
    return hipGetLastError();
}

static hipError_t launch_main(const uint8_t* qx, int64_t ldq, const float* dx, const uint8_t* wp,
                              const float* dw, int64_t T, int64_t Ci, int64_t Co, uint16_t* out,
                              int64_t ldo, float* fp32_out, hipStream_t s, int ts) {
    switch (gemm_plan(T, Ci, Co)) {
        case GemmPlan::k16_256x256:
            return launch_tiles16<256, 256, 2, 2>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s, ts);
        case GemmPlan::k16_192x256:
            return launch_tiles16<192, 256, 2, 2>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s, ts);
        case GemmPlan::k16_256x224:
            return launch_tiles16<256, 224, 4, 1>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s, ts);
        case GemmPlan::k16_256x160:
            return launch_tiles16<256, 160, 2, 2>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s, ts);
        case GemmPlan::k16_128x256:
            return launch_tiles16<128, 256, 2, 2>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s, ts);
        case GemmPlan::k16_128x224:
            return launch_tiles16<128, 224, 2, 2>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s, ts);
        case GemmPlan::k16_128x128:
            return launch_tiles16<128, 128, 2, 2>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s, ts);
        case GemmPlan::k16s_64x64:
            return launch_tiles16s(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s, ts);
        case GemmPlan::k32_64x64:
            return launch_tiles<64, 64, 2, 2, 4>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s, ts);
        case GemmPlan::k32_64x128:
            return launch_tiles<64, 128, 2, 2, 4>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s, ts);
        case GemmPlan::k32_128x128:   // 33..64 tokens: one row tile
            return launch_tiles<128, 128, 2, 2, 4, true>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s, ts);
        case GemmPlan::k32_32x64:     // 9..32 tokens: one row tile
            return launch_tiles<32, 64, 1, 2, 4, true>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s, ts);
        case GemmPlan::kDecode_2x2:
            return launch_decode<2, 2, 4, 4>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s, ts);
        case GemmPlan::kDecode_2x1:
            return launch_decode<2, 1, 4, 4>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s, ts);
        case GemmPlan::kDecode_1x2:
            return launch_decode<1, 2, 4, 4>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s, ts);
        case GemmPlan::kDecode_1x1:
            return launch_decode<1, 1, 4, 4>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s, ts);
    }
    return hipErrorInvalidValue;
}

static int64_t rescale_blocks(int64_t T, int64_t Co) {
    const int64_t n = T * (Co / 4);
    int64_t blocks = (n + 255) / 256;
    return blocks > 65536 ? 65536 : blocks;
}

hipError_t launch_gemm(const uint8_t* qx, int64_t ldq, const float* dx, const uint8_t* wp,
                       const float* dw, int64_t T, int64_t Ci, int64_t Co, uint16_t* out,
                       int64_t ldo, float* fp32_out, hipStream_t s, bool per_tensor) {
    const hipError_t e = launch_main(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, fp32_out, s,
                                     per_tensor ? kTensorScales : kTokenChannelScales);
    if (e != hipSuccess || fp32_out == nullptr) return e;
    hipLaunchKernelGGL(rescale_kernel, dim3((unsigned)rescale_blocks(T, Co)), dim3(256), 0, s,
                       fp32_out, dx, dw, T, Co, out, ldo);
    return hipGetLastError();
}

hipError_t launch_gemm_splitk(const uint8_t* qx, int64_t ldq, const float* dx, const uint8_t* wp,
                              const float* dw, int64_t T, int64_t Ci, int64_t Co, uint16_t* out,
                              int64_t ldo, float* ws, int splits, hipStream_t s) {
    if (gemm_split_fixup(T, Ci, Co)) {
        // Two K ranges of 256x256 tiles joined inside the GEMM kernel: tile
        // slots of fp32 sums, then 4 record words per tile, cleared first.
        const int ntiles = (int)(((T + 255) / 256) * ((Co + 255) / 256));
        uint32_t* const rec = reinterpret_cast<uint32_t*>(ws + (int64_t)ntiles * 256 * 256);
        hipLaunchKernelGGL(clear_records_kernel, dim3((unsigned)((4 * ntiles + 255) / 256)),
                           dim3(256), 0, s, rec, 4 * ntiles);
        hipLaunchKernelGGL((gemm16_kernel<256, 256, 2, 2, true, true>), dim3((unsigned)(2 * ntiles)),
                           dim3(256), 0, s, qx, ldq, dx, wp, round_up_k(Ci), dw, T, Ci, Co,
                           (void*)out, ldo, (int)kTokenChannelScales, 2, ws);
        return hipGetLastError();
    }
    // 256x256 tiles of the 16x16x128 kernel (from 256 tokens on, and some
    // shapes of 129..255 tokens) or 128x128 tiles of the 32x32x64 kernel
    const hipError_t e =
        gemm_split_tiles256(T, Ci, Co) ? launch_tiles16<256, 256, 2, 2>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, ws, s,
                                                  kTokenChannelScales, splits)
        : Ci >= kLongK ? launch_tiles<128, 128, 2, 2, 4, true>(qx, ldq, dx, wp, dw, T, Ci, Co, out,
                                                               ldo, ws, s, kTokenChannelScales, splits)
                       : launch_tiles<128, 128, 2, 2, 4>(qx, ldq, dx, wp, dw, T, Ci, Co, out, ldo, ws,
                                                         s, kTokenChannelScales, splits);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)rescale_blocks(T, Co)), dim3(256), 0,
                       s, ws, splits, dx, dw, T, Co, out, ldo);
    return hipGetLastError();
}

// Scratch of ptpc_gemm_noalloc (for callers that cannot allocate): the fp32
// partial sums of the split-K form live in this file-scope device array
// instead of a caller workspace.  Each GPU holds its own copy for the life of
// the process.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in, not a device address): the device address is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and kept.  Every split range writes its whole slice, so nothing
// needs clearing between calls; calls that overlap on one GPU share the
// array and race.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

#ifdef PTPC_TIMELINE
extern "C" int ptpc_debug_set_timeline(void* buf) {
    return (int)hipMemcpyToSymbol(HIP_SYMBOL(g_timeline), &buf, sizeof(buf));
}
#endif

hipError_t noalloc_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_gemm_unfused_bf16(const uint8_t* qx, int64_t ldq, const float* dx,
                                    const uint8_t* wp, const float* dw, int64_t T, int64_t Ci,
                                    int64_t Co, uint16_t* out, int64_t ldo, uint16_t* ws,
                                    hipStream_t s) {
    const hipError_t e =
        launch_main(qx, ldq, dx, wp, dw, T, Ci, Co, ws, Co, nullptr, s, kUnitScales);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(rescale_bf16_kernel, dim3((unsigned)rescale_blocks(T, Co)), dim3(256), 0,
                       s, ws, dx, dw, T, Co, out, ldo);
    return hipGetLastError();
}

}  // namespace ptpc
