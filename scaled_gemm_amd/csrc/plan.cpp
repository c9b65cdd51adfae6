// Kernel choice of libptpc, made on the host from the extents alone: which
// GEMM kernel and tile, the split-K plan of ptpc_gemm_ws, and the launch shape
// of the activation quantizer.  Plain host C++ (no device code), shared by
// the launchers and the diagnostic queries of the C ABI.
#include "kernels.h"

namespace ptpc {

// Time of one tile relative to a 256x256 tile at the same K, measured with
// every operand streamed from HBM (inputs rotated over copies larger than the
// memory-side cache, as a layer's weight arrives in a model's forward pass):
// one round of tiles of each shape on the 70B O, down and QKV layers at 1024
// tokens (the three layers agree within 0.02), and 128x128 per round on the
// same layers' two- and three-round grids.
constexpr double kCost256x224 = 0.94;
constexpr double kCost192x256 = 0.85;
constexpr double kCost256x160 = 0.90;
constexpr double kCost128x256 = 0.75;    // 256x128 tiles, the same count, cost 0.88
constexpr double kCost128x128 = 0.42;

// 65..128 tokens where the tile rule below picks 64x64 tiles: those run
// gemm16s_kernel (K split inside the workgroup), which needs no workspace
// and is not split further across workgroups.
static bool split16_tiles(int64_t T, int64_t Co) {
    if (T <= 64 || T > 128) return false;
    auto rounds = [](int64_t tiles) { return (tiles + kCus - 1) / kCus; };
    auto tiles = [&](int64_t bm, int64_t bn) { return ((T + bm - 1) / bm) * ((Co + bn - 1) / bn); };
    const int64_t r64 = rounds(tiles(64, 64));
    return r64 <= rounds(tiles(128, 128)) && r64 <= rounds(tiles(64, 128));
}

GemmPlan gemm_plan(int64_t T, int64_t Ci, int64_t Co) {
    auto rounds = [](int64_t tiles) { return (tiles + kCus - 1) / kCus; };
    auto tiles = [&](int64_t bm, int64_t bn) { return ((T + bm - 1) / bm) * ((Co + bn - 1) / bn); };
    if (T >= 256) {
        // Each tile shape costs (rounds of 256 CUs it needs) x (its tile
        // cost); the cheapest wins, the larger tile on a tie.  256x256 keeps
        // the most MFMA work per loaded byte; the smaller tiles pay off where
        // 256x256 tiles leave CUs idle or a badly filled last round (70B QKV
        // at 1024 tokens: 240 tiles of 192x256 for 160 of 256x256; O and down:
        // 256 tiles of 128x256; gate_up: 1024 of 256x224 for 3.5 rounds of
        // 256x256; 384..600 tokens of the 8192-column layers: 128x128, and
        // fewer tokens the 64x128 tiles below).
        struct Cand {
            GemmPlan plan;
            int64_t bm, bn;
            double cost;
        };
        const Cand cands[] = {
            {GemmPlan::k16_256x256, 256, 256, 1.0},
            {GemmPlan::k16_256x224, 256, 224, kCost256x224},
            {GemmPlan::k16_192x256, 192, 256, kCost192x256},
            {GemmPlan::k16_256x160, 256, 160, kCost256x160},
            {GemmPlan::k16_128x256, 128, 256, kCost128x256},
            {GemmPlan::k16_128x128, 128, 128, kCost128x128},
        };
        GemmPlan best = GemmPlan::k16_256x256;
        double best_cost = 1e300;
        for (const Cand& c : cands) {
            const double cost = c.cost * (double)rounds(tiles(c.bm, c.bn));
            if (cost < best_cost) {
                best_cost = cost;
                best = c.plan;
            }
        }
        // 128x128 tiles that leave CUs idle (256..~600 tokens with few output
        // columns): 64x128 tiles of the 32x32x64 kernel instead.  Each moves a
        // quarter fewer operand bytes, and two of its workgroups share a CU
        // (56 KB of LDS, 136 registers per lane; the 16x16x128 kernel's
        // 128x128 workgroup needs 264), so up to 512 run at once.  Cold-timed:
        // the 70B O / QKV / down and 8B down layers at 256 tokens 1.45 / 1.24 /
        // 1.53 / 1.56x faster, the 8B down layer at 384 and 512 tokens 1.56x,
        // the 70B O and down layers at 384 tokens 1.04x and level.
        if (best == GemmPlan::k16_128x128 && tiles(128, 128) < kCus && tiles(64, 128) <= 2 * kCus)
            return GemmPlan::k32_64x128;
        return best;
    }
    if (T > 64) {
        // 65..255 tokens: the fewest rounds of 256 CUs, and among equal
        // rounds the smaller tile (more CUs streaming the weight): 128x128
        // tiles leave most CUs idle on the 8192-column layers.  64x64 tiles
        // of up to 128 tokens (two row tiles) run gemm16s_kernel, the K
        // steps split between the waves: 19-48% faster than the same tiles
        // with a barrier per 64-byte step.  Where the rule picks larger
        // tiles the split kernel's 64x64 tiles would double the operand
        // traffic into LDS and lose (70B gate_up at 128 tokens: 1.5x slower).
        const int64_t r128 = rounds(tiles(128, 128)), r64w = rounds(tiles(64, 128));
        const int64_t r64 = rounds(tiles(64, 64));
        if (split16_tiles(T, Co)) return GemmPlan::k16s_64x64;
        if (r64 <= r128 && r64 <= r64w) return GemmPlan::k32_64x64;
        if (r64w <= r128) return GemmPlan::k32_64x128;
        // Wide layers whose 128x128 tiles need more than one round: one row
        // tile of 224 columns (rows past T read as zero) where those fill
        // more than half the CUs in one round -- the weight is read once,
        // by every CU at once.  Cold-timed on the 70B gate_up layer (57344
        // columns, 256 such tiles) at 96 / 128 / 160 / 200 / 255 tokens:
        // 5 / 9 / 21 / 19 / 18% faster than 128x128 tiles; level at 72; on
        // the 8B gate_up layer (128 tiles, half the CUs) 4-10% slower.
        const int64_t wide = (Co + 223) / 224;
        if (T > 80 && r128 > 1 && wide <= kCus && 2 * wide > kCus)
            return T <= 128 ? GemmPlan::k16_128x224 : GemmPlan::k16_256x224;
        return GemmPlan::k16_128x128;   // the 16x16x128 kernel, 3-5% faster here (70B gate_up)
    }
    // Up to 64 tokens the weight stream decides.  The tiled kernel reads
    // each weight byte once per row tile and keeps the activation in LDS, but
    // with few column tiles it leaves CUs idle; the few-token kernel splits K
    // inside a workgroup instead.  It is taken unless the tiled grid has at
    // least two workgroups per CU (32x64 tiles) or one (128x128 tiles): the
    // crossover measured on the 8B / 70B projection shapes.  Its 64-column
    // form (half the activation re-reads) pays off from 16 tokens on, once
    // the 32-column grid no longer fits the CUs in one round.
    if (T > 32 && (Co + 127) / 128 >= kCus) return GemmPlan::k32_128x128;
    if (T > 32 && (Co + 31) / 32 > kCus) return GemmPlan::kDecode_2x2;
    if (T > 32) return GemmPlan::kDecode_2x1;
    if (T > 8 && (Co + 63) / 64 >= 2 * kCus) return GemmPlan::k32_32x64;
    if (T > 8 && (Co + 31) / 32 > kCus) return GemmPlan::kDecode_1x2;
    return GemmPlan::kDecode_1x1;
}

const char* gemm_plan_name(GemmPlan p) {
    switch (p) {
        case GemmPlan::k16_256x256: return "gemm16_kernel<256,256,2,2>";
        case GemmPlan::k16_192x256: return "gemm16_kernel<192,256,2,2>";
        case GemmPlan::k16_256x224: return "gemm16_kernel<256,224,4,1>";
        case GemmPlan::k16_256x160: return "gemm16_kernel<256,160,2,2>";
        case GemmPlan::k16_128x256: return "gemm16_kernel<128,256,2,2>";
        case GemmPlan::k16_128x128: return "gemm16_kernel<128,128,2,2>";
        case GemmPlan::k16_128x224: return "gemm16_kernel<128,224,2,2>";
        case GemmPlan::k16s_64x64: return "gemm16s_kernel";
        case GemmPlan::k32_64x64: return "gemm_kernel<64,64,2,2,4>";
        case GemmPlan::k32_64x128: return "gemm_kernel<64,128,2,2,4>";
        case GemmPlan::k32_128x128: return "gemm_kernel<128,128,2,2,4>";
        case GemmPlan::k32_32x64: return "gemm_kernel<32,64,1,2,4>";
        case GemmPlan::kDecode_2x2: return "gemm_decode_kernel<2,2,4,4>";
        case GemmPlan::kDecode_2x1: return "gemm_decode_kernel<2,1,4,4>";
        case GemmPlan::kDecode_1x2: return "gemm_decode_kernel<1,2,4,4>";
        case GemmPlan::kDecode_1x1: return "gemm_decode_kernel<1,1,4,4>";
    }
    return nullptr;
}

// Split-K plan for shapes whose tiled grid leaves most CUs idle: 65..255
// tokens on 128x128 tiles, K cut into S ranges of at least 16 steps so that
// tiles x S fills the CUs.  Returns S (1: no split).  Where ptpc_gemm runs
// the K-split 64x64 tiles, splitting across workgroups instead pays only for
// long K: with two 64-row tiles per weight slab those tiles move twice the
// operand bytes of 128x128 tiles into LDS, which outweighs the fp32 partials'
// round trip once K is long (70B down projection, K = 28672, 72 / 128 tokens:
// 19% / 28% faster; 70B O projection, K = 8192: 6% slower).
//   From 256 tokens on, with K of at least kSplitK256 bytes: 256x256 tiles
// (the 16x16x128 kernel), K cut into S ranges of at least 8 steps of 128
// bytes, S = the largest that keeps tiles x S within one round of the CUs
// (at most 8).  ptpc_gemm's own tiles there are smaller (64x128, 128x128 or
// 128x256: more operand bytes per flop) or leave CUs idle.  Cold-timed
// against ptpc_gemm in one run, partial sums and their reduction included:
// the 70B down projection (K = 28672) at 256 / 512 / 768 / 1024 tokens
// 1.28 / 1.42 / 1.13 / 1.07x faster; the 8B one (K = 14336) at 256 and 1024
// tokens 1.39 / 1.16x and K = 12288 at 1024 tokens 1.13x, but the 8B one at
// 512 tokens, where ptpc_gemm's 64x128 tiles already give every CU one, 0.86x
// (8 ranges), and at 2048 tokens (2 ranges) 0.97x.  So below kLongK the split
// needs at least 4 ranges and a ptpc_gemm grid that leaves CUs idle.  K =
// 8192 (the 70B O projection at 512..1024 tokens) lost 5-17%, so shorter K is
// not split.  S x tiles <= 256 bounds the workspace: 4 * S * T * Co <= 4 *
// 256 * 256 * 256 bytes = 64 MiB.
// K ranges for 256x256 tiles: the most that keep tiles x S within one round
// of the CUs, at most 8, each at least 8 steps of 128 bytes.
static int64_t splits256(int64_t T, int64_t Ci, int64_t Co) {
    int64_t S = kCus / (((T + 255) / 256) * ((Co + 255) / 256));
    const int64_t n128 = round_up_k(Ci) / 128;
    if (S > n128 / 8) S = n128 / 8;
    if (S > 8) S = 8;
    return S;
}

// Whether the split runs 256x256 tiles of the 16x16x128 kernel (else 128x128
// tiles of the 32x32x64 kernel).  From 256 tokens on always; at 129..255
// tokens, where 128-row tiles read every weight byte twice and one 256-row
// tile reads it once, for long K or where ptpc_gemm itself would run 128x128
// tiles (cold, through ptpc_gemm_ws: the 70B down projection at 200 / 255
// tokens 88.0 -> 70.5 / 81.0 -> 78.4 us, the 70B QKV projection at 200
// tokens 51.1 -> 39.7 us; where ptpc_gemm runs 64-row tiles with K < 16384
// -- the 70B O layer at 144 / 200 tokens, QKV at 160, 8B down at 192 -- the
// 256x256 split was 3-20% slower).
bool gemm_split_tiles256(int64_t T, int64_t Ci, int64_t Co) {
    if (T >= 256) return true;
    if (T <= 128 || splits256(T, Ci, Co) < 2) return false;
    return Ci >= kLongK || gemm_plan(T, Ci, Co) == GemmPlan::k16_128x128;
}

int gemm_splitk_plan(int64_t T, int64_t Ci, int64_t Co) {
    if (T >= 256) {
        if (Ci < kSplitK256) return 1;
        const int64_t S = splits256(T, Ci, Co);
        if (Ci < kLongK) {
            if (S < 4) return 1;
            if (gemm_plan(T, Ci, Co) == GemmPlan::k32_64x128 &&
                ((T + 63) / 64) * ((Co + 127) / 128) >= kCus)
                return 1;
        }
        return S < 2 ? 1 : (int)S;
    }
    if (gemm_split_tiles256(T, Ci, Co)) return (int)splits256(T, Ci, Co);
    if (T <= 64 || (split16_tiles(T, Co) && Ci < kLongK)) return 1;
    const int64_t tiles = ((T + 127) / 128) * ((Co + 127) / 128);
    int64_t S = kCus / tiles;
    const int64_t nks = round_up_k(Ci) / 64;   // 64-byte K steps of the split kernel
    if (S > nks / 16) S = nks / 16;
    if (S > 8) S = 8;
    return S < 2 ? 1 : (int)S;
}

bool gemm_split_fixup(int64_t T, int64_t Ci, int64_t Co) {
    return gemm_splitk_plan(T, Ci, Co) == 2 && gemm_split_tiles256(T, Ci, Co);
}

size_t gemm_splitk_workspace_bytes(int64_t T, int64_t Ci, int64_t Co) {
    const int S = gemm_splitk_plan(T, Ci, Co);
    if (S < 2) return 0;
    if (gemm_split_fixup(T, Ci, Co)) {
        const size_t tiles = (size_t)(((T + 255) / 256) * ((Co + 255) / 256));
        return tiles * (256 * 256 * sizeof(float) + 4 * sizeof(uint32_t));
    }
    return (size_t)S * (size_t)T * (size_t)Co * sizeof(float);
}

static int pow2_ceil(int64_t v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// Launch shape of the activation quantizer for rows of Ci elements: G
// threads per row holding VPT 16-byte vectors each, or (G = 0) the two-pass
// kernel for rows longer than 256 threads x 32 vectors (65536 elements).
// Rows of 256 or more vectors get a whole 256-thread workgroup (more loads in
// flight per row beat more vectors per thread); shorter rows share a
// workgroup, about 8 vectors per thread, at least 16 threads.  Holding rows
// of up to 65536 elements in registers (32 vectors per thread, 202 VGPRs, no
// spills) reads X once where the two-pass kernel reads it twice: rows of
// 40960-65536 elements went from 3.2-3.4 to 6.0-6.2 TB/s.  Reachable shapes:
// G = 16 with VPT 1..8 (up to 128 vectors), G = 32 with VPT 8 (129..255
// vectors), G = 256 with VPT 1 or 2 (256..512 vectors), G = 128 with VPT 8
// (513..1024), G = 256 with VPT 8..32 (1025..8192), and the long-row kernel.
ActPlan act_plan(int64_t Ci) {
    const int64_t nchunk = Ci / 8;
    int64_t G = 256;
    // Rows of 513..1024 vectors: two rows per workgroup, 8 vectors per
    // thread instead of 4 (8192 tokens, each input streamed from HBM: rows of
    // 6144 elements 65.7 -> 68.9% of HBM, rows of 8192 69.1 -> 69.7% and
    // 69.9 -> 71.4% in two runs; 16 vectors per thread, for longer rows, was
    // 2-3% slower, and rows of 4096 elements lost).
    if (nchunk > 512 && nchunk <= 1024) G = 128;
    if (nchunk < 256) {
        G = pow2_ceil((nchunk + 7) / 8);
        if (G < 16) G = 16;
    }
    const int64_t per = (nchunk + G - 1) / G;
    if (per > 32) return {0, 0};
    return {(int)G, pow2_ceil(per)};
}

const char* quant_act_plan_name(int64_t T, int64_t Ci) {
    if (T <= 0) return nullptr;
    if (Ci == 0) return "fill_f32_kernel";
    const ActPlan p = act_plan(Ci);
    static const char* const names[] = {
        "quant_act_kernel<16,1>",   "quant_act_kernel<16,2>",  "quant_act_kernel<16,4>",
        "quant_act_kernel<16,8>",   "quant_act_kernel<32,8>",  "quant_act_kernel<256,1>",
        "quant_act_kernel<256,2>",  "quant_act_kernel<256,4>", "quant_act_kernel<256,8>",
        "quant_act_kernel<256,16>", "quant_act_kernel<256,32>"};
    if (p.G == 0) return "quant_act_long_kernel";
    const int lv = __builtin_ctz((unsigned)p.vpt);
    if (p.G == 16) return names[lv];
    if (p.G == 32) return names[4];
    if (p.G == 128) return "quant_act_kernel<128,8>";
    return names[5 + lv];
}

}  // namespace ptpc
