"""The shapes the GPU parity tests run, in one place (host side only).

The GPU tests take their cases from here, and ``test_kernel_coverage.py``
checks on the CPU, through the library's kernel-choice queries, that these
cases together launch every GEMM and activation-quantization kernel the
library can pick.
"""
import workloads

# Whole outputs against the full oracle: (name, T, Ci, Co).
FULL_CASES = [
    ("tiny", 16, 256, 512),
    ("8b_qkv_decode", 32, 4096, 6144),
    ("ragged", 300, 1040, 784),
    ("ragged", 257, 384, 272),
    ("ragged", 1, 16, 16),
    ("ragged", 3, 144, 48),
    ("ragged", 33, 272, 2064),
    ("ragged", 97, 400, 1040),
    ("ragged", 130, 272, 8208),      # 64x128 tiles (65..255 tokens, fewest rounds)
    ("ragged", 200, 144, 1040),      # 64x64 tiles, four row tiles
    ("ragged", 48, 272, 10256),
    ("ragged", 48, 272, 32784),      # 128x128 tiles of the 32x32x64 kernel at 33..64 tokens
    ("ragged", 20, 144, 32784),
    ("ragged", 24, 208, 8208),
    ("ragged", 600, 256, 2048),
    ("ragged", 513, 512, 2064),
    ("ragged", 600, 144, 22000),
    ("ragged", 500, 144, 28656),
    # the 16x16x128 tiled kernel runs its 128-byte K steps in periods of 6,
    # the rest one by one: 12, 7 and 11 steps (remainders 0, 1 and 5; the
    # other cases cover 2, 3 and 4), on 128x256 tiles with ragged rows and
    # columns
    ("ragged", 280, 1536, 16400),
    ("ragged", 272, 880, 16656),
    ("ragged", 520, 1392, 8208),
    # the same K extents at 256+ tokens with few output columns: 64x128
    # tiles of the 32x32x64 kernel
    ("ragged", 280, 1536, 528),
    ("ragged", 272, 880, 1296),
    ("ragged", 520, 1392, 400),
    # 65..128 tokens on 64x64 tiles: K steps dealt to 4 waves (1 step: three
    # waves idle; 13 and 27 steps: uneven counts per wave)
    ("ragged", 100, 16, 2064),
    ("ragged", 65, 1552, 528),
    ("ragged", 120, 3344, 1040),
    ("ragged", 200, 272, 36864),     # 128x128 tiles of the 16x16x128 kernel at 65..255 tokens
    # near the longest K the contract accepts (2^17), with a K tail past the
    # last whole 128-byte step (the few-token kernel)
    ("ragged", 8, 131072 - 16, 256),
]

FULL_SEEDS = [("tiny", 1), ("tiny", 2), ("8b_qkv_decode", 1), ("8b_qkv_decode", 2)]

# Sampled outputs at full size; these select each of the other tile shapes of
# the 128-byte-step kernel, with K remainders the full-size configs do not
# have (ragged K, periods of 6 steps plus 1, 5, 0, 1).  (T, Ci, Co).
TILE_CASES = [
    (4096, 1648, 4096),     # 256x256 tiles, 13 K steps
    (1536, 592, 8192),      # 192x256 tiles, 5 K steps
    (1024, 880, 10240),     # 192x256 tiles with a partial last row tile, 7 K steps
    (256, 1040, 40944),     # 256x160 tiles with a partial last column tile, 9 K steps
    (1024, 752, 14336),     # 256x224 tiles, 6 K steps
    # wide layers at 81..255 tokens: one row tile of 224 columns per weight slab
    (100, 1040, 50192),     # 128x224 tiles, rows past T, a 16-column last tile, 9 K steps
    (200, 1040, 50192),     # 256x224 tiles with a partial row tile, 9 K steps
    (512, 16400, 8192),     # 128x128 tiles at 256+ tokens, long K: 129 K steps
    (512, 1040, 8192),      # 128x128 tiles at 256+ tokens, 9 K steps
    # where 128x128 tiles would leave CUs idle at 256+ tokens: 64x128 tiles of
    # the 32x32x64 kernel (two workgroups per CU)
    (512, 16400, 1024),     # long K: 257 K steps of 64 bytes
    (256, 131072 - 16, 512),  # K near the contract's 2^17 limit: 2048 K steps
]

CONFIG_CASES = ["8b_gate_up", "70b_down"]

# 70B layer shapes at token counts outside the sweep (sampled outputs):
# (layer, T).  64 tokens of the gate_up layer run 128x128 tiles of the
# 32x32x64 kernel (every CU gets one).
EXTRA_SWEEP_CASES = [("gate_up", 64)]

PER_TENSOR_CASES = [("tiny", 16, 256, 512), ("ragged", 48, 272, 10256),
                    ("ragged", 300, 1040, 784), ("ragged", 1, 16, 16),
                    ("8b_qkv_decode", 32, 4096, 6144),
                    ("ragged", 100, 528, 1040)]   # the K-split 64x64 tiles, scalar scales

# Epilogue edge values: T picks the kernel family (Ci = 4112, Co = 528).
# (T, Ci, Co) of the epilogue edge-value test: T picks the kernel family --
# 16 the few-token kernel, 100 the K-split 64x64 tiles, 200 the 64x64 tiles
# of the 32x32x64 kernel (and 4 K ranges through the workspace form), 512
# its 64x128 tiles at 256+ tokens, 520 x 8208 columns the 16x16x128 tiled
# kernel (128x256 tiles).
EPILOGUE_CASES = [(16, 4112, 528), (100, 4112, 528), (200, 4112, 528), (512, 4112, 528),
                  (520, 1040, 8208)]

# (T, Ci, Co) of the pitched-buffer test: the K-split 64x64 tiles, the 64x128
# tiles of the 32x32x64 kernel, the 16x16x128 tiled kernel.
PITCHED_CASES = [(70, 528, 208), (300, 528, 208), (520, 528, 8208)]

# Long activation rows, with the row maxima placed anywhere, the last row's
# in its last vector: (T, Ci).  40960 and 65536: 32 vectors per thread in
# registers; 65552: longer than one workgroup holds (the two-pass kernel).
LONG_ROW_CASES = [(7, 40960), (4, 65536), (7, 65552)]

# Row lengths of the exhaustive (x, amax) quantizer check: every launch shape
# of rows of 256 or more vectors (the amax values are dealt to the lengths in
# order, so the longest bucket gets the largest ones).
EXHAUSTIVE_CI = [512, 1024, 2048, 4096, 8192, 16384, 24576, 28672, 65536]


def gemm_shapes():
    """Every (T, Ci, Co) a GPU test sends through ptpc_gemm."""
    out = [(T, Ci, Co) for _, T, Ci, Co in FULL_CASES]
    out += [(workloads.CONFIGS[n].T, workloads.CONFIGS[n].Ci, workloads.CONFIGS[n].Co)
            for n, _ in FULL_SEEDS]
    out += list(TILE_CASES)
    out += [(workloads.CONFIGS[n].T, workloads.CONFIGS[n].Ci, workloads.CONFIGS[n].Co)
            for n in CONFIG_CASES]
    for layer, (Ci, Co) in workloads.SWEEP_LAYERS.items():
        out += [(T, Ci, Co) for T in workloads.SWEEP_T]
    out += [(T, *workloads.SWEEP_LAYERS[layer]) for layer, T in EXTRA_SWEEP_CASES]
    out += [(T, Ci, Co) for _, T, Ci, Co in PER_TENSOR_CASES]
    out += list(EPILOGUE_CASES)
    out += list(PITCHED_CASES)
    return out


def quant_act_shapes():
    """Every (T, Ci) a GPU test sends through ptpc_quant_act."""
    out = [(T, Ci) for T, Ci, _ in gemm_shapes()]
    out += list(LONG_ROW_CASES)
    out += [(2, Ci) for Ci in EXHAUSTIVE_CI]
    return out
