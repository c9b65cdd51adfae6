"""Static check of the inline-asm MFMAs in gemm16_kernel and gemm16s_kernel
(no GPU needed).

Both kernels issue their v_mfma_f32_16x16x128_f8f6f4 from inline asm, which
the compiler's hazard tracking does not see, so the kernels keep every
dependence on an MFMA's registers far apart by construction.  This test
compiles gemm.hip to gfx950 assembly and checks, for every instantiation, on
straight-line code, across every loop back edge and along every forward
branch:

  * after an MFMA writes its accumulator registers, no other instruction
    touches them within the next 24 wait states (an s_nop N counts N + 1);
  * before an MFMA, no vector-ALU instruction wrote one of its source or
    accumulator registers within the previous 6 wait states.

Both windows are several times the wait states a 16x16x128 MFMA needs.

The same assembly also shows that no GEMM kernel spills registers inside its
K loop (a spill there would reload from memory between MFMAs).
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
AFTER_WRITE = 24
BEFORE_READ = 6


def _regs(tok):
    """Registers named in an operand string, as (kind, index) with kind 'a'
    (AGPR) or 'v' (VGPR)."""
    out = set()
    for m in re.finditer(r"\b([av])\[(\d+):(\d+)\]|\b([av])(\d+)\b", tok):
        if m.group(4):
            out.add((m.group(4), int(m.group(5))))
        else:
            out.update((m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _wait_states(ins):
    return int(ins.split()[1]) + 1 if ins.startswith("s_nop") else 1


def _functions(asm):
    for m in re.finditer(r"\n(_ZN4ptpc1[34]gemm16s?_kernel\w+):", asm):
        body = asm[m.start():asm.index(".Lfunc_end", m.start())]
        ins, labels = [], {}
        for line in body.split("\n")[2:]:
            line = line.split(";")[0].strip()
            if not line or (line.startswith(".") and not line.startswith(".LBB")):
                continue
            if line.startswith(".LBB"):
                labels[line.rstrip(":")] = len(ins)
                continue
            ins.append(line)
        yield m.group(1), ins, labels


def _sequences(ins, labels):
    """The straight-line order, every loop body followed by its start, and
    every forward branch taken (the code before it, then its target)."""
    yield list(range(len(ins)))
    for k, line in enumerate(ins):
        if line.startswith("s_cbranch") or line.startswith("s_branch"):
            target = line.split()[-1]
            if target in labels and labels[target] <= k:
                start = labels[target]
                yield list(range(start, k + 1)) + list(range(start, k + 1))
            elif target in labels:
                t = labels[target]
                yield list(range(max(0, k - 64), k + 1)) + list(range(t, min(len(ins), t + 64)))


def _violations(ins, labels):
    bad = []
    for seq in _sequences(ins, labels):
        for p, k in enumerate(seq):
            line = ins[k]
            if not line.startswith("v_mfma"):
                continue
            ops = line.split(None, 1)[1].split(", ")
            dst = _regs(ops[0])
            waited = 0
            for q in range(p + 1, len(seq)):
                other = ins[seq[q]]
                if waited >= AFTER_WRITE:
                    break
                if dst & _regs(other):
                    bad.append(("after write", line, other, waited))
                    break
                waited += _wait_states(other)
            srcs = set()
            for op in ops[1:4]:
                srcs |= _regs(op)
            waited = 0
            for q in range(p - 1, -1, -1):
                other = ins[seq[q]]
                if waited >= BEFORE_READ:
                    break
                if other.startswith("v_") and not other.startswith("v_mfma") \
                        and not other.startswith("v_cmp"):
                    d = other.split(None, 1)[1].split(",")[0] if " " in other else ""
                    written = _regs(d)
                    if written & srcs:
                        bad.append(("before read", other, line, waited))
                        break
                waited += _wait_states(other)
    return bad


def test_checker_catches_planted_hazards():
    """The scanner itself: a read of an accumulator right after the MFMA that
    writes it, a source written just before an MFMA, and the same hazard
    across a loop back edge are flagged; the spaced-out forms are not."""
    mfma = "v_mfma_f32_16x16x128_f8f6f4 a[0:3], v[8:15], v[16:23], a[0:3]"
    assert _violations([mfma, "v_accvgpr_read_b32 v1, a2"], {})
    assert _violations(["v_mov_b32 v9, 0", mfma], {})
    assert _violations(["v_accvgpr_write_b32 a1, 0", "s_nop 1", mfma], {})
    assert not _violations([mfma] + ["s_nop 7"] * 3 + ["v_accvgpr_read_b32 v1, a2"], {})
    assert not _violations(["v_mov_b32 v9, 0", "s_nop 7", mfma], {})
    assert not _violations([mfma, "v_mfma_f32_16x16x128_f8f6f4 a[4:7], v[8:15], v[16:23], a[4:7]"], {})
    loop = ["v_accvgpr_read_b32 v1, a2", "s_nop 7", "s_nop 7", "s_nop 7", mfma,
            "s_cbranch_scc1 .LBB0_1"]
    assert not _violations(loop, {})
    assert _violations(loop, {".LBB0_1": 0})
    skip = [mfma, "s_cbranch_scc1 .LBB0_2", "s_nop 7", "s_nop 7", "s_nop 7",
            "v_accvgpr_read_b32 v1, a3"]
    assert not _violations(skip, {})
    assert _violations(skip, {".LBB0_2": 5})


VARIANTS = {"release": [], "lds_poison": ["-DPTPC_LDS_POISON"]}


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    """gfx950 assembly of gemm.hip for the release and LDS-poison builds
    (compiled once, in parallel)."""
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("asm")

    def compile_one(item):
        name, defines = item
        out = d / f"gemm_{name}.s"
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++20", "-ffp-contract=off",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *defines,
               "-I", os.path.join(ROOT, "include"),
               "-I", os.path.join(ROOT, "scaled_gemm_amd", "csrc"),
               "--cuda-device-only", "-S", "-x", "hip",
               os.path.join(ROOT, "scaled_gemm_amd", "csrc", "gemm.hip"), "-o", str(out)]
        subprocess.run(cmd, check=True, capture_output=True, timeout=600)
        return name, out.read_text()

    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=2) as ex:
        return dict(ex.map(compile_one, VARIANTS.items()))


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_gemm16_inline_mfma_hazards(gemm_asm, variant):
    asm = gemm_asm[variant]
    found = 0
    for name, ins, labels in _functions(asm):
        found += 1
        n_mfma = sum(1 for line in ins if line.startswith("v_mfma"))
        assert n_mfma > 0, name
        bad = _violations(ins, labels)
        assert not bad, (name, bad[:5])
    assert found >= 10, "expected the fused and two-step forms of five kernels"


def test_lds_poison_build_writes_its_poison(gemm_asm):
    """The debug build really adds the poisoning LDS writes (16-byte writes
    of 0x7F7F7F7F) to every pipelined kernel: more ds_write_b128 than the
    release build in each of them, and the NaN pattern in the code."""
    def writes(asm):
        counts = {}
        for m in re.finditer(r"\n(_ZN4ptpc(?:11gemm_kernel|13gemm16_kernel|14gemm16s_kernel)\w+):",
                             asm):
            body = asm[m.start():asm.index(".Lfunc_end", m.start())]
            counts[m.group(1)] = sum(1 for line in body.split("\n")
                                     if line.strip().startswith("ds_write_b128"))
        return counts
    rel = writes(gemm_asm["release"])
    poi_asm = gemm_asm["lds_poison"]
    poi = writes(poi_asm)
    assert "0x7f7f7f7f" in poi_asm.lower()
    piped = list(rel)
    assert len(piped) >= 18          # fused and two-step forms of every tiled kernel
    for n in piped:
        assert poi[n] > rel[n], (n, rel[n], poi[n])


def _kernels(asm):
    """(name, instructions, private bytes per lane) of every kernel in the file."""
    for m in re.finditer(r"\n(_ZN4ptpc\w+):", asm):
        end = asm.find(".Lfunc_end", m.start())
        if end < 0:
            continue
        ins = [line.split(";")[0].strip() for line in asm[m.start():end].split("\n")[1:]]
        ins = [line for line in ins if line and not line.startswith(".")]
        meta = re.search(r"\.amdhsa_kernel " + re.escape(m.group(1)) + r"\n(.*?)\.end_amdhsa_kernel",
                         asm, re.S)
        priv = int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", meta.group(1)).group(1))
        yield m.group(1), ins, priv


def _spills_inside(ins):
    """Scratch accesses between the first and the last MFMA of a kernel."""
    mfma = [k for k, line in enumerate(ins) if line.startswith("v_mfma")]
    if not mfma:
        return []
    return [ins[k] for k in range(mfma[0], mfma[-1] + 1) if ins[k].startswith("scratch_")]


def test_no_spills_in_k_loops(gemm_asm):
    """Every GEMM kernel's accumulators and operand registers fit: no scratch
    (spill) access between a kernel's first and last MFMA, that is inside its
    K loop and remainder steps, and at most 128 bytes of private memory per
    lane anywhere (the two-range join keeps a few accumulator slabs there
    while it waits for the other range, after its K loop)."""
    asm = gemm_asm["release"]
    seen = 0
    for name, ins, priv in _kernels(asm):
        seen += 1
        assert priv <= 128, (name, priv)
        inside = _spills_inside(ins)
        assert not inside, (name, inside[:4])
    assert seen >= 30


def test_spill_check_catches_a_planted_spill():
    """The scan above on a synthetic kernel: a spill between two MFMAs is
    found, one after the last MFMA is not."""
    body = ("\n_ZN4ptpc1xEv:\n\tv_mfma_f32_16x16x128_f8f6f4 a[0:3], v[8:15], v[16:23], a[0:3]\n"
            "\tscratch_store_dwordx4 off, a[4:7], off\n"
            "\tv_mfma_f32_16x16x128_f8f6f4 a[0:3], v[8:15], v[16:23], a[0:3]\n"
            "\tscratch_store_dwordx4 off, a[8:11], off\n.Lfunc_end0:\n"
            ".amdhsa_kernel _ZN4ptpc1xEv\n\t.amdhsa_private_segment_fixed_size 32\n.end_amdhsa_kernel\n")
    ((name, ins, priv),) = list(_kernels(body))
    assert priv == 32
    assert _spills_inside(ins) == ["scratch_store_dwordx4 off, a[4:7], off"]
