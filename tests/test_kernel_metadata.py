"""Structural checks of the built gfx950 code object (CPU only): the device
code embedded in libnt.so is unbundled and its kernel metadata read with the
ROCm LLVM tools.  Every kernel must run in wave64 without scratch (no
register spills), the row-reduction kernels must contain no matrix-core
(MFMA) instructions (they are no contraction) while the attention kernels
must (Q K^T and P V are), and every launch shape the planner can choose must
have an instantiated kernel."""
import os
import re
import shutil
import subprocess

import pytest

import row_wise_reductions_amd as nt

from row_wise_reductions_amd import codeobj

LLVM = codeobj.LLVM
CSRC = os.path.join(os.path.dirname(nt.LIB_PATH), "csrc")
TARGET = codeobj.TARGET
MAGIC = codeobj.MAGIC


@pytest.fixture(scope="module")
def code_objects(tmp_path_factory):
    """One gfx950 code object per translation unit of libnt.so."""
    if not codeobj.tools_available():
        pytest.skip("binutils / ROCm LLVM tools not available")
    return codeobj.code_objects(nt.LIB_PATH, str(tmp_path_factory.mktemp("co")))


@pytest.fixture(scope="module")
def kernels(code_objects):
    out = codeobj.kernel_metadata(code_objects)
    assert out, "no kernels found in the code objects"
    return out


def test_no_spills_wave64(kernels):
    bad = {k: v for k, v in kernels.items() if v["scratch"] != 0 or v["wave"] != 64}
    assert not bad, bad


def test_no_mfma(code_objects):
    seen_rows = seen_attention = False
    for co in code_objects:
        asm = subprocess.run([f"{LLVM}/llvm-objdump", "-d", str(co)], check=True,
                             capture_output=True, text=True).stdout
        if "attention_fwd" in asm:
            seen_attention = True
            assert re.search(r"\bv_mfma_f32_32x32x16_bf16", asm) and re.search(r"\bv_mfma_f32_32x32x16_f16", asm)
        if "row_resident" not in asm:
            continue
        seen_rows = True
        assert "global_load_dwordx4" in asm
        assert not re.search(r"\bv_mfma", asm), "MFMA instruction in a row-reduction kernel"
    assert seen_rows and seen_attention


def _vregs(spec):
    m = re.match(r"v\[(\d+):(\d+)\]", spec)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", spec)
    return {int(m.group(1))} if m else set()


STREAM_STORES = ("global_store_dwordx4", "buffer_store_dwordx4")


def _store_hazards(code_object, need=2):
    """16-byte device-scope streaming stores (`nt sc1`, global or buffer
    form) followed, within `need` wait states in straight-line order, by a
    VALU writing one of their data registers (s_nop N counts N + 1, any other
    instruction 1).  gfx950 needs 2 after a global store of more than 64
    bits (with 1 the store writes the new register values) and after a
    buffer store with a constant scalar offset; a buffer store whose scalar
    offset is an SGPR has no such hazard (the compiler's hazard rules for
    gfx940-class targets).  Returns (stores, hazards)."""
    asm = subprocess.run([f"{LLVM}/llvm-objdump", "-d", str(code_object)], check=True,
                         capture_output=True, text=True).stdout.splitlines()
    ins, fn = [], None
    for line in asm:
        if line.endswith(">:"):
            fn = line
            continue
        m = re.match(r"\s+([a-z_0-9]+)(?:\s+([^/]*))?", line)
        if m and fn:
            ins.append((fn, m.group(1), (m.group(2) or "").strip()))
    stores, bad = 0, []
    for j, (f, op, args) in enumerate(ins):
        if op not in STREAM_STORES or "nt sc1" not in args:
            continue
        stores += 1
        # a buffer store whose scalar offset is an SGPR reads its data at
        # issue: the data hazard exists only with a constant offset
        ops = [a.strip() for a in args.split(",")]
        if op.startswith("buffer") and len(ops) > 3 and ops[3].split()[0].startswith("s"):
            continue
        data = _vregs(args.split(",")[0 if op.startswith("buffer") else 1].strip())
        ws = 0
        for f2, op2, a2 in ins[j + 1:j + 1 + 2 * need]:
            if f2 != f or ws >= need or op2 in ("s_endpgm", "s_branch", "s_setpc_b64"):
                break           # the straight line ends (what follows is reached by a jump)
            if op2.startswith("v_") and _vregs(a2.split(",")[0].strip()) & data:
                bad.append(f"{f} {op} {args} -> {op2} {a2} after {ws} wait states")
                break
            ws += int(a2.split()[0], 0) + 1 if op2 == "s_nop" else 1
    return stores, bad


def test_streaming_stores_are_compiler_visible(code_objects):
    """Row data leaves through device-scope streaming stores (nt sc1) that
    the compiler emits itself (raw buffer stores with that cache policy), so
    it keeps their hazards and wait counts: no kernel source writes a store
    in inline assembly, every nt sc1 store in the code objects is a buffer
    store, and none is followed by a VALU rewriting its data registers within
    2 wait states."""
    for name in os.listdir(CSRC):
        src = open(os.path.join(CSRC, name)).read()
        for m in re.finditer(r"asm\s+volatile\s*\(\s*\"([^\"]*)", src):
            assert "store" not in m.group(1) and "waitcnt" not in m.group(1), (name, m.group(1))
    total, bad, global_sc1 = 0, [], 0
    for co in code_objects:
        n, b = _store_hazards(co)
        total += n
        bad += b
        asm = subprocess.run([f"{LLVM}/llvm-objdump", "-d", str(co)], check=True, capture_output=True,
                             text=True).stdout
        global_sc1 += len(re.findall(r"global_store_dwordx4[^\n]*nt sc1", asm))
    assert total > 0, "no nt sc1 stores found"
    assert global_sc1 == 0, global_sc1
    assert not bad, bad[:5]


def test_calibration_copy_store_hazard(tmp_path):
    cal = os.path.join(os.path.dirname(nt.LIB_PATH), "libntcal.so")
    if not os.path.exists(cal) or not shutil.which("objcopy"):
        pytest.skip("libntcal.so or objcopy not available")
    fat = tmp_path / "cal.bin"
    subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", cal, str(fat)], check=True)
    data = fat.read_bytes()
    s0 = data.index(MAGIC)
    part, co = tmp_path / "b.bin", tmp_path / "cal.co"
    part.write_bytes(data[s0:])
    subprocess.run([f"{LLVM}/clang-offload-bundler", "--unbundle", "--type=o", f"--input={part}",
                    f"--targets={TARGET}", f"--output={co}"], check=True)
    n, bad = _store_hazards(co)
    assert n >= 1 and not bad, (n, bad)


def test_all_types_present(kernels):
    for dt in (0, 1, 2):
        assert any(f"row_residentILi0ELi{dt}E" in k for k in kernels), dt


def _shapes(kernels):
    have = set()
    for name in kernels:
        m = re.search(r"row_residentILi(\d)ELi(\d)ELi(\d+)ELi(\d+)ELb(\d)ELb\dELb(\d)", name)
        if m:
            have.add(("res",) + tuple(int(g) for g in m.groups()))
        m = re.search(r"row_loopedILi(\d)ELi(\d)ELi(\d+)ELi(\d+)ELb(\d)ELb(\d)", name)
        if m:
            have.add(("loop",) + tuple(int(g) for g in m.groups()))
        m = re.search(r"row_norm_persistentILi(\d)ELi(\d)ELi(\d+)ELi(\d+)ELb(\d)", name)
        if m:
            have.add(("pers",) + tuple(int(g) for g in m.groups()))
        m = re.search(r"softmax_split_(partial|finalize)ILi(\d)ELi(\d+)ELi(\d+)ELb(\d)ELb(\d)", name)
        if m:
            have.add((m.group(1),) + tuple(int(g) for g in m.groups()[1:]))
        m = re.search(r"softmax_coopILi(\d)ELi(\d+)ELi(\d+)ELb(\d)ELb(\d)", name)
        if m:
            have.add(("coop",) + tuple(int(g) for g in m.groups()))
        m = re.search(r"norm_split_(partial|finalize)ILi(\d)ELi(\d)ELi(\d+)ELi(\d+)ELb(\d)", name)
        if m:
            have.add(("n" + m.group(1),) + tuple(int(g) for g in m.groups()[1:]))
        m = re.search(r"norm_coopILi(\d)ELi(\d)ELi(\d+)ELi(\d+)ELb(\d)", name)
        if m:
            have.add(("ncoop",) + tuple(int(g) for g in m.groups()))
    return have


def test_every_planned_shape_is_built(kernels):
    """Every launch the planner can choose (fused add + norm included) has an
    instantiated kernel: (op, type, W, K, aligned, residual)."""
    have = _shapes(kernels)
    for op in (0, 1, 2, 3, 4, 5, 6, 7):
        # public op -> (kernel op, residual, causal)
        base, res, causal = {3: (1, 1, 0), 4: (2, 1, 0), 5: (3, 0, 1), 6: (1, 0, 0), 7: (2, 0, 0)}.get(op, (op, 0, 0))
        for dt in (0, 1, 2):
            for N in (1, 7, 64, 255, 781, 1000, 4096, 4097, 8192, 16384, 30000, 32768, 65536, 100000, 262144):
                for al in (True, False):
                    try:
                        p = nt.nt_plan_launch(op, 64, N, dt, al)
                    except nt.NtError:
                        continue
                    W, K, A = p["waves_per_row"], p["chunks_per_lane"], p["aligned"]
                    if p["split"] == 1:
                        if p["cooperative"]:
                            assert ("coop", dt, W, K, A, causal) in have, (dt, N, al, p)
                        assert ("partial", dt, W, K, A, causal) in have, (op, dt, N, al, p)
                        assert ("finalize", dt, W, K, A, causal) in have, (op, dt, N, al, p)
                    elif p["split"] == 2:
                        assert ("loop", base, dt, W, K, A, res) in have, (op, dt, N, al, p)
                    elif p["split"] == 3:
                        assert ("npartial", base, dt, W, K, A) in have, (op, dt, N, al, p)
                        assert ("nfinalize", base, dt, W, K, A) in have, (op, dt, N, al, p)
                        if p["cooperative"]:
                            assert ("ncoop", base, dt, W, K, A) in have, (op, dt, N, al, p)
                    else:
                        assert ("res", base, dt, W, K, A, res) in have, (op, dt, N, al, p)
                        if p["persistent"]:
                            assert ("pers", base, dt, W, K, res) in have, (op, dt, N, al, p)
