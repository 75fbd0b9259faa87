"""The gfx950 code objects inside the built library, read on the host.

The ``.hip_fatbin`` section of a linked HIP library is a concatenation of
offload bundles, one per translation unit; each holds the gfx950 code object
of that unit.  This module unbundles them with the ROCm LLVM tools and reads
each kernel's resource metadata (registers, LDS, scratch), from which it
derives the static occupancy limit.  Nothing here touches a GPU.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess

LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

# gfx950 compute unit: 4 SIMDs, at most 8 waves per SIMD, 512 registers per
# lane per SIMD (architectural and accumulation registers share the file,
# allocated in granules of 8), 160 KiB of LDS.
SIMDS_PER_CU = 4
MAX_WAVES_PER_SIMD = 8
REGS_PER_SIMD_LANE = 512
REG_GRANULE = 8
LDS_PER_CU = 160 * 1024


def tools_available() -> bool:
    return bool(shutil.which("objcopy")) and os.path.exists(f"{LLVM}/clang-offload-bundler")


def code_objects(lib_path: str, workdir: str) -> list[str]:
    """Unbundle the gfx950 code object of every translation unit of `lib_path`
    into `workdir`; returns their paths."""
    os.makedirs(workdir, exist_ok=True)
    fat = os.path.join(workdir, "fatbin.bin")
    subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", lib_path, fat], check=True)
    with open(fat, "rb") as f:
        data = f.read()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    if not starts:
        raise RuntimeError(f"no offload bundle in {lib_path}")
    out = []
    for i, s0 in enumerate(starts):
        end = starts[i + 1] if i + 1 < len(starts) else len(data)
        part, co = os.path.join(workdir, f"bundle{i}.bin"), os.path.join(workdir, f"k{i}.co")
        with open(part, "wb") as f:
            f.write(data[s0:end])
        subprocess.run([f"{LLVM}/clang-offload-bundler", "--unbundle", "--type=o", f"--input={part}",
                        f"--targets={TARGET}", f"--output={co}"], check=True)
        out.append(co)
    return out


def kernel_metadata(cos: list[str]) -> dict:
    """Mangled kernel name -> resource metadata of the code objects."""
    out = {}
    for co in cos:
        notes = subprocess.run([f"{LLVM}/llvm-readelf", "--notes", co], check=True,
                               capture_output=True, text=True).stdout
        for block in notes.split("  - .agpr_count:")[1:]:
            block = ".agpr_count:" + block
            name = re.search(r"\.name:\s+(\S+)", block).group(1)
            get = lambda k: int(re.search(rf"\.{k}:\s+(\d+)", block).group(1))  # noqa: E731
            out[name] = {"agpr": get("agpr_count"), "vgpr": get("vgpr_count"), "sgpr": get("sgpr_count"),
                         "lds": get("group_segment_fixed_size"), "scratch": get("private_segment_fixed_size"),
                         "wave": get("wavefront_size"), "max_threads": get("max_flat_workgroup_size")}
    return out


def demangle(names: list[str]) -> dict:
    """Mangled -> demangled names (binutils c++filt)."""
    r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True, check=True)
    return dict(zip(names, r.stdout.splitlines()))


def waves_per_simd(meta: dict, threads: int) -> dict:
    """Static occupancy of a kernel launched with `threads` per workgroup:
    resident waves per SIMD as limited by registers, by LDS, and overall
    (whole workgroups only)."""
    regs = -(-((meta["vgpr"] + 3) // 4 * 4 + meta["agpr"]) // REG_GRANULE) * REG_GRANULE
    by_regs = min(MAX_WAVES_PER_SIMD, REGS_PER_SIMD_LANE // max(regs, REG_GRANULE))
    waves_per_wg = -(-threads // 64)
    wg_by_regs = by_regs * SIMDS_PER_CU // waves_per_wg
    wg_by_lds = LDS_PER_CU // meta["lds"] if meta["lds"] else 1 << 30
    wg = min(wg_by_regs, wg_by_lds)
    return {"regs_allocated": regs, "by_regs": by_regs,
            "by_lds": min(MAX_WAVES_PER_SIMD, wg_by_lds * waves_per_wg // SIMDS_PER_CU),
            "waves_per_simd": wg * waves_per_wg / SIMDS_PER_CU, "workgroups_per_cu": wg}
