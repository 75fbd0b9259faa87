"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's host side (planning, workspace sizes, argument validation:
csrc/nt_api.cpp) is built for the host alone with both sanitizers, linked
against stub kernel launchers that abort, and driven over extreme arguments
(tests/host_checks_main.cpp).  The oracle's C code is built the same way with
gcc and run on every entry point (tests/oracle_checks_main.c).  A sanitizer
report, an abort or a failed expectation fails the test.  Nothing here
touches a GPU: the sanitizers apply to host code only."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "row_wise_reductions_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-6000:]}"
    return r


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_library_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_checks")
    # each -fsanitize= applies to the host side only (the device side of
    # nt_api.cpp is the no-alloc entry point's scratch array)
    _run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all", "-Wno-unused-command-line-argument",
          f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
          os.path.join(CSRC, "nt_api.cpp"), os.path.join(ROOT, "tests", "host_checks_main.cpp"), "-o", exe],
         timeout=600)
    r = _run([exe], env=ENV, timeout=300)
    assert r.stdout.startswith("ok ") and "0 failures" in r.stdout, r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_per_call_path_is_quiet(tmp_path):
    """After the first call on a device, no call of any entry point reads the
    environment or queries a device attribute: the host code is linked with
    counting stand-ins for getenv and the HIP property queries, and with
    launchers that succeed without launching (tests/percall_checks_main.cpp)."""
    exe = str(tmp_path / "percall_checks")
    _run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-Wno-unused-command-line-argument",
          f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
          os.path.join(CSRC, "nt_api.cpp"), os.path.join(ROOT, "tests", "percall_checks_main.cpp"), "-o", exe],
         timeout=600)
    r = _run([exe], env=dict(os.environ, NT_COOP="1", NT_DEBUG="0"), timeout=120)
    assert "ok, 0 failures" in r.stdout and "getenv 0," in r.stdout, r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-fno-fast-math", "-ffp-contract=off",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "tests", "oracle_checks_main.c"), "-o", exe, "-lm"], timeout=300)
    r = _run([exe], env=dict(ENV, OMP_NUM_THREADS="4"), timeout=300)
    assert r.stdout.strip() == "ok", r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="gcc/g++ not available")
@pytest.mark.parametrize("lang", ["c", "c++"])
def test_header_compiles_cleanly(lang, tmp_path):
    """include/nt.h on its own, as C11 and as C++17, with every warning an
    error; the enumerations keep the size of an int in both."""
    src = tmp_path / ("t.c" if lang == "c" else "t.cpp")
    src.write_text('#include "nt.h"\n'
                   '_Static_assert(sizeof(nt_op) == sizeof(int) && sizeof(nt_dtype) == sizeof(int) &&\n'
                   '               sizeof(nt_status) == sizeof(int), "int-sized enums");\n'
                   '#ifdef NT_ENUM\n#error "helper macro leaked"\n#endif\n'
                   'int main(void) { return (int)NT_OK; }\n'
                   if lang == "c" else
                   '#include "nt.h"\n'
                   'static_assert(sizeof(nt_op) == sizeof(int) && sizeof(nt_dtype) == sizeof(int) &&\n'
                   '              sizeof(nt_status) == sizeof(int), "int-sized enums");\n'
                   '#ifdef NT_ENUM\n#error "helper macro leaked"\n#endif\n'
                   'int main() { return (int)NT_OK; }\n')
    cc = ["gcc", "-std=c11"] if lang == "c" else ["g++", "-std=c++17"]
    _run([*cc, "-Wall", "-Wextra", "-Werror", "-pedantic", f"-I{os.path.join(ROOT, 'include')}", str(src), "-o",
          str(tmp_path / "t")], timeout=120)
