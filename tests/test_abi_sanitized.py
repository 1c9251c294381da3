"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Every source is compiled again with the sanitizers on the host side only (the device code is the
ordinary gfx950 build and is never run here) and linked into tests/sanitize/abi_host_checks.cpp,
which drives every argument check and workspace plan of the C ABI over a grid of shapes, ranks,
flags and tuning settings without launching a kernel.  Any sanitizer report aborts the program.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_rank_adapter_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def _run(cmd, cwd=None):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, cwd=cwd)
    return p.returncode, p.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not found")
def test_host_code_under_asan_ubsan(tmp_path):
    from sparse_rank_adapter_amd.build import SOURCES
    objs, cmds = [], []
    for src in SOURCES:
        o = str(tmp_path / src.replace(".hip", ".o"))
        objs.append(o)
        cmds.append([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-Xclang", "-target-feature",
                     "-Xclang", "-packed-fp32-ops", *HOST_SAN, "-I", INCLUDE, "-I", CSRC, "-c",
                     os.path.join(CSRC, src), "-o", o])
    with ThreadPoolExecutor(min(8, len(cmds))) as ex:
        results = list(ex.map(_run, cmds))
    for (rc, out), src in zip(results, SOURCES):
        assert rc == 0, f"{src}:\n{out}"
    main_o = str(tmp_path / "checks.o")
    rc, out = _run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", INCLUDE, "-c", os.path.join(HERE, "abi_host_checks.cpp"), "-o", main_o])
    assert rc == 0, out
    exe = str(tmp_path / "abi_host_checks")
    rc, out = _run([CLANG, "-fsanitize=address,undefined", main_o, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    assert rc == 0, out
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env,
                       timeout=600)
    print(p.stdout[-3000:])
    assert p.returncode == 0 and "all checks passed" in p.stdout
    shutil.rmtree(tmp_path, ignore_errors=True)
