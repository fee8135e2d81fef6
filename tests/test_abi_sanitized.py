"""The C-ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer.

nosa_api.cpp (every host-side check of the library) is built for the host
alone with g++ and -fsanitize=address,undefined, and the ABI tests
(tests/test_abi.py) run against that build in a child process with the ASan
runtime preloaded.  The kernel launchers are replaced by stubs, generated
from the declarations in nosa_launch.hpp, that return hipErrorNoDevice: no
kernel is built, none can run, and no GPU is needed.  Any sanitizer report
ends the child with an error.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_kv_score_amd", "csrc")
ROCM = "/opt/rocm"
GXX = shutil.which("g++")

pytestmark = pytest.mark.skipif(GXX is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")),
                                reason="needs g++ and the HIP runtime library")


def launcher_stubs() -> str:
    """A translation unit defining every launcher nosa_launch.hpp declares,
    each returning hipErrorNoDevice without touching its arguments."""
    text = open(os.path.join(CSRC, "nosa_launch.hpp")).read()
    decls = re.findall(r"^hipError_t (launch_\w+)\((.*?)\);", text, re.M | re.S)
    assert len(decls) >= 20, "launcher declarations not found"
    out = ['#include "nosa_launch.hpp"', "", "namespace nosa {", ""]
    for name, params in decls:
        out.append(f"hipError_t {name}({params}) {{ return hipErrorNoDevice; }}")
    out += ["", "}  // namespace nosa", ""]
    return "\n".join(out)


def test_host_checks_under_asan_and_ubsan(tmp_path):
    stub = tmp_path / "launch_stubs.cpp"
    stub.write_text(launcher_stubs())
    lib = tmp_path / "libnosa_host_sanitized.so"
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
             "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), "-I", CSRC]
    cmd = [GXX, *flags, os.path.join(CSRC, "nosa_api.cpp"), str(stub), "-o", str(lib),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    needed = subprocess.run(["readelf", "-d", str(lib)], capture_output=True, text=True).stdout
    assert "libasan" in needed and "libubsan" in needed, needed  # the sanitizers are in

    asan_rt = subprocess.run([GXX, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    assert os.path.exists(asan_rt), asan_rt
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan_rt
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=97"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=98"
    child = (
        "import sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "from block_sparse_kv_score_amd import nosa\n"
        f"nosa.LIB_PATH = {str(lib)!r}\n"
        "import pytest\n"
        f"sys.exit(pytest.main([{os.path.join(ROOT, 'tests', 'test_abi.py')!r}, '-q', '-m', 'not gpu',\n"
        "                      '-p', 'no:cacheprovider', '-o', 'addopts=']))\n"
    )
    r = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, env=env, timeout=600,
                       cwd=str(tmp_path))
    report = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, report
    assert "ERROR: AddressSanitizer" not in report and "runtime error:" not in report, report
    n_tests = len(re.findall(r"^def test_", open(os.path.join(ROOT, "tests", "test_abi.py")).read(), re.M))
    m = re.search(r"(\d+) passed", r.stdout)
    assert m and int(m.group(1)) == n_tests, report  # every ABI test ran, none skipped
